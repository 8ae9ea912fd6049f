// gdr_timing.hip -- opt-in per-kernel timing with HIP events.
//
// For the kernels selected by gdr_timing_enable's mask, every launch goes
// through hipExtLaunchKernelGGL with two events that the dispatch records at
// the kernel's start and end (GDR_LAUNCH), so the durations measured are
// those of the kernels as they run in the caller's sequence, and no event
// packet sits between them (a timed launch still costs the stream a few
// microseconds).  gdr_timing_read waits for the recorded events,
// returns the summed durations and launch counts per kernel, and forgets
// them.  Disabled (the default), the hooks cost one relaxed atomic load per
// launch.
//
// It also holds the MFMA issue-rate probe behind gdr_mfma_peak_probe: the
// dense rate of each MFMA kind the kernels use, measured on the part for the
// roofline's compute ceiling.
#include "gdr.h"
#include "gdr_internal.h"

#include <atomic>
#include <mutex>
#include <vector>

namespace gdr {
namespace {

struct Rec {
    int id;
    hipEvent_t begin, end;
};

std::atomic<int> g_mask{0};
std::mutex g_mu;
std::vector<Rec> g_recs;            // launches recorded since the last read
std::vector<hipEvent_t> g_free;     // events ready for reuse

hipEvent_t take_event() {
    hipEvent_t e = nullptr;
    {
        std::lock_guard<std::mutex> lk(g_mu);
        if (!g_free.empty()) {
            e = g_free.back();
            g_free.pop_back();
        }
    }
    if (!e && hipEventCreate(&e) != hipSuccess) e = nullptr;
    return e;
}

}  // namespace

const char* kernel_name(int id) {
    static const char* names[kKernelCount] = {"gdr_chunkmap", "gdr_intra", "gdr_scan", "gdr_output",
                                              "gdr_decode"};
    return (id >= 0 && id < kKernelCount) ? names[id] : "";
}

bool timing_events(int id, hipEvent_t* start, hipEvent_t* stop) {
    if (!((g_mask.load(std::memory_order_relaxed) >> id) & 1)) return false;
    hipEvent_t b = take_event(), e = take_event();
    std::lock_guard<std::mutex> lk(g_mu);
    if (!b || !e) {   // no event to be had: this launch goes untimed
        if (b) g_free.push_back(b);
        if (e) g_free.push_back(e);
        return false;
    }
    g_recs.push_back(Rec{id, b, e});
    *start = b;
    *stop = e;
    return true;
}

// ------------------------------------------------------------------ MFMA issue-rate probe
// Every wave runs kProbeChains[KIND] independent accumulator chains of one
// MFMA kind for `iters` rounds (eight waves per SIMD keep the matrix pipe fed);
// the accumulators' sum goes to sink, so no product is dead, except in
// thread 0 of each workgroup, which writes the shader clock over the
// workgroup's run.  Operands are small constants, so the sums stay finite.
namespace {

typedef _Float16 probe_h8 __attribute__((ext_vector_type(8)));
typedef _Float16 probe_h4 __attribute__((ext_vector_type(4)));
typedef __bf16 probe_b8 __attribute__((ext_vector_type(8)));
typedef float probe_f4 __attribute__((ext_vector_type(4)));
typedef float probe_f16 __attribute__((ext_vector_type(16)));

template <int KIND>
__global__ __launch_bounds__(256) void mfma_rate_kernel(int64_t iters, float* sink) {
    constexpr int NCH = kProbeChains[KIND];
    const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    asm volatile("" ::: "memory");
    const float x = 1e-3f * (float)(1 + (threadIdx.x & 7));
    probe_f4 acc[NCH];
#pragma unroll
    for (int j = 0; j < NCH; ++j) acc[j] = probe_f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (KIND == 4) {   // fp16 32x32x16, 16 accumulators a lane
        probe_h8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) { a[e] = (_Float16)x; b[e] = (_Float16)(0.5f * x); }
        probe_f16 big[NCH];
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) big[j][e] = 0.f;
        for (int64_t i = 0; i < iters; ++i)
#pragma unroll
            for (int j = 0; j < NCH; ++j) big[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, big[j], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < NCH; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][e] = big[j][e] + big[j][4 + e] + big[j][8 + e] + big[j][12 + e];
    } else if constexpr (KIND == 0) {   // fp16 16x16x32
        probe_h8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) { a[e] = (_Float16)x; b[e] = (_Float16)(0.5f * x); }
        for (int64_t i = 0; i < iters; ++i)
#pragma unroll
            for (int j = 0; j < NCH; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
    } else if constexpr (KIND == 1) {   // bf16 16x16x32
        probe_b8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) { a[e] = (__bf16)x; b[e] = (__bf16)(0.5f * x); }
        for (int64_t i = 0; i < iters; ++i)
#pragma unroll
            for (int j = 0; j < NCH; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    } else if constexpr (KIND == 2) {   // fp16 16x16x16
        probe_h4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) { a[e] = (_Float16)x; b[e] = (_Float16)(0.5f * x); }
        for (int64_t i = 0; i < iters; ++i)
#pragma unroll
            for (int j = 0; j < NCH; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, acc[j], 0, 0, 0);
    } else {   // fp32 16x16x4
        const float a = x, b = 0.5f * x;
        for (int64_t i = 0; i < iters; ++i)
#pragma unroll
            for (int j = 0; j < NCH; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    asm volatile("" : "+v"(s) :: "memory");
    // thread 0 reports the shader clock over its workgroup's run (shader
    // cycles against the 100 MHz real-time counter), in MHz
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    const float mhz = r1 > r0 ? (float)((double)(t1 - t0) * 100.0 / (double)(r1 - r0)) : 0.f;
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = threadIdx.x == 0 ? mhz : s;
}

}  // namespace

// ------------------------------------------------------------------ slab-stream probe
// The one-token decode's memory traffic alone: workgroup (row b, head h,
// 64-column half), placed as the decode places it (place_slab), streams its
// half of the 16-bit 128 x 128 slab of slot idx[b], head h, with the decode's
// thread layout (8 lanes per 64-column row piece, 32 rows a pass, 4 passes)
// and its non-temporal 16-byte loads, then writes the same bytes back with
// non-temporal stores.  Slots outside [0, num_slots) are skipped.  The decode
// fits six workgroups on a CU (its registers); the probe needs far fewer
// registers, so its launch reserves 24 KiB of LDS per workgroup (unused) to
// hold it to the same six.
namespace {
typedef uint32_t probe_u4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256, 4) void slab_stream_kernel(uint16_t* pool, int32_t num_slots, const int32_t* idx,
                                                             int32_t B, int32_t Nv) {
    constexpr int D = 128, CW = 64, LPR = 8, RP = 32, RPT = 4;
    int b, h, slice;
    place_slab(blockIdx.x, B, Nv, D / CW, b, h, slice);
    const int slot = idx[b];
    if (slot < 0 || slot >= num_slots) return;
    const int tid = threadIdx.x, col = slice * CW + (tid % LPR) * 8, rg = tid / LPR;
    uint16_t* base = pool + ((size_t)slot * Nv + h) * D * D + col;
    probe_u4 raw[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        raw[m] = __builtin_nontemporal_load(reinterpret_cast<const probe_u4*>(base + (size_t)(rg + RP * m) * D));
    // the bytes pass through an opaque statement, so that the compiler cannot
    // drop the write-back of unchanged values (and with it the loads)
#pragma unroll
    for (int m = 0; m < RPT; ++m) asm volatile("" : "+v"(raw[m]));
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_nontemporal_store(raw[m], reinterpret_cast<probe_u4*>(base + (size_t)(rg + RP * m) * D));
}
}  // namespace

hipError_t slab_stream_launch(uint16_t* pool, int32_t num_slots, const int32_t* idx, int32_t B, int32_t Nv,
                              hipStream_t stream) {
    hipLaunchKernelGGL(slab_stream_kernel, dim3((unsigned)((int64_t)B * Nv * 2)), dim3(256), 24 * 1024, stream, pool,
                       num_slots, idx, B, Nv);
    return hipGetLastError();
}

hipError_t mfma_probe_launch(int kind, int64_t iters, float* sink, int grid, hipStream_t stream) {
    switch (kind) {
        case 0: hipLaunchKernelGGL(mfma_rate_kernel<0>, dim3(grid), dim3(256), 0, stream, iters, sink); break;
        case 1: hipLaunchKernelGGL(mfma_rate_kernel<1>, dim3(grid), dim3(256), 0, stream, iters, sink); break;
        case 2: hipLaunchKernelGGL(mfma_rate_kernel<2>, dim3(grid), dim3(256), 0, stream, iters, sink); break;
        case 3: hipLaunchKernelGGL(mfma_rate_kernel<3>, dim3(grid), dim3(256), 0, stream, iters, sink); break;
        default: hipLaunchKernelGGL(mfma_rate_kernel<4>, dim3(grid), dim3(256), 0, stream, iters, sink); break;
    }
    return hipGetLastError();
}

}  // namespace gdr

extern "C" {

gdr_status gdr_timing_enable(int kernel_mask) {
    gdr::g_mask.store(kernel_mask);
    return GDR_OK;
}

const char* gdr_timing_kernel_name(int32_t id) { return gdr::kernel_name(id); }

gdr_status gdr_timing_read(double* total_ms, int32_t* launches, int32_t n) {
    if (!total_ms || !launches || n < 1) return GDR_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < n; ++i) {
        total_ms[i] = 0.0;
        launches[i] = 0;
    }
    std::vector<gdr::Rec> recs;
    {
        std::lock_guard<std::mutex> lk(gdr::g_mu);
        recs.swap(gdr::g_recs);
    }
    gdr_status st = GDR_OK;
    for (const gdr::Rec& r : recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.end) != hipSuccess || hipEventElapsedTime(&ms, r.begin, r.end) != hipSuccess)
            st = GDR_ERR_HIP;
        else if (r.id < n) {
            total_ms[r.id] += ms;
            launches[r.id] += 1;
        }
    }
    std::lock_guard<std::mutex> lk(gdr::g_mu);
    for (const gdr::Rec& r : recs) {
        gdr::g_free.push_back(r.begin);
        gdr::g_free.push_back(r.end);
    }
    return st;
}

}  // extern "C"
