// gdr_internal.h -- host-side interface between the C ABI layer and the
// kernel launchers (not part of the public ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

constexpr int kMaxDecodeTokens = 8;   // the decode page limits S to 8
constexpr int kChunk = 128;           // L, fixed by the prefill page
constexpr int kHeadDim = 128;         // D, fixed by the prefill page

// Kernel ids for the opt-in per-kernel timing (gdr_timing_*).
enum KernelId { kChunkmap = 0, kIntra = 1, kScan = 2, kOutput = 3, kDecode = 4, kKernelCount = 5 };
// When kernel id is selected for timing: two events for one launch of it,
// already recorded as that launch's pair (true); false otherwise.
bool timing_events(int id, hipEvent_t* start, hipEvent_t* stop);
const char* kernel_name(int id);

// Launch KERNEL on STREAM.  A launch of a kernel selected for timing goes
// through hipExtLaunchKernelGGL, whose start and stop events the dispatch
// itself records at the kernel's start and end (no marker packets beside the
// kernel).  A timed launch still costs the stream a few microseconds (about
// 5 us per step of the T=8192 prefill), so time only the kernels needed.
#define GDR_LAUNCH(ID, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)                                          \
    do {                                                                                                \
        hipEvent_t gdr_t0_, gdr_t1_;                                                                    \
        if (::gdr::timing_events((ID), &gdr_t0_, &gdr_t1_))                                             \
            hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, gdr_t0_, gdr_t1_, 0u, __VA_ARGS__); \
        else                                                                                            \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);                         \
    } while (0)

// The MFMA issue-rate probe (gdr_mfma_peak_probe): kinds, flops per
// instruction, and one launch of `grid` workgroups of four waves.
constexpr int kProbeKinds = 5;
constexpr int kProbeWgsPerCu = 8;     // four-wave workgroups per CU: 32 waves, eight per SIMD
// independent accumulator chains per wave, and flops per instruction
constexpr int kProbeChains[kProbeKinds] = {8, 8, 8, 8, 4};
constexpr double kProbeFlops[kProbeKinds] = {16.0 * 16 * 32 * 2, 16.0 * 16 * 32 * 2, 16.0 * 16 * 16 * 2,
                                             16.0 * 16 * 4 * 2, 32.0 * 32 * 16 * 2};
hipError_t mfma_probe_launch(int kind, int64_t iters, float* sink, int grid, hipStream_t stream);
// The slab-stream probe (gdr_slab_stream_probe): one 16-bit 128 x 128 slab
// per (row, head) workgroup, read and written back in place, in the
// one-token decode's workgroup order and access pattern.
hipError_t slab_stream_launch(uint16_t* pool, int32_t num_slots, const int32_t* idx, int32_t B, int32_t Nv,
                              hipStream_t stream);

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* gk;
    const void* beta;
    void* pool;
    const int32_t* idx;
    const int32_t* lens;
    const int32_t* nacc;   // accepted tokens per row, or null (= 1)
    void* out;
    int32_t num_slots, B, S, Nk, Nv, Dk, Dv;
    float scale;
    int32_t rule;          // update rule code (0 gated_delta, 1 delta, 2 gated, 3 linear)
};

// Element dtype codes (the values of gdr_dtype): fp32, bf16 (stored as
// uint16_t bit patterns), IEEE half (_Float16).
constexpr int kActFp32 = 0, kActBf16 = 1, kActFp16 = 2;

hipError_t decode_launch(const DecodeArgs& a, int act, int state, hipStream_t stream);

// Which (row b, value head h, column slice) workgroup wg of the one-token
// decode (and of the slab-stream probe, its traffic alone) streams.  Rows go in
// groups of eight; inside a group, consecutive workgroups take the group's
// rows in turn, and each row's slabs follow in (head, slice) order.  The
// hardware hands workgroup ids to the eight XCDs in turn (id mod 8), so each
// row's slot, one contiguous region of Nv slabs, is streamed through one
// XCD, and each XCD walks its rows' slots one after another.  Measured on the
// B = 256 workload (random slots, whole 128-column slabs) against one row
// after another with its slabs spread over all XCDs: 97.7 against 102.6 us
// per call, same box; groups of 2, 4 and 16 rows gave 101.6, 100.5 and
// 99.2 us.  A last group of
// fewer than eight rows (B not a multiple of 8) keeps the same order with
// its own row count.
__device__ __forceinline__ void place_slab(int wg, int B, int Nv, int nslice, int& b, int& h, int& slice) {
    constexpr int R = 8;
    const int per = Nv * nslice;               // workgroups per row
    const int b0 = (wg / (R * per)) * R;       // first row of the group
    const int rows = min(R, B - b0);
    const int w = wg - b0 * per;               // place inside the group
    b = b0 + w % rows;
    const int rest = w / rows;
    h = rest / nslice;
    slice = rest % nslice;
}

// ---------------------------------------------------------------- prefill
//
// Workspace layout.  NC = upper bound on the number of 128-token chunks over
// all sequences: sum_b ceil(len_b / 128) <= (T + B*127) / 128.  Every
// per-(chunk, head) tile is 128 x 128 fp16 (32 KiB), zero-padded past the
// chunk's valid rows.  Tiles marked "fragment order" hold their elements in
// the order of the MFMA registers that write or read them (the prefill
// source defines the two orders), not row-major.
struct PrefillLayout {
    int64_t nc;             // chunk bound
    size_t off_meta;        // int32 [B+2]: first chunk of each sequence, then the total
    size_t off_cmap;        // int4  [NC]: (sequence, first token, valid rows, -)
    bool gk;                // a per-key gate is applied (the tiles below change as noted)
    size_t off_khatT;       // fp16  [NC][Nqk] 128 dk x 128 tok, fragment order: normalised keys, transposed
                            //       (per-key gate: [NC][Nv], k^ exp(G_last - G) per value head)
    size_t off_w;           // fp16  [NC][Nv]  128 tok x 128 dk, fragment order: w = T (k^ beta e^gcum)
    size_t off_u;           // fp16  [NC][Nv]  128 tok x 128 col, fragment order: u = T (v beta)
    size_t off_gc;          // fp32  [NC][Nv][128]               chunk-local cumulative gate
                            //       (per-key gate: G_last[dk], the chunk's decay of state row dk)
    size_t off_scvn;        // fp16  [NC][Nv]  2 x 128 x 128, paired fragment order: state at chunk
                            //                 start S_c [dk][col] with v_new = u - w S [tok][col]
    // Two-level scan for few, long streams (nseg > 1): every sequence is cut
    // into segments of seg_len chunks (at most nseg of them); each segment's
    // affine map S_end = M S_start + B is found first, then the start states.
    int32_t nseg;           // segments per sequence (1: one-level scan)
    int32_t seg_len;        // chunks per segment
    size_t off_mb;          // fp32  [B][nseg][Nv] 128 dk x 256: M (cols 0..127) | B (cols 128..255)
    size_t off_sstart;      // fp32  [B][nseg][Nv] 128 dk x 128: start state of each segment
    size_t off_qt;          // per-key gate only: fp16 [NC][Nv] 128 tok x 128 dk, fragment order:
                            //       q^ exp(G), the decayed queries of the state term
    size_t off_pm;          // per-key gate only: fp16 [NC][Nv] 128 x 128 tok, fragment order: the
                            //       decayed intra-chunk scores P (zero above the diagonal)
    size_t total;
};

PrefillLayout prefill_layout(int64_t T, int32_t B, int32_t Nqk, int32_t Nv, bool gk);

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* gk;       // per-key gate [T, Nv, 128] or NULL (none, or a rule without decay)
    const void* beta;
    const float* state_in;
    const int32_t* cu;
    void* out;
    float* state_out;
    char* ws;
    int64_t T;
    int32_t B, Nqk, Nv;
    float scale;
    int32_t rule;          // update rule code (0 gated_delta, 1 delta, 2 gated, 3 linear)
};

hipError_t prefill_launch(const PrefillArgs& a, const PrefillLayout& lay, int act,
                          hipStream_t stream);

}  // namespace gdr
