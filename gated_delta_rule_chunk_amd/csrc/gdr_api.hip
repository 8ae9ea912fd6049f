// gdr_api.hip -- the extern "C" entry points declared in include/gdr.h:
// host-side argument validation (before any HIP call), workspace sizing and
// dispatch to the kernel launchers on the caller's stream.
#include "gdr.h"
#include "gdr_internal.h"

#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>

namespace {

thread_local char g_last_error[512] = "";

gdr_status fail(gdr_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

gdr_status ok() {
    g_last_error[0] = '\0';
    return GDR_OK;
}

gdr_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(GDR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

namespace gdr {

PrefillLayout prefill_layout(int64_t T, int32_t B, int32_t Nqk, int32_t Nv, bool gk) {
    PrefillLayout L{};
    L.nc = (T + (int64_t)B * (kChunk - 1)) / kChunk;
    const size_t tile16 = (size_t)kChunk * kHeadDim * 2;   // one 128x128 fp16 tile
    const size_t nc = (size_t)L.nc;
    size_t off = 0;
    L.off_meta = off;  off = align256(off + sizeof(int32_t) * ((size_t)B + 2));
    L.off_cmap = off;  off = align256(off + sizeof(int32_t) * 4 * nc);
    L.gk = gk;
    // with a per-key gate, k^T carries the value head's decays (one per value head)
    L.off_khatT = off; off = align256(off + tile16 * nc * (size_t)(gk ? Nv : Nqk));
    L.off_w = off;     off = align256(off + tile16 * nc * (size_t)Nv);
    L.off_u = off;     off = align256(off + tile16 * nc * (size_t)Nv);
    L.off_gc = off;    off = align256(off + sizeof(float) * kChunk * nc * (size_t)Nv);
    L.off_scvn = off;  off = align256(off + 2 * tile16 * nc * (size_t)Nv);
    L.off_qt = off;
    if (gk) off = align256(off + tile16 * nc * (size_t)Nv);
    L.off_pm = off;
    if (gk) off = align256(off + tile16 * nc * (size_t)Nv);
    // Two-level scan when the (sequence, value head) streams cannot fill the
    // GPU (even at 8 column slices each, 16 streams are 128 workgroups) and
    // the sequences are long: segments are sized so that the segment maps of
    // all streams make about 256 workgroups (two per stream segment), and
    // kept at 8 chunks or more.  nc bounds every sequence's chunk count, so
    // no sequence has more than nseg segments.
    const int64_t streams = (int64_t)B * Nv;
    L.nseg = 1;
    L.seg_len = 1 << 30;
    if (streams <= 16 && L.nc >= 64 * (int64_t)B) {
        const int64_t want = std::min<int64_t>(32, std::max<int64_t>(2, 256 / (2 * streams)));
        const int64_t len = std::max<int64_t>(8, (L.nc + want - 1) / want);
        L.seg_len = (int32_t)len;
        L.nseg = (int32_t)((L.nc + len - 1) / len);
    }
    const size_t nsd = (size_t)B * (size_t)L.nseg * (size_t)Nv;
    L.off_mb = off;
    if (L.nseg > 1) off = align256(off + sizeof(float) * nsd * kHeadDim * 2 * kHeadDim);
    L.off_sstart = off;
    if (L.nseg > 1) off = align256(off + sizeof(float) * nsd * kHeadDim * kHeadDim);
    L.total = off;
    return L;
}

}  // namespace gdr

static gdr_status check_prefill_sizes(int64_t T, int32_t B, int32_t Nqk, int32_t Nv, int32_t D) {
    if (T < 0) return fail(GDR_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %lld)", (long long)T);
    if (B < 1) return fail(GDR_ERR_INVALID_ARGUMENT, "B must be >= 1 (got %d)", B);
    if (Nqk < 1 || Nv < 1)
        return fail(GDR_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (Nqk=%d, Nv=%d)", Nqk, Nv);
    if (Nv % Nqk != 0)
        return fail(GDR_ERR_INVALID_ARGUMENT, "Nv (%d) must be a multiple of Nqk (%d)", Nv, Nqk);
    if (D < 1) return fail(GDR_ERR_INVALID_ARGUMENT, "D must be >= 1 (got %d)", D);
    if (D != gdr::kHeadDim)
        return fail(GDR_ERR_UNSUPPORTED, "prefill supports D = 128 only (got %d)", D);
    if (T > 0x7fffffffLL) return fail(GDR_ERR_INVALID_ARGUMENT, "T must be < 2^31 (got %lld)", (long long)T);
    return ok();
}

extern "C" {

const char* gdr_status_string(int status) {
    switch (status) {
        case GDR_OK: return "GDR_OK";
        case GDR_ERR_INVALID_ARGUMENT: return "GDR_ERR_INVALID_ARGUMENT";
        case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED";
        case GDR_ERR_DTYPE: return "GDR_ERR_DTYPE";
        case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE";
        case GDR_ERR_HIP: return "GDR_ERR_HIP";
        default: return "unknown status";
    }
}

const char* gdr_last_error(void) { return g_last_error; }

int gdr_version(void) { return 200; }

gdr_status gdr_chunk_prefill_workspace_size(int64_t T, int32_t B, int32_t Nqk, int32_t Nv, int32_t D,
                                            int32_t with_gk, size_t* bytes) {
    if (!bytes) return fail(GDR_ERR_INVALID_ARGUMENT, "bytes must not be NULL");
    gdr_status s = check_prefill_sizes(T, B, Nqk, Nv, D);
    if (s != GDR_OK) return s;
    *bytes = gdr::prefill_layout(T, B, Nqk, Nv, with_gk != 0).total;
    return ok();
}

static bool rule_ok(gdr_update_rule r) {
    return r == GDR_RULE_GATED_DELTA || r == GDR_RULE_DELTA || r == GDR_RULE_GATED || r == GDR_RULE_LINEAR;
}
static bool rule_gated(gdr_update_rule r) { return r == GDR_RULE_GATED_DELTA || r == GDR_RULE_GATED; }
static bool rule_delta(gdr_update_rule r) { return r == GDR_RULE_GATED_DELTA || r == GDR_RULE_DELTA; }

}  // extern "C"

// Device scratch of gdr_chunk_prefill_noalloc: one copy of this array per GPU,
// resident from the library's load until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a
// device address); it uses the address hipGetSymbolAddress returns for the
// current device, looked up once per device and kept in g_scratch.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's address of `scratch`.
gdr_status scratch_address(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return from_hip(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(GDR_ERR_HIP, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(GDR_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch[dev] = p;
    }
    *ptr = g_scratch[dev];
    return ok();
}

// Validation and launch shared by both prefill entry points.  With
// `use_scratch`, the workspace is this device's scratch array (the size
// check against its capacity comes before any HIP call).
gdr_status prefill_entry(const void* q, const void* k, const void* v, const float* g, const float* gk,
                         const void* beta, const float* state_in, const int32_t* cu_seqlens, int64_t T,
                         int32_t B, int32_t Nqk, int32_t Nv, int32_t D, float scale, gdr_update_rule rule,
                         gdr_dtype act, void* out, float* state_out, void* workspace, size_t workspace_bytes,
                         bool use_scratch, void* hip_stream) {
    gdr_status s = check_prefill_sizes(T, B, Nqk, Nv, D);
    if (s != GDR_OK) return s;
    if (act != GDR_BF16 && act != GDR_FP32 && act != GDR_FP16)
        return fail(GDR_ERR_DTYPE, "activation dtype must be GDR_BF16, GDR_FP16 or GDR_FP32 (got %d)", (int)act);
    if (!rule_ok(rule)) return fail(GDR_ERR_INVALID_ARGUMENT, "unknown update rule %d", (int)rule);
    if (!cu_seqlens || !state_out)
        return fail(GDR_ERR_INVALID_ARGUMENT, "cu_seqlens and state_out must not be NULL");
    if (T > 0 && (!q || !k || !v || !out || (rule_gated(rule) && !g) || (rule_delta(rule) && !beta)))
        return fail(GDR_ERR_INVALID_ARGUMENT,
                    "q, k, v, out (and g for the gated rules, beta for the delta rules) must not be NULL "
                    "when T > 0");
    // the per-key gate applies only to the rules with decay
    const float* gk_used = rule_gated(rule) ? gk : nullptr;
    const gdr::PrefillLayout lay = gdr::prefill_layout(T, B, Nqk, Nv, gk_used != nullptr);
    if (use_scratch) {
        if (lay.total > (size_t)GDR_NOALLOC_SCRATCH_BYTES)
            return fail(GDR_ERR_WORKSPACE,
                        "these sizes need %zu bytes of workspace%s, more than the %zu-byte scratch of "
                        "gdr_chunk_prefill_noalloc; use gdr_chunk_prefill with a caller workspace",
                        lay.total, gk_used ? " (with a per-key gate)" : "", (size_t)GDR_NOALLOC_SCRATCH_BYTES);
        s = scratch_address(&workspace);
        if (s != GDR_OK) return s;
        workspace_bytes = GDR_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < lay.total)
        return fail(GDR_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu, ptr %p)%s", lay.total,
                    workspace_bytes, workspace, gk_used ? " (with a per-key gate)" : "");
    gdr::PrefillArgs a{q, k, v, g, gk_used, beta, state_in, cu_seqlens, out, state_out,
                       static_cast<char*>(workspace), T, B, Nqk, Nv, scale, (int32_t)rule};
    return from_hip(gdr::prefill_launch(a, lay, (int)act, static_cast<hipStream_t>(hip_stream)),
                    "prefill launch");
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_prefill(const void* q, const void* k, const void* v, const float* g,
                             const float* gk, const void* beta, const float* state_in,
                             const int32_t* cu_seqlens,
                             int64_t T, int32_t B, int32_t Nqk, int32_t Nv, int32_t D, float scale,
                             gdr_update_rule rule, gdr_dtype act, void* out, float* state_out,
                             void* workspace, size_t workspace_bytes, void* hip_stream) {
    return prefill_entry(q, k, v, g, gk, beta, state_in, cu_seqlens, T, B, Nqk, Nv, D, scale, rule, act, out,
                         state_out, workspace, workspace_bytes, false, hip_stream);
}

gdr_status gdr_chunk_prefill_noalloc(const void* q, const void* k, const void* v, const float* g,
                                     const float* gk, const void* beta, const float* state_in,
                                     const int32_t* cu_seqlens, int64_t T, int32_t B, int32_t Nqk, int32_t Nv,
                                     int32_t D, float scale, gdr_update_rule rule, gdr_dtype act, void* out,
                                     float* state_out, void* hip_stream) {
    return prefill_entry(q, k, v, g, gk, beta, state_in, cu_seqlens, T, B, Nqk, Nv, D, scale, rule, act, out,
                         state_out, nullptr, 0, true, hip_stream);
}

gdr_status gdr_recurrent_decode(const void* q, const void* k, const void* v, const float* g,
                                const float* gk, const void* beta, void* state_pool, int32_t num_slots,
                                const int32_t* ssm_state_indices, const int32_t* actual_seq_lengths,
                                const int32_t* num_accepted_tokens, int32_t B, int32_t S, int32_t Nk,
                                int32_t Nv, int32_t Dk, int32_t Dv, float scale, gdr_update_rule rule,
                                gdr_dtype act, gdr_dtype state_dtype, void* out, void* hip_stream) {
    if (B < 1) return fail(GDR_ERR_INVALID_ARGUMENT, "B must be >= 1 (got %d)", B);
    if (S < 1 || S > gdr::kMaxDecodeTokens)
        return fail(GDR_ERR_INVALID_ARGUMENT, "S must be in [1, %d] (got %d)", gdr::kMaxDecodeTokens, S);
    if (Nk < 1 || Nv < 1)
        return fail(GDR_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (Nk=%d, Nv=%d)", Nk, Nv);
    if (Nv % Nk != 0)
        return fail(GDR_ERR_INVALID_ARGUMENT, "Nv (%d) must be a multiple of Nk (%d)", Nv, Nk);
    if (num_slots < 1) return fail(GDR_ERR_INVALID_ARGUMENT, "num_slots must be >= 1 (got %d)", num_slots);
    if (Dk < 1 || Dv < 1) return fail(GDR_ERR_INVALID_ARGUMENT, "Dk, Dv must be >= 1 (Dk=%d, Dv=%d)", Dk, Dv);
    if (Dk != 64 && Dk != 128) return fail(GDR_ERR_UNSUPPORTED, "decode supports Dk in {64, 128} (got %d)", Dk);
    if (Dv != 64 && Dv != 128 && Dv != 256 && Dv != 512)
        return fail(GDR_ERR_UNSUPPORTED, "decode supports Dv in {64, 128, 256, 512} (got %d)", Dv);
    auto dt_ok = [](gdr_dtype d) { return d == GDR_BF16 || d == GDR_FP32 || d == GDR_FP16; };
    if (!dt_ok(act) || !dt_ok(state_dtype))
        return fail(GDR_ERR_DTYPE, "dtypes must be GDR_BF16, GDR_FP16 or GDR_FP32 (act=%d, state=%d)", (int)act,
                    (int)state_dtype);
    if (!rule_ok(rule)) return fail(GDR_ERR_INVALID_ARGUMENT, "unknown update rule %d", (int)rule);
    if (!q || !k || !v || !state_pool || !ssm_state_indices || !actual_seq_lengths || !out ||
        (rule_gated(rule) && !g) || (rule_delta(rule) && !beta))
        return fail(GDR_ERR_INVALID_ARGUMENT,
                    "only gk, num_accepted_tokens, g (rules without a gate) and beta (rules without the "
                    "delta term) may be NULL");
    if ((int64_t)B * Nv * (Dv / (Dv == 64 ? 64 : 128)) > 0x7fffffffLL)
        return fail(GDR_ERR_INVALID_ARGUMENT, "B * Nv too large");
    gdr::DecodeArgs a{q, k, v, g, gk, beta, state_pool, ssm_state_indices, actual_seq_lengths,
                      num_accepted_tokens, out, num_slots, B, S, Nk, Nv, Dk, Dv, scale, (int32_t)rule};
    return from_hip(gdr::decode_launch(a, (int)act, (int)state_dtype,
                                       static_cast<hipStream_t>(hip_stream)),
                    "decode launch");
}

gdr_status gdr_mfma_peak_probe(int32_t kind, int64_t iters, float* sink, int64_t sink_floats,
                               double* flops_per_launch, void* hip_stream) {
    if (kind < 0 || kind >= gdr::kProbeKinds)
        return fail(GDR_ERR_INVALID_ARGUMENT, "probe kind must be 0..%d (got %d)", gdr::kProbeKinds - 1, kind);
    if (iters < 1 || iters > (int64_t(1) << 24))
        return fail(GDR_ERR_INVALID_ARGUMENT, "probe iterations must be 1..2^24 (got %lld)", (long long)iters);
    if (!sink || !flops_per_launch) return fail(GDR_ERR_INVALID_ARGUMENT, "sink and flops_per_launch must not be NULL");
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return from_hip(e, "querying the device");
    const int64_t grid = (int64_t)cus * gdr::kProbeWgsPerCu;
    if (sink_floats < grid * 256)
        return fail(GDR_ERR_INVALID_ARGUMENT, "sink holds %lld floats; the probe writes %lld", (long long)sink_floats,
                    (long long)(grid * 256));
    *flops_per_launch = (double)grid * 4 * (double)iters * gdr::kProbeChains[kind] * gdr::kProbeFlops[kind];
    return from_hip(gdr::mfma_probe_launch(kind, iters, sink, (int)grid, static_cast<hipStream_t>(hip_stream)),
                    "probe launch");
}

gdr_status gdr_slab_stream_probe(void* pool, int32_t num_slots, const int32_t* ssm_state_indices, int32_t B,
                                 int32_t Nv, void* hip_stream) {
    if (!pool || !ssm_state_indices) return fail(GDR_ERR_INVALID_ARGUMENT, "pool and ssm_state_indices must not be NULL");
    if (B < 1 || Nv < 1 || num_slots < 1)
        return fail(GDR_ERR_INVALID_ARGUMENT, "B, Nv and num_slots must be >= 1 (B=%d, Nv=%d, num_slots=%d)", B, Nv,
                    num_slots);
    if ((int64_t)B * Nv > 0x7fffffffLL) return fail(GDR_ERR_INVALID_ARGUMENT, "B * Nv must be < 2^31");
    return from_hip(gdr::slab_stream_launch(static_cast<uint16_t*>(pool), num_slots, ssm_state_indices, B, Nv,
                                            static_cast<hipStream_t>(hip_stream)),
                    "probe launch");
}

}  // extern "C"
