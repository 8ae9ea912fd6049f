/*
 * gdr.h -- C ABI of the MI355X (gfx950) Gated Delta Rule library (libgdr.so).
 *
 * Two operations, each a direct statement of a page:
 *
 *   gdr_chunk_prefill     chunked prefill over varlen-packed sequences
 *                         ("Qwen3Next Samples" PyPTO page: chunk_gated_delta_rule,
 *                         Mathematical Formulas and Parameter Description)
 *   gdr_recurrent_decode  token-by-token decode over a slot-indexed state pool
 *                         ("lite_boost.ops.recurrent_gated_delta_rule" page:
 *                         algorithm flow, parameters, returns, exceptions)
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers, dense, row-major (C order), in the
 *     layouts stated per argument.  Non-contiguous tensors are not supported
 *     (the prefill page says the same of every tensor).  All pointers are
 *     owned by the caller; the library never allocates, frees or keeps them.
 *   - Scratch memory is the caller's: query its size first, then pass it in
 *     (the two-phase workspace-then-execute convention of the CANN aclnn
 *     pages).  The library holds no device memory of its own.
 *   - All work is enqueued on `hip_stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises the host with the device.
 *   - Arguments are validated on the host, before any HIP call; a failed
 *     check returns a status code and enqueues nothing.  The value ranges
 *     the pages leave unchecked stay unchecked (log-gates g, gk negative;
 *     decode q, k of unit norm; cu_seqlens monotone with last = T; slot
 *     indices inside the pool): outside them the results are meaningless,
 *     but the kernels clamp every index and offset they derive from device
 *     data, so no such input makes them access memory out of bounds.
 *   - Results are deterministic: repeated calls on the same inputs give
 *     bit-identical outputs (no floating-point atomics).
 *   - A thread-local text describing the last failed check is available
 *     from gdr_last_error().
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below are passed and returned as C ints.  In C++ they get int as
 * their fixed underlying type, so that an implementation may receive any int
 * value (and reject the unknown ones) without undefined behaviour; in C an
 * enum with these values is an int already. */
#ifdef __cplusplus
#define GDR_ENUM_INT : int
#else
#define GDR_ENUM_INT
#endif

/* Status codes.  The Python binding maps GDR_ERR_INVALID_ARGUMENT to
 * ValueError (shape / count / grouping errors, as the decode page's
 * exceptions section assigns them) and every other failure to RuntimeError
 * (dtype errors and backend failures, as the same section assigns them). */
typedef enum gdr_status GDR_ENUM_INT {
    GDR_OK = 0,
    GDR_ERR_INVALID_ARGUMENT = 1, /* bad size, count, head grouping or NULL pointer */
    GDR_ERR_UNSUPPORTED = 2,      /* allowed by the pages but not built here (e.g. D != 128) */
    GDR_ERR_DTYPE = 3,            /* unsupported dtype combination */
    GDR_ERR_WORKSPACE = 4,        /* workspace NULL or smaller than required */
    GDR_ERR_HIP = 5               /* a HIP launch or runtime call failed */
} gdr_status;

/* Element types of activation and state tensors. */
/* Element dtypes.  GDR_FP16 is IEEE binary16 (the LinearAttention page
 * allows float16 or float32 activations and state); GDR_BF16 is the
 * recurrent_gated_delta_rule page's dtype. */
typedef enum gdr_dtype GDR_ENUM_INT {
    GDR_FP32 = 0,
    GDR_BF16 = 1,
    GDR_FP16 = 2
} gdr_dtype;

/* State update rule ("LinearAttention" contrib-operator page, attribute
 * update_rule, which names linear, gated, delta and gated_delta without
 * formulas).  Readings: each rule drops parts of the gated delta rule
 *   S = S exp(g) exp(gk);  S = S + k ((v - S^T k) beta)^T;  o = S^T q:
 *   GDR_RULE_GATED_DELTA  all of it (the default of both pages)
 *   GDR_RULE_DELTA        no decay (g and gk are ignored and may be NULL)
 *   GDR_RULE_GATED        no delta term: S = S exp(g) exp(gk) + k v^T
 *                         (beta is ignored and may be NULL)
 *   GDR_RULE_LINEAR       neither: S = S + k v^T */
typedef enum gdr_update_rule GDR_ENUM_INT {
    GDR_RULE_GATED_DELTA = 0,
    GDR_RULE_DELTA = 1,
    GDR_RULE_GATED = 2,
    GDR_RULE_LINEAR = 3
} gdr_update_rule;

/* Static text for a status code ("unknown status" for other values). */
const char *gdr_status_string(int status);

/* Thread-local description of the last non-OK status returned on this
 * thread ("" if none). */
const char *gdr_last_error(void);

/* Library ABI version (major * 100 + minor). */
int gdr_version(void);

/* ------------------------------------------------------------------ prefill
 *
 * gdr_chunk_prefill_workspace_size
 *   Bytes of device workspace gdr_chunk_prefill needs for these sizes.
 *   T >= 0 total packed tokens; B >= 1 sequences; Nqk >= 1 query/key heads;
 *   Nv a multiple of Nqk; D must be 128; with_gk != 0 if the call will pass
 *   a per-key gate (it needs more workspace).  Writes *bytes; returns
 *   GDR_ERR_INVALID_ARGUMENT / GDR_ERR_UNSUPPORTED on bad sizes.
 */
gdr_status gdr_chunk_prefill_workspace_size(int64_t T, int32_t B, int32_t Nqk, int32_t Nv,
                                            int32_t D, int32_t with_gk, size_t *bytes);

/*
 * gdr_chunk_prefill -- chunked Gated Delta Rule forward ("Qwen3Next
 * Samples" page, chunk_gated_delta_rule).
 *
 * Per sequence b (tokens cu_seqlens[b] .. cu_seqlens[b+1]-1) and value head h
 * (query/key head h / (Nv/Nqk)), with the state S [Dk=D, Dv=D] starting at
 * state_in[b,h] (zeros if state_in is NULL), the operator computes, token
 * by token (the chunked form with L = 128 is an exact rearrangement):
 *   q^ = q / sqrt(sum q^2 + 1e-6) * scale,  k^ = k / sqrt(sum k^2 + 1e-6)
 *   S = exp(g) S  (row i also times exp(gk[i]) with a per-key gate);
 *   S = S + k^ ((v - S^T k^) beta)^T;  out = S^T q^
 * and writes the final S to state_out[b,h].  A sequence of length 0 passes
 * its state through unchanged.  `rule` selects a reduced update (see
 * gdr_update_rule); q and k are L2-normalised inside for every rule.
 *
 * Arithmetic: MFMA operands are fp16 with fp32 accumulation.  The state is
 * carried in fp32, but u, v_new, the chunk-start states and the operand of
 * the state in w S are held in fp16, so entries of v (times beta) and of the
 * state must stay inside the fp16 range: magnitudes beyond about 3e4 can
 * overflow to inf.  Unit keys and decaying gates keep both at the scale of v.
 *
 *   q, k        [T, Nqk, D]   act dtype   (raw; normalised inside)
 *   v           [T, Nv, D]    act dtype
 *   g           [T, Nv]       fp32        log-decay gate (expected < 0)
 *   gk          [T, Nv, D]    fp32 or NULL: per-key log-decay gate (the decode
 *                             page's gk, applied at every token; expected < 0,
 *                             of any magnitude: a gk of -1e4 resets its key
 *                             row of the state); ignored by the rules without
 *                             decay.  A non-NULL gk needs the workspace
 *                             queried with with_gk = 1.  Per-token log-decays
 *                             (g, or g + gk) below -80 act as -80: exp(-80) is
 *                             below fp32 resolution, so this changes nothing
 *                             visible and keeps the chunk sums in range
 *   beta        [T, Nv]       act dtype   (expected in [0, 1])
 *   state_in    [B, Nv, D, D] fp32 or NULL (= zeros); key dim = rows
 *   cu_seqlens  [B + 1]       int32, device; cu[0] = 0, non-decreasing, cu[B] = T
 *   T, B, Nqk, Nv, D          sizes; D must be 128 (the page fixes D = L = 128)
 *   scale                     multiplies the normalised q (e.g. 1/sqrt(D))
 *   rule                      update rule; g may be NULL without a gate,
 *                             beta without the delta term
 *   act                       GDR_BF16, GDR_FP16 or GDR_FP32 (q, k, v, beta, out)
 *   out         [T, Nv, D]    act dtype
 *   state_out   [B, Nv, D, D] fp32; may be the same pointer as state_in
 *   workspace   device memory of at least the size the query returns
 *   hip_stream                hipStream_t the work is enqueued on
 */
gdr_status gdr_chunk_prefill(const void *q, const void *k, const void *v, const float *g,
                             const float *gk, const void *beta, const float *state_in,
                             const int32_t *cu_seqlens,
                             int64_t T, int32_t B, int32_t Nqk, int32_t Nv, int32_t D,
                             float scale, gdr_update_rule rule, gdr_dtype act, void *out,
                             float *state_out, void *workspace, size_t workspace_bytes,
                             void *hip_stream);

/*
 * gdr_chunk_prefill_noalloc -- gdr_chunk_prefill without a caller workspace,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * The library keeps one scratch array of GDR_NOALLOC_SCRATCH_BYTES per GPU
 * (a static device array, resident on every GPU the library runs on from
 * its load until the process ends) and runs the prefill in it.  Sizes whose
 * workspace (gdr_chunk_prefill_workspace_size) exceeds that return
 * GDR_ERR_WORKSPACE before any HIP call.  The call allocates and frees no
 * memory; the first call on a device looks up that device's address of the
 * array (hipGetSymbolAddress) and keeps it.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (no part of it needs to start at zero: each call writes every
 * region before reading it).  Calls ordered on one stream are safe; calls
 * that may overlap in time on one GPU (different streams, or threads without
 * ordering between them) race on the array and give wrong results.
 *
 * Arguments, results and errors are those of gdr_chunk_prefill, without
 * workspace and workspace_bytes.
 */
#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
gdr_status gdr_chunk_prefill_noalloc(const void *q, const void *k, const void *v, const float *g,
                                     const float *gk, const void *beta, const float *state_in,
                                     const int32_t *cu_seqlens, int64_t T, int32_t B, int32_t Nqk,
                                     int32_t Nv, int32_t D, float scale, gdr_update_rule rule,
                                     gdr_dtype act, void *out, float *state_out, void *hip_stream);

/* ------------------------------------------------------------------ decode
 *
 * gdr_recurrent_decode -- token-by-token Gated Delta Rule over a state pool
 * ("lite_boost.ops.recurrent_gated_delta_rule" page).
 *
 * For batch row b, value head h (key head h / (Nv/Nk)), the token chain
 * starts from the slot state_pool[ssm_state_indices[b*S + n - 1], h], where
 * n is num_accepted_tokens[b] clamped to [1, S] (n = 1 if the pointer is
 * NULL); for each valid token t < actual_seq_lengths[b]:
 *   S = S * exp(g) * exp(gk)     (gk per key row; omitted if gk is NULL)
 *   S = S + k ((v - S^T k) beta)^T
 *   out[b,h,t] = S^T (q * scale)
 * and the state after token t is stored, in the pool's dtype (bf16 rounds
 * to nearest even), into slot ssm_state_indices[b*S + t].  When several
 * tokens of a row name one slot, the last one's state is what remains.
 * Tokens t >= actual_seq_lengths[b] are neither read nor written in the
 * pool, and their out rows are written as zeros.  Slots no token writes keep
 * their bits.  Rows must not write slots that other rows read or write.
 *
 * num_accepted_tokens is the page's count of accepted (not rejected) tokens
 * in speculative decoding, equal to actual_seq_lengths in ordinary
 * inference: a call that drafted S tokens leaves the state after each draft
 * token t in slot ssm_state_indices[b*S + t], and the next call, given the
 * same index positions and n accepted tokens, resumes from the state after
 * the n-th.  In ordinary inference a row's indices all name one slot and n
 * does not matter.
 *
 *   q, k                [B, Nk, S, Dk]  act dtype, caller-normalised (unit L2 norm)
 *   v                   [B, Nv, S, Dv]  act dtype
 *   g                   [B, Nv, S]      fp32 (expected < 0)
 *   gk                  [B, Nv, S, Dk]  fp32 (expected < 0) or NULL
 *   beta                [B, Nv, S]      act dtype (expected in [0, 1])
 *   state_pool          [num_slots, Nv, Dk, Dv]  state dtype, updated in place
 *   ssm_state_indices   [B * S]         int32, device
 *   actual_seq_lengths  [B]             int32, device, each in [0, S]
 *   num_accepted_tokens [B]             int32, device, or NULL
 *   B >= 1; 1 <= S <= 8 (decode only, as the page limits it);
 *   Nv a multiple of Nk; Dk in {64, 128}; Dv in {64, 128, 256, 512}
 *   scale               multiplies q before use (the page's scale_value)
 *   rule                update rule (see gdr_update_rule); g may be NULL
 *                       without a gate, beta without the delta term
 *   act                 GDR_BF16, GDR_FP16 or GDR_FP32 (q, k, v, beta, out)
 *   state_dtype         GDR_BF16 (the page's pool), GDR_FP16 or GDR_FP32
 *   out                 [B, Nv, S, Dv]  act dtype
 * Out-of-range slot indices are not checked on the host (they live on the
 * device); a token whose slot is out of range stores nothing, and a chain
 * whose first slot is out of range starts from a zero state.  Lengths are
 * clamped to [0, S].
 */
gdr_status gdr_recurrent_decode(const void *q, const void *k, const void *v, const float *g,
                                const float *gk, const void *beta, void *state_pool,
                                int32_t num_slots, const int32_t *ssm_state_indices,
                                const int32_t *actual_seq_lengths,
                                const int32_t *num_accepted_tokens, int32_t B, int32_t S,
                                int32_t Nk, int32_t Nv, int32_t Dk, int32_t Dv, float scale,
                                gdr_update_rule rule, gdr_dtype act, gdr_dtype state_dtype,
                                void *out, void *hip_stream);

/* ------------------------------------------------------------------ timing
 *
 * Opt-in per-kernel timing, for benchmarks and profiling.  gdr_timing_enable
 * takes a bit mask of kernel ids (bit i for kernel i; GDR_TIMING_ALL for
 * every kernel, 0 to switch timing off).  Every launch of a selected kernel
 * goes through hipExtLaunchKernelGGL with two hipEvents that its dispatch on
 * the caller's stream records at the kernel's start and end (a timed launch
 * still adds a few microseconds to the stream, so time only the kernels
 * needed).
 * gdr_timing_read waits for those events, writes for each kernel id i < n the
 * summed duration total_ms[i] and the number of launches launches[i]
 * recorded since the previous read, and forgets them.  Kernel ids:
 * 0 gdr_chunkmap, 1 gdr_intra, 2 gdr_scan, 3 gdr_output (the prefill
 * kernels, in launch order) and 4 gdr_decode.  With a per-key gate and a
 * one-level scan the scan forms the output itself and gdr_output records no
 * launch.  Off is the default; the hooks then cost nothing measurable.
 */
#define GDR_TIMING_KERNELS 5
#define GDR_TIMING_ALL (-1)
gdr_status gdr_timing_enable(int kernel_mask);
gdr_status gdr_timing_read(double *total_ms, int32_t *launches, int32_t n);
const char *gdr_timing_kernel_name(int32_t id);

/* gdr_mfma_peak_probe -- the dense MFMA issue rate of this GPU, for the
 * roofline's compute peak measured on the part rather than taken from its
 * data sheet.  Enqueues on hip_stream one launch of 8 workgroups of four
 * waves per CU; every wave runs 8 independent accumulator chains (4 for
 * kind 4) of `iters` instructions of one kind:
 *   kind 0  v_mfma_f32_16x16x32_f16   (the prefill's main products)
 *   kind 1  v_mfma_f32_16x16x32_bf16
 *   kind 2  v_mfma_f32_16x16x16_f16   (the block substitution)
 *   kind 3  v_mfma_f32_16x16x4_f32    (the per-key gate's wide diagonal blocks)
 *   kind 4  v_mfma_f32_32x32x16_f16   (the larger fp16 tile, for comparison)
 * and writes one float per thread to sink (device memory the caller owns, at
 * least sink_floats = CUs * 8 * 256 floats): in thread 0 of each workgroup,
 * sink[256 * workgroup], the shader clock in MHz over that workgroup's run
 * (s_memtime cycles against the 100 MHz real-time counter); elsewhere a sum
 * of the products, with no meaning.
 * *flops_per_launch (host) receives the launch's flop count; timing it (for
 * example with hipEvents on the same stream) gives the rate.  iters is
 * 1..2^24.  Errors: GDR_ERR_INVALID_ARGUMENT (kind, iters, NULL pointers, a
 * sink too small) before any launch, GDR_ERR_HIP from the runtime.
 */
gdr_status gdr_mfma_peak_probe(int32_t kind, int64_t iters, float *sink, int64_t sink_floats,
                               double *flops_per_launch, void *hip_stream);

/* gdr_slab_stream_probe -- the memory traffic of the one-token decode alone,
 * for the HBM ceiling of its access pattern: enqueues on hip_stream two
 * workgroups per (row b < B, value head h < Nv), one per 64-column half,
 * that read the 16-bit 128 x 128 slab state_pool[ssm_state_indices[b], h] (a
 * pool of num_slots x Nv such slabs, bf16 or fp16, device memory) and write
 * the same bytes back, with the decode's thread layout, workgroup order and
 * non-temporal 16-byte accesses; rows whose index is outside [0, num_slots)
 * are skipped.  The
 * pool's values do not change.  ssm_state_indices is int32 [B] on the device.
 * Errors: GDR_ERR_INVALID_ARGUMENT (NULL pointers, sizes below 1) before any
 * launch, GDR_ERR_HIP from the runtime.
 */
gdr_status gdr_slab_stream_probe(void *state_pool, int32_t num_slots, const int32_t *ssm_state_indices, int32_t B,
                                 int32_t Nv, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
