/*
 * gdr_oracle.c -- fp64 CPU oracle for the Gated Delta Rule.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it and shares no code with it.
 *
 * What it computes is the plain per-token recurrence, in double precision,
 * one (sequence or batch row, value head) stream at a time:
 *
 *   S <- S * exp(g) * exp(gk)           (gk per key row; absent = 0)
 *   kv_mem = S^T k
 *   S <- S + k ((v - kv_mem) * beta)^T
 *   o = S^T (q * scale)
 *
 * Source: "lite_boost.ops.recurrent_gated_delta_rule" (MindSpore Lite API
 * page), algorithm-flow section: state decay, memory retrieval, delta update,
 * output.  S is [Dk, Dv] with the key dimension as rows (same page, parameter
 * "state": D_k rows, D_v columns).
 *
 * The chunked prefill is an exact rearrangement of the same recurrence
 * ("Qwen3Next Samples" PyPTO page, Mathematical Formulas); the oracle
 * therefore runs the recurrence token by token over each packed sequence.
 * Prefill additionally L2-normalises q and k inside the operator with
 * eps = 1e-6 under the square root ("Qwen3Next Samples", L2 Normalization
 * formula and the l2norm submodule, default eps 1e-6) and multiplies q by
 * `scale` (the decode page states that q is multiplied by the scale before
 * computation; the same convention is used for prefill).
 *
 * Update rules ("LinearAttention" contrib-operator page, attribute
 * update_rule: linear, gated, delta, gated_delta; the page names them
 * without formulas).  The plain readings, each dropping parts of the
 * recurrence above:
 *   rule 0  gated_delta   the recurrence above (default)
 *   rule 1  delta         no decay: g and gk are ignored (exp(.) = 1)
 *   rule 2  gated         no delta term: S <- S * exp(g) * exp(gk) + k v^T
 *                         (beta and kv_mem are not used)
 *   rule 3  linear        neither: S <- S + k v^T
 * The codes are part of the C ABI of the GPU library as well.
 *
 * Value head h reads query/key head h / (Nv / Nqk) (contiguous GQA groups).
 * The pages only require Nv to be a multiple of Nqk; the contiguous grouping
 * is a convention both sides of the parity tests fix.
 *
 * Parity pins: every function here is pinned by the CPU tests against
 * brute-force agreement with an independent statement of the chunked
 * formulas, hand-derived golden values and closed forms (unit-key read-back,
 * beta = 0 identity, pure decay, orthonormal keys = causal linear attention,
 * per-key reset).  None of the functions is "parity unpinned".
 *
 * Parallelism: OpenMP over independent (sequence, value head) streams when
 * compiled with -fopenmp; results do not depend on the thread count (each
 * stream is computed by one thread in a fixed order).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GDR_ORACLE_EPS 1e-6

/* Round a double to the nearest bfloat16 value (8 significant bits, ties to
 * even), returned as a double.  Used only to state what a bf16 state pool
 * stores after an exact update. */
double gdr_oracle_round_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double m = frexp(x, &e);            /* x = m * 2^e, 0.5 <= |m| < 1 */
    m = nearbyint(m * 256.0) / 256.0;    /* 8 significant bits, ties-to-even */
    return ldexp(m, e);
}

/* Round a double to the nearest IEEE binary16 value (11 significant bits,
 * ties to even; subnormals below 2^-14 in steps of 2^-24; magnitudes that
 * round past 65504 become infinite), returned as a double.  Used only to
 * state what an fp16 state pool stores after an exact update. */
double gdr_oracle_round_fp16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    const double ax = fabs(x);
    double r;
    if (ax < ldexp(1.0, -14)) {
        r = nearbyint(ax * ldexp(1.0, 24)) * ldexp(1.0, -24);
    } else {
        int e;
        const double m = frexp(ax, &e);          /* ax = m * 2^e, 0.5 <= m < 1 */
        r = ldexp(nearbyint(m * 2048.0) / 2048.0, e);
        if (r > 65504.0) r = INFINITY;
    }
    return x < 0 ? -r : r;
}

/* One token of the recurrence on an fp64 state S [Dk][Dv] (row-major).
 *   decay_row[i] = exp(g) * exp(gk[i]) (precomputed by the caller; 1 for
 *   rules without a gate)
 *   delta: nonzero for the delta rules; otherwise S += k v^T (beta unused)
 *   q_scaled = q * scale
 * Writes o [Dv].  kv is caller scratch of length Dv. */
static void token_step(double *S, int Dk, int Dv,
                       const double *decay_row,
                       const double *k, const double *v, double beta, int delta,
                       const double *q_scaled, double *o, double *kv)
{
    /* state decay: row i scaled by exp(g) * exp(gk_i) */
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j)
            S[(size_t)i * Dv + j] *= decay_row[i];
    if (delta) {
        /* memory retrieval: kv_mem = S^T k */
        for (int j = 0; j < Dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < Dk; ++i) acc += S[(size_t)i * Dv + j] * k[i];
            kv[j] = acc;
        }
        /* delta update: S += k ((v - kv_mem) * beta)^T */
        for (int i = 0; i < Dk; ++i)
            for (int j = 0; j < Dv; ++j)
                S[(size_t)i * Dv + j] += k[i] * ((v[j] - kv[j]) * beta);
    } else {
        /* additive update: S += k v^T */
        for (int i = 0; i < Dk; ++i)
            for (int j = 0; j < Dv; ++j)
                S[(size_t)i * Dv + j] += k[i] * v[j];
    }
    /* output: o = S^T (q * scale) */
    for (int j = 0; j < Dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < Dk; ++i) acc += S[(size_t)i * Dv + j] * q_scaled[i];
        o[j] = acc;
    }
}

/* x / sqrt(sum x^2 + eps), times mul. */
static void l2norm(const double *x, int n, double mul, double *y)
{
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss + GDR_ORACLE_EPS);
    for (int i = 0; i < n; ++i) y[i] = x[i] * inv * mul;
}

/*
 * Chunked-prefill semantics, computed token by token.
 *   q, k      [T][Nqk][Dk]   raw (normalised here)
 *   v         [T][Nv][Dv]
 *   g, beta   [T][Nv]
 *   gk        [T][Nv][Dk] or NULL (no per-key gate): state row i of value
 *             head h at token t decays by exp(g[t][h]) * exp(gk[t][h][i]),
 *             the decode page's per-key gate applied to every prefill token
 *   state_in  [B][Nv][Dk][Dv] or NULL (= zeros)
 *   cu_seqlens[B+1], cu[0] = 0, non-decreasing, cu[B] = T
 *   out       [T][Nv][Dv]
 *   state_out [B][Nv][Dk][Dv]
 *   rule      update rule 0..3 (see above)
 * Returns 0 on success, -1 on invalid sizes, -2 on allocation failure.
 */
int gdr_oracle_prefill(const double *q, const double *k, const double *v,
                       const double *g, const double *gk, const double *beta,
                       const double *state_in, const int32_t *cu_seqlens,
                       int T, int B, int Nqk, int Nv, int Dk, int Dv,
                       double scale, int rule, double *out, double *state_out)
{
    if (T < 0 || B < 1 || Nqk < 1 || Nv < 1 || Dk < 1 || Dv < 1 || Nv % Nqk || rule < 0 || rule > 3)
        return -1;
    const int gated = rule == 0 || rule == 2, delta = rule == 0 || rule == 1;
    const int G = Nv / Nqk;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long sh = 0; sh < (long)B * Nv; ++sh) {
        const int b = (int)(sh / Nv), h = (int)(sh % Nv), hq = h / G;
        double *S = state_out + (size_t)sh * Dk * Dv;
        double *scratch = (double *)malloc(sizeof(double) * (size_t)(3 * Dk + Dv));
        if (!scratch) { failed = 1; continue; }
        double *qs = scratch, *ks = qs + Dk, *kv = ks + Dk, *decay = kv + Dv;
        if (state_in) memcpy(S, state_in + (size_t)sh * Dk * Dv, sizeof(double) * (size_t)Dk * Dv);
        else memset(S, 0, sizeof(double) * (size_t)Dk * Dv);
        for (int t = cu_seqlens[b]; t < cu_seqlens[b + 1]; ++t) {
            l2norm(q + ((size_t)t * Nqk + hq) * Dk, Dk, scale, qs);
            l2norm(k + ((size_t)t * Nqk + hq) * Dk, Dk, 1.0, ks);
            const double a = gated ? exp(g[(size_t)t * Nv + h]) : 1.0;
            for (int i = 0; i < Dk; ++i)
                decay[i] = (gated && gk) ? a * exp(gk[((size_t)t * Nv + h) * Dk + i]) : a;
            token_step(S, Dk, Dv, decay, ks, v + ((size_t)t * Nv + h) * Dv,
                       delta ? beta[(size_t)t * Nv + h] : 0.0, delta, qs,
                       out + ((size_t)t * Nv + h) * Dv, kv);
        }
        free(scratch);
    }
    return failed ? -2 : 0;
}

/*
 * Recurrent decode over a slot-indexed state pool.
 *   q, k      [B][Nk][S][Dk]  caller-normalised; NOT re-normalised here
 *   v         [B][Nv][S][Dv]
 *   g         [B][Nv][S]
 *   gk        [B][Nv][S][Dk] or NULL (no per-key gate)
 *   beta      [B][Nv][S]
 *   pool_in   [slots][Nv][Dk][Dv]  state before the call
 *   pool_out  [slots][Nv][Dk][Dv]  must hold a copy of pool_in on entry;
 *                                  receives the state after each token
 *   idx       [B*S]   slot per flattened token
 *   lens      [B]     valid tokens per row, 0..S
 *   num_accepted [B] or NULL: accepted-token count per row ("num_accepted_tokens"
 *               in the "lite_boost.ops.recurrent_gated_delta_rule" page's
 *               parameter list: the tokens accepted, not rejected, in
 *               speculative decoding; equal to the valid length in ordinary
 *               inference).  NULL means 1 for every row.
 *   round_mode: 1 (2): what is stored into pool_out is the bf16 (fp16)
 *               rounding of the exact state (what such a pool holds); 0
 *               stores it exactly.  The token chain itself stays exact.
 *   out       [B][Nv][S][Dv]
 *   rule      update rule 0..3 (see above)
 *
 * Routing (the pages give one index per flattened token and say ordinary
 * inference uses one slot per row): with n = num_accepted[b] clamped to
 * 1..S, the chain of row b starts from slot idx[b*S + n - 1] -- the slot that
 * holds the state after the last accepted token of the previous call, whose
 * per-token states went to the same index positions; in ordinary inference
 * all of a row's indices name one slot, so n does not matter.  An initial
 * slot outside 0..slots-1 starts the chain from a zero state.  The state
 * after token t is stored into slot idx[b*S + t]; tokens t >= lens[b] are
 * neither read nor written and their out rows are 0.
 * Returns 0, -1 on invalid sizes / an index out of range, -2 on allocation
 * failure.
 */
int gdr_oracle_decode(const double *q, const double *k, const double *v,
                      const double *g, const double *gk, const double *beta,
                      const double *pool_in, double *pool_out, int num_slots,
                      const int32_t *idx, const int32_t *lens, const int32_t *num_accepted,
                      int B, int S, int Nk, int Nv, int Dk, int Dv,
                      double scale, int round_mode, int rule, double *out)
{
    if (B < 1 || S < 1 || Nk < 1 || Nv < 1 || Dk < 1 || Dv < 1 || Nv % Nk || num_slots < 1 ||
        rule < 0 || rule > 3)
        return -1;
    const int gated = rule == 0 || rule == 2, delta = rule == 0 || rule == 1;
    for (int b = 0; b < B; ++b) {
        if (lens[b] < 0 || lens[b] > S) return -1;
        for (int t = 0; t < lens[b]; ++t)
            if (idx[b * S + t] < 0 || idx[b * S + t] >= num_slots) return -1;
    }
    const int G = Nv / Nk;
    const size_t slab = (size_t)Dk * Dv;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
    for (long bh = 0; bh < (long)B * Nv; ++bh) {
        const int b = (int)(bh / Nv), h = (int)(bh % Nv), hk = h / G;
        double *Sm = (double *)malloc(sizeof(double) * (slab + 2 * (size_t)Dk + Dv));
        if (!Sm) { failed = 1; continue; }
        double *qs = Sm + slab, *decay = qs + Dk, *kv = decay + Dk;
        for (int t = 0; t < S; ++t)
            memset(out + (((size_t)b * Nv + h) * S + t) * Dv, 0, sizeof(double) * (size_t)Dv);
        if (lens[b] > 0) {
            int n = num_accepted ? num_accepted[b] : 1;
            n = n < 1 ? 1 : (n > S ? S : n);
            const int s0 = idx[b * S + n - 1];
            if (s0 >= 0 && s0 < num_slots)
                memcpy(Sm, pool_in + ((size_t)s0 * Nv + h) * slab, sizeof(double) * slab);
            else
                memset(Sm, 0, sizeof(double) * slab);
            for (int t = 0; t < lens[b]; ++t) {
                const size_t tq = (((size_t)b * Nk + hk) * S + t) * Dk;
                const size_t tv = ((size_t)b * Nv + h) * S + t;
                for (int i = 0; i < Dk; ++i) qs[i] = q[tq + i] * scale;
                const double a = gated ? exp(g[tv]) : 1.0;
                for (int i = 0; i < Dk; ++i)
                    decay[i] = (gated && gk) ? a * exp(gk[tv * Dk + i]) : a;
                token_step(Sm, Dk, Dv, decay, k + tq, v + tv * Dv, delta ? beta[tv] : 0.0, delta, qs,
                           out + tv * Dv, kv);
                double *dst = pool_out + ((size_t)idx[b * S + t] * Nv + h) * slab;
                for (size_t e = 0; e < slab; ++e)
                    dst[e] = round_mode == 1 ? gdr_oracle_round_bf16(Sm[e])
                           : round_mode == 2 ? gdr_oracle_round_fp16(Sm[e]) : Sm[e];
            }
        }
        free(Sm);
    }
    return failed ? -2 : 0;
}

/* Number of threads the OpenMP runtime will use (1 without OpenMP). */
int gdr_oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
