// gdr_decode.hip -- token-by-token Gated Delta Rule decode over a slot pool.
//
// Operation ("lite_boost.ops.recurrent_gated_delta_rule" page, algorithm flow):
// per token, S = S*exp(g)*exp(gk); kv = S^T k; S += k ((v - kv) beta)^T;
// o = S^T (q*scale).  S is [Dk, Dv] (key dim = rows) per (slot, value head).
//
// The op is HBM-bound: each (row b, head h) streams its slot's state slab in
// once and out once per call (32 KiB each way for a bf16 128x128 slab), so
// the kernel is built around that stream:
//   * one workgroup (256 threads, 4 waves) per (b, h, column slice of CW);
//     columns of S are independent in every step of the recurrence, so a
//     slice needs no communication with the others; the one-token kernel
//     takes its rows in groups of eight, one row per XCD (place_slab);
//   * each lane owns 8 consecutive columns (one 16-byte bf16 load per row)
//     of RPT rows; rows are interleaved so that each load instruction of a
//     wave covers whole contiguous rows -- fully coalesced 128-bit traffic;
//   * the whole slab is loaded up front (RPT independent 16-byte loads per
//     lane in flight), kept in fp32 registers across the <= 8-token chain,
//     and written back once per distinct slot the chain stores into; slab
//     traffic uses non-temporal loads and stores (each byte is touched once);
//   * both reductions over the key dim (S^T k and S^T q) come out of ONE
//     pass over the decayed state: o = S_new^T q = (aS)^T q + delta (k.q),
//     so each token needs one cross-lane reduction (xor shuffles inside a
//     wave, then one LDS exchange across the 4 waves).
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

template <int DK, int CW, typename ActT, typename StT, bool ANY_RULE>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int NT = 256;
    constexpr int WAVES = NT / 64;
    constexpr int LPR = CW / 8;        // lanes per row (8 columns each)
    constexpr int RP = NT / LPR;       // rows covered by one pass of the workgroup
    constexpr int RPT = DK / RP;       // rows per thread
    static_assert(CW % 8 == 0 && LPR <= 64 && DK % RP == 0 && RPT >= 1, "bad decode tiling");
    constexpr int NRED = 17;           // 8 x (S^T k) + 8 x (S^T q) + (k . q)

    __shared__ float s_k[kMaxDecodeTokens][DK];
    __shared__ float s_q[kMaxDecodeTokens][DK];
    __shared__ float s_a[kMaxDecodeTokens][DK];
    __shared__ float s_red[2][NRED][WAVES][LPR];

    const int S = a.S, Nv = a.Nv, Dv = a.Dv;
    const int nslice = Dv / CW;
    // one row after another, each row's slabs in (head, slice) order: with
    // several tokens per row the tokens store to slots of their own, and the
    // grouped order of the one-token kernel (place_slab) measured slower here
    // (B = 64, S = 4 workload: 142.0 against 137.1 us per call, same box)
    const int wg = blockIdx.x;
    const int slice = wg % nslice;
    const int h = (wg / nslice) % Nv;
    const int b = wg / nslice / Nv;
    const int hk = h / (Nv / a.Nk);
    const int tid = threadIdx.x;
    const int cg = tid % LPR;
    const int rg = tid / LPR;
    const int wave = tid / 64, lane = tid % 64;
    const int col = slice * CW + cg * 8;

    const ActT* q = static_cast<const ActT*>(a.q);
    const ActT* k = static_cast<const ActT*>(a.k);
    const ActT* v = static_cast<const ActT*>(a.v);
    const ActT* beta = static_cast<const ActT*>(a.beta);
    ActT* out = static_cast<ActT*>(a.out);
    StT* pool = static_cast<StT*>(a.pool);
    const int32_t* idx = a.idx + (size_t)b * S;

    int len = a.lens[b];
    len = len < 0 ? 0 : (len > S ? S : len);

    const size_t tok0 = ((size_t)b * Nv + h) * S;           // token index base for [B,Nv,S]
    const size_t slab = (size_t)DK * Dv;
    const size_t slot_stride = (size_t)Nv * slab;

    // state slab (rows rg + RP*m, columns col..col+7) -> fp32 registers
    float st[RPT][8];
    // the chain resumes from the state after the last accepted token of the
    // previous call (index position n - 1; n = 1 in ordinary inference)
    int nacc = a.nacc ? a.nacc[b] : 1;
    nacc = nacc < 1 ? 1 : (nacc > S ? S : nacc);
    const int slot0 = len > 0 ? idx[nacc - 1] : -1;
    if (slot0 >= 0 && slot0 < a.num_slots) {
        const StT* base = pool + (size_t)slot0 * slot_stride + (size_t)h * slab + col;
#pragma unroll
        for (int m = 0; m < RPT; ++m) load8_nt(base + (size_t)(rg + RP * m) * Dv, st[m]);
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
#pragma unroll
            for (int c = 0; c < 8; ++c) st[m][c] = 0.f;
    }

    // update rule ("LinearAttention" page, update_rule): the delta and linear
    // rules have no decay, the gated and linear rules no delta term.  The
    // gated delta rule is compiled without the run-time choice (ANY_RULE
    // false): the choice costs registers and about a tenth of the bandwidth.
    const bool gated = !ANY_RULE || a.rule == 0 || a.rule == 2;
    const bool delta = !ANY_RULE || a.rule == 0 || a.rule == 1;
    // without the delta term, d = v: kv enters with weight 0 and beta is 1
    // (branch-free, so the token loop is not duplicated per rule)
    const float kvw = delta ? 1.f : 0.f;

    // per-token key rows, scaled query rows and row decays -> LDS
    for (int e = tid; e < len * DK; e += NT) {
        const int t = e / DK, i = e % DK;
        const size_t qi = (((size_t)b * a.Nk + hk) * S + t) * DK + i;
        s_k[t][i] = load1(k + qi);
        s_q[t][i] = load1(q + qi) * a.scale;
        const float eg = gated ? expf(a.g[tok0 + t]) : 1.f;
        s_a[t][i] = (gated && a.gk) ? eg * expf(a.gk[(tok0 + t) * DK + i]) : eg;
    }
    __syncthreads();

    for (int t = 0; t < len; ++t) {
        float vv[8];
        load8(v + (tok0 + t) * Dv + col, vv);
        const float bt = delta ? load1(beta + tok0 + t) : 1.f;

        // decay + partial reductions over this thread's rows
        float pk[8], pq[8], pkq = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) { pk[c] = 0.f; pq[c] = 0.f; }
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RP * m;
            const float ai = s_a[t][i], ki = s_k[t][i], qi = s_q[t][i];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                st[m][c] *= ai;
                pk[c] = fmaf(st[m][c], ki, pk[c]);
                pq[c] = fmaf(st[m][c], qi, pq[c]);
            }
            pkq = fmaf(ki, qi, pkq);
        }
        // reduce over the row groups inside the wave (lanes with equal cg)
#pragma unroll
        for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                pk[c] += __shfl_xor(pk[c], off);
                pq[c] += __shfl_xor(pq[c], off);
            }
            pkq += __shfl_xor(pkq, off);
        }
        // ... and across the waves (double-buffered: one barrier per token)
        float(*red)[WAVES][LPR] = s_red[t & 1];
        if (lane < LPR) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                red[c][wave][lane] = pk[c];
                red[8 + c][wave][lane] = pq[c];
            }
            red[16][wave][lane] = pkq;
        }
        __syncthreads();
        float kv[8], qs[8], kq = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) { kv[c] = 0.f; qs[c] = 0.f; }
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                kv[c] += red[c][w][cg];
                qs[c] += red[8 + c][w][cg];
            }
            kq += red[16][w][cg];
        }
        // delta rule update and output
        float d[8], o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            d[c] = bt * (vv[c] - kvw * kv[c]);
            o[c] = fmaf(d[c], kq, qs[c]);
        }
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const float ki = s_k[t][rg + RP * m];
#pragma unroll
            for (int c = 0; c < 8; ++c) st[m][c] = fmaf(ki, d[c], st[m][c]);
        }
        if (rg == 0) store8(out + (tok0 + t) * Dv + col, o);

        // store the state after token t into its slot, unless a later token
        // of this chain stores into the same slot (its write would win)
        const int slot = idx[t];
        bool later = false;
        for (int t2 = t + 1; t2 < len; ++t2) later |= (idx[t2] == slot);
        if (!later && slot >= 0 && slot < a.num_slots) {
            StT* base = pool + (size_t)slot * slot_stride + (size_t)h * slab + col;
#pragma unroll
            for (int m = 0; m < RPT; ++m) store8_nt(base + (size_t)(rg + RP * m) * Dv, st[m]);
        }
    }
    if (rg == 0) {
        float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int t = len; t < S; ++t) store8(out + (tok0 + t) * Dv + col, z);
    }
}

// One token per row (S = 1, the ordinary decode step) with a 16-bit pool:
// the slab stays in its packed 16-bit form in registers (half the registers
// of the fp32 copy the multi-token chain needs), so more workgroups fit on a
// CU and more of the stream is in flight.  Every value is widened exactly
// when used: the decay and the reductions read the packed rows once, the
// update reads them again and writes the new state.  The arithmetic per
// element is the same as in decode_kernel.
__device__ __forceinline__ void unpack8(const u32x4& r, uint16_t, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(r[i] << 16);
        x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void unpack8(const u32x4& r, _Float16, float (&x)[8]) {
    const half8 h = __builtin_bit_cast(half8, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
}

// (the register bound asks for four waves per SIMD where a lane holds at
// most 8 packed rows, which fits without spilling)
template <int DK, int CW, typename ActT, typename StT, bool ANY_RULE>
__global__ __launch_bounds__(256, DK * CW <= 128 * 128 ? 4 : 2) void decode1_kernel(DecodeArgs a) {
    constexpr int NT = 256;
    constexpr int WAVES = NT / 64;
    constexpr int LPR = CW / 8;
    constexpr int RP = NT / LPR;
    constexpr int RPT = DK / RP;
    static_assert(CW % 8 == 0 && LPR <= 64 && DK % RP == 0 && RPT >= 1, "bad decode tiling");
    static_assert(sizeof(StT) == 2, "packed slabs are 16-bit");
    constexpr int NRED = 17;

    __shared__ float s_k[DK];
    __shared__ float s_q[DK];
    __shared__ float s_a[DK];
    __shared__ float s_red[NRED][WAVES][LPR];

    const int Nv = a.Nv, Dv = a.Dv;
    const int nslice = Dv / CW;
    int b, h, slice;
    place_slab(blockIdx.x, a.B, Nv, nslice, b, h, slice);
    const int hk = h / (Nv / a.Nk);
    const int tid = threadIdx.x;
    const int cg = tid % LPR;
    const int rg = tid / LPR;
    const int wave = tid / 64, lane = tid % 64;
    const int col = slice * CW + cg * 8;

    const ActT* q = static_cast<const ActT*>(a.q);
    const ActT* k = static_cast<const ActT*>(a.k);
    const ActT* v = static_cast<const ActT*>(a.v);
    const ActT* beta = static_cast<const ActT*>(a.beta);
    ActT* out = static_cast<ActT*>(a.out);
    StT* pool = static_cast<StT*>(a.pool);

    int len = a.lens[b];
    len = len < 0 ? 0 : (len > 1 ? 1 : len);
    const size_t tok0 = (size_t)b * Nv + h;   // [B,Nv,1]
    const size_t slab = (size_t)DK * Dv;
    const size_t slot_stride = (size_t)Nv * slab;
    const int slot = len > 0 ? a.idx[b] : -1;   // the read slot is the written slot
    const bool in_pool = slot >= 0 && slot < a.num_slots;

    u32x4 raw[RPT];
    if (in_pool) {
        const StT* base = pool + (size_t)slot * slot_stride + (size_t)h * slab + col;
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            raw[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + (size_t)(rg + RP * m) * Dv));
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) raw[m] = u32x4{0u, 0u, 0u, 0u};
    }
    if (len == 0) {
        if (rg == 0) {
            float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            store8(out + tok0 * Dv + col, z);
        }
        return;
    }

    const bool gated = !ANY_RULE || a.rule == 0 || a.rule == 2;
    const bool delta = !ANY_RULE || a.rule == 0 || a.rule == 1;
    const float kvw = delta ? 1.f : 0.f;
    if (tid < DK) {
        const size_t qi = ((size_t)b * a.Nk + hk) * DK + tid;
        s_k[tid] = load1(k + qi);
        s_q[tid] = load1(q + qi) * a.scale;
        const float eg = gated ? expf(a.g[tok0]) : 1.f;
        s_a[tid] = (gated && a.gk) ? eg * expf(a.gk[tok0 * DK + tid]) : eg;
    }
    float vv[8];
    load8(v + tok0 * Dv + col, vv);
    const float bt = delta ? load1(beta + tok0) : 1.f;
    __syncthreads();

    float pk[8], pq[8], pkq = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) { pk[c] = 0.f; pq[c] = 0.f; }
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rg + RP * m;
        const float ai = s_a[i], ki = s_k[i], qi = s_q[i];
        float x[8];
        unpack8(raw[m], StT(), x);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float sd = x[c] * ai;
            pk[c] = fmaf(sd, ki, pk[c]);
            pq[c] = fmaf(sd, qi, pq[c]);
        }
        pkq = fmaf(ki, qi, pkq);
    }
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            pk[c] += __shfl_xor(pk[c], off);
            pq[c] += __shfl_xor(pq[c], off);
        }
        pkq += __shfl_xor(pkq, off);
    }
    if (lane < LPR) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            s_red[c][wave][lane] = pk[c];
            s_red[8 + c][wave][lane] = pq[c];
        }
        s_red[16][wave][lane] = pkq;
    }
    __syncthreads();
    float kv[8], qs[8], kq = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) { kv[c] = 0.f; qs[c] = 0.f; }
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            kv[c] += s_red[c][w][cg];
            qs[c] += s_red[8 + c][w][cg];
        }
        kq += s_red[16][w][cg];
    }
    float d[8], o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        d[c] = bt * (vv[c] - kvw * kv[c]);
        o[c] = fmaf(d[c], kq, qs[c]);
    }
    if (rg == 0) store8(out + tok0 * Dv + col, o);
    if (in_pool) {
        StT* base = pool + (size_t)slot * slot_stride + (size_t)h * slab + col;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rg + RP * m;
            const float ai = s_a[i], ki = s_k[i];
            float x[8];
            unpack8(raw[m], StT(), x);
#pragma unroll
            for (int c = 0; c < 8; ++c) x[c] = fmaf(ki, d[c], x[c] * ai);
            store8_nt(base + (size_t)(rg + RP * m) * Dv, x);
        }
    }
}

template <int DK, int CW, typename ActT, typename StT>
static hipError_t launch(const DecodeArgs& a, hipStream_t stream) {
    const size_t nwg = (size_t)a.B * a.Nv * (a.Dv / CW);
    if constexpr (sizeof(StT) == 2) {
        if (a.S == 1) {
            if (a.rule == 0) GDR_LAUNCH(kDecode, (decode1_kernel<DK, CW, ActT, StT, false>), dim3((unsigned)nwg), dim3(256), 0, stream, a);
            else GDR_LAUNCH(kDecode, (decode1_kernel<DK, CW, ActT, StT, true>), dim3((unsigned)nwg), dim3(256), 0, stream, a);
            return hipGetLastError();
        }
    }
    if (a.rule == 0) GDR_LAUNCH(kDecode, (decode_kernel<DK, CW, ActT, StT, false>), dim3((unsigned)nwg), dim3(256), 0, stream, a);
    else GDR_LAUNCH(kDecode, (decode_kernel<DK, CW, ActT, StT, true>), dim3((unsigned)nwg), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int DK, typename ActT, typename StT>
static hipError_t launch_dv(const DecodeArgs& a, hipStream_t stream) {
    // column slices: all of Dv up to 128; 256-column slices for wider states,
    // which keeps 32 KiB of bf16 slab in flight per workgroup when Dk = 64.
    // The one-token kernel with a 16-bit pool takes 64-column slices at
    // Dv = 128: each row piece is still one whole 128-byte line, the kernel
    // needs 78 registers instead of 113, and six workgroups share a CU instead
    // of four (B = 256 workload: 96.1 against 98.0 us per call, same box;
    // 32-column slices, half a line per row piece, took 138.9 us).
    if (a.Dv == 64) return launch<DK, 64, ActT, StT>(a, stream);
    if (a.Dv == 128) {
        if (sizeof(StT) == 2 && a.S == 1) return launch<DK, 64, ActT, StT>(a, stream);
        return launch<DK, 128, ActT, StT>(a, stream);
    }
    return launch<DK, 256, ActT, StT>(a, stream);
}

template <typename ActT, typename StT>
static hipError_t launch_dk(const DecodeArgs& a, hipStream_t stream) {
    if (a.Dk == 64) return launch_dv<64, ActT, StT>(a, stream);
    return launch_dv<128, ActT, StT>(a, stream);
}

template <typename ActT>
static hipError_t launch_st(const DecodeArgs& a, int st, hipStream_t stream) {
    if (st == kActBf16) return launch_dk<ActT, uint16_t>(a, stream);
    if (st == kActFp16) return launch_dk<ActT, _Float16>(a, stream);
    return launch_dk<ActT, float>(a, stream);
}

hipError_t decode_launch(const DecodeArgs& a, int act, int st, hipStream_t stream) {
    if (act == kActBf16) return launch_st<uint16_t>(a, st, stream);
    if (act == kActFp16) return launch_st<_Float16>(a, st, stream);
    return launch_st<float>(a, st, stream);
}

}  // namespace gdr
