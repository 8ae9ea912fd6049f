// gdr_prefill.hip -- chunked Gated Delta Rule prefill on gfx950.
//
// Method ("Qwen3Next Samples" PyPTO page, Mathematical Formulas), per
// sequence, value head and chunk of L = 128 tokens with r valid rows:
//   q^, k^   L2-normalised rows (eps 1e-6 under the root); q^ also * scale
//   g_cum    chunk-local inclusive prefix sum of the gate
//   D        D_ij = exp(g_cum_i - g_cum_j) for i >= j, else 0
//   L        L_ij = beta_i (k^_i . k^_j) D_ij for i > j, else 0
//            (the page's A = (k_beta k^T) . D . M_mask with M_mask = -1 below
//            the diagonal, i.e. A = -L)
//   T        (I - A)^-1 = (I + L)^-1   ("Matrix Inversion")
//   u, w     u = T (v beta),  w = T (k^ beta exp(g_cum))
//            ("Value and Key Cumulative Decay")
//   scan     v_new = u - w S;  o = (q^ exp(g_cum)) S + P v_new with
//            P = (q^ k^T) . D (inclusive lower triangle);
//            S <- exp(g_last) S + (k^ exp(g_last - g_cum))^T v_new
//            ("Recurrent State Attention", "State Update"; S here is the
//            [Dk, Dv] state, the page's S transposed)
//
// Kernels (all on the caller's stream, no host synchronisation):
//   chunkmap  one workgroup: cu_seqlens -> chunk table on the device.
//   intra     K1, one workgroup (8 waves) per (chunk, value head): every step
//             that does not depend on S -- norms, cumsum, decay, L, the
//             triangular inverse, u and w.  Fully parallel over chunks.
//   scan      K2, one workgroup (4 waves) per (sequence, value head, slice of
//             DS state columns).  Columns of S are independent in every step,
//             so the serial chunk loop is split over 128/DS workgroups.  S
//             stays in fp32 MFMA accumulators for the whole sequence; per
//             chunk it computes v_new = u - w S and the update, and records
//             v_new and the chunk's starting state for K3.
//   output    K3, one workgroup per (chunk, value head): o = (q^ e^g) S_c +
//             P v_new, fully parallel over chunks again.
//
// Matrix products run on the gfx950 MFMA v_mfma_f32_16x16x32_f16 (fp16
// operands, fp32 accumulation).  fp16 rather than bf16 operands: at the
// tolerances these results are held to, bf16 rounding of the operands is too
// coarse, fp16's 11-bit significand is not, and both run at the same rate.
// The triangular inverse, the gates, the decays and the carried state stay
// fp32; the merge products of the inverse use a hi/lo fp16 split (three
// MFMAs per product) so that T itself is accurate to about fp32 before it is
// rounded once for use.
//
// MFMA 16x16x32 lane layout (lane l, lr = l % 16, lq = l / 16):
//   A[16 x 32]: lane holds A[lr][8 lq + e], e = 0..7
//   B[32 x 16]: lane holds B[8 lq + e][lr]
//   C[16 x 16]: lane holds C[4 lq + e][lr], e = 0..3
#include "gdr_device.h"
#include "gdr_internal.h"

namespace gdr {

namespace {

constexpr int LD16 = 136;   // fp16 LDS row stride (elements): 272 B, 16-byte aligned rows
constexpr int LD32 = 132;   // fp32 LDS row stride (elements): 528 B
constexpr int TILE = 128 * 128;
constexpr float kNormEps = 1e-6f;

struct PrefillDev {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const float* state_in;
    void* out;
    float* state_out;
    int32_t* meta;
    int32_t* cmap;
    _Float16* khat;
    _Float16* khatT;
    _Float16* w;
    _Float16* uT;
    float* gc;
    _Float16* vnT;
    _Float16* ST;
    int64_t T;
    int64_t nc;
    int32_t B, Nqk, Nv;
    float scale;
};

__device__ __forceinline__ f32x4 mma(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 ld_h8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
__device__ __forceinline__ void st_h8(_Float16* p, half8 v) { *reinterpret_cast<half8*>(p) = v; }
__device__ __forceinline__ half4 ld_h4(const _Float16* p) { return *reinterpret_cast<const half4*>(p); }
__device__ __forceinline__ void st_h4(_Float16* p, half4 v) { *reinterpret_cast<half4*>(p) = v; }

__device__ __forceinline__ half8 to_h8(const float (&x)[8]) {
    half8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)x[e];
    return h;
}
__device__ __forceinline__ half4 to_h4(f32x4 x) {
    half4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)x[e];
    return h;
}
// x = hi + lo with hi, lo fp16: the product of two such splits keeps ~22 bits.
__device__ __forceinline__ void split8(const float (&x)[8], half8& hi, half8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const _Float16 hh = (_Float16)x[e];
        hi[e] = hh;
        lo[e] = (_Float16)(x[e] - (float)hh);
    }
}
__device__ __forceinline__ f32x4 mma_split(const float (&a)[8], const float (&b)[8], f32x4 acc) {
    half8 ah, al, bh, bl;
    split8(a, ah, al);
    split8(b, bh, bl);
    acc = mma(al, bh, acc);
    acc = mma(ah, bl, acc);
    return mma(ah, bh, acc);
}
__device__ __forceinline__ void lds_row8(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}

// ------------------------------------------------------------------ chunk map
__global__ __launch_bounds__(256) void chunkmap_kernel(const int32_t* cu, PrefillDev p) {
    __shared__ int32_t s_scan[256];
    __shared__ int32_t s_carry;
    const int tid = threadIdx.x;
    const int B = p.B;
    const int64_t T = p.T;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < B; base += 256) {
        const int b = base + tid;
        int32_t nb = 0;
        if (b < B) {
            const int64_t s0 = min<int64_t>(max<int64_t>(cu[b], 0), T);
            const int64_t e0 = min<int64_t>(max<int64_t>(cu[b + 1], s0), T);
            nb = (int32_t)((e0 - s0 + kChunk - 1) / kChunk);
        }
        s_scan[tid] = nb;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {
            const int32_t y = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += y;
            __syncthreads();
        }
        const int64_t excl = (int64_t)s_carry + s_scan[tid] - nb;
        if (b < B) p.meta[b] = (int32_t)min<int64_t>(excl, p.nc);
        __syncthreads();
        if (tid == 255) s_carry = (int32_t)min<int64_t>((int64_t)s_carry + s_scan[255], p.nc);
        __syncthreads();
    }
    if (tid == 0) p.meta[B] = s_carry;
    __syncthreads();
    const int32_t total = s_carry;
    for (int32_t c = tid; c < total; c += 256) {
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (p.meta[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int64_t s0 = min<int64_t>(max<int64_t>(cu[lo], 0), T);
        const int64_t e0 = min<int64_t>(max<int64_t>(cu[lo + 1], s0), T);
        const int64_t t = s0 + (int64_t)kChunk * (c - p.meta[lo]);
        const int64_t r = min<int64_t>(kChunk, e0 - t);
        p.cmap[4 * c + 0] = lo;
        p.cmap[4 * c + 1] = (int32_t)t;
        p.cmap[4 * c + 2] = (int32_t)max<int64_t>(r, 0);
        p.cmap[4 * c + 3] = c - p.meta[lo];
    }
}

// lower-triangular tile index n (0..35) -> (I, J) with J <= I
__device__ __forceinline__ void tri_tile(int n, int& I, int& J) {
    I = 0;
    while ((I + 1) * (I + 2) / 2 <= n) ++I;
    J = n - I * (I + 1) / 2;
}

// ------------------------------------------------------------------ K1: intra-chunk
template <typename ActT>
__global__ __launch_bounds__(512) void intra_kernel(PrefillDev p) {
    __shared__ __align__(16) _Float16 sK[128 * LD16];   // k^ [tok][dk]; after the Gram: k^T [dk][tok]
    __shared__ __align__(16) float sT[128 * LD32];      // L, then T = (I + L)^-1, row-major
    __shared__ __align__(16) _Float16 sV[128 * LD16];   // merge scratch X; then (v beta)^T [col][tok]
    __shared__ float sGc[128], sBeta[128], sBE[128];
    float* sX = reinterpret_cast<float*>(sV);

    const int Nv = p.Nv, Nqk = p.Nqk, G = Nv / Nqk;
    const int c = blockIdx.x / Nv, h = blockIdx.x % Nv, hq = h / G;
    if (c >= p.meta[p.B]) return;
    const int t0 = p.cmap[4 * c + 1], r = p.cmap[4 * c + 2];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const ActT* K = static_cast<const ActT*>(p.k);
    const ActT* V = static_cast<const ActT*>(p.v);
    const ActT* BETA = static_cast<const ActT*>(p.beta);
    const size_t ch = (size_t)c * Nv + h;
    const size_t cq = (size_t)c * Nqk + hq;
    const bool writes_keys = (h % G) == 0;   // one value head per group stores k^ for K2/K3

    // ---- 1a. gate cumulative sum and beta (wave 0; each lane owns rows 2l, 2l+1)
    if (wave == 0) {
        const int i0 = 2 * lane, i1 = i0 + 1;
        const float g0 = i0 < r ? p.g[(size_t)(t0 + i0) * Nv + h] : 0.f;
        const float g1 = i1 < r ? p.g[(size_t)(t0 + i1) * Nv + h] : 0.f;
        const float b0 = i0 < r ? load1(BETA + (size_t)(t0 + i0) * Nv + h) : 0.f;
        const float b1 = i1 < r ? load1(BETA + (size_t)(t0 + i1) * Nv + h) : 0.f;
        const float s = g0 + g1;
        float incl = s;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(incl, off);
            if (lane >= off) incl += y;
        }
        float gc0 = (incl - s) + g0, gc1 = incl;
        // rows past the chunk's end repeat g_cum of the last valid row
        const float mine = ((r - 1) & 1) ? gc1 : gc0;
        const float glast = __shfl(mine, (r - 1) >> 1);
        if (i0 >= r) gc0 = glast;
        if (i1 >= r) gc1 = glast;
        sGc[i0] = gc0; sGc[i1] = gc1;
        sBeta[i0] = b0; sBeta[i1] = b1;
        sBE[i0] = b0 * expf(gc0); sBE[i1] = b1 * expf(gc1);
        p.gc[ch * 128 + i0] = gc0;
        p.gc[ch * 128 + i1] = gc1;
    }

    // ---- 1b. k^ rows 16*wave + lr (A-fragment layout), L2-normalised
    half8 kh[4];
    {
        const int row = 16 * wave + lr;
        float kx[4][8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (row < r) load8(K + ((size_t)(t0 + row) * Nqk + hq) * 128 + 32 * ks + 8 * lq, kx[ks]);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) kx[ks][e] = 0.f;
            }
        }
        float ssq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) ssq = fmaf(kx[ks][e], kx[ks][e], ssq);
        ssq += __shfl_xor(ssq, 16);
        ssq += __shfl_xor(ssq, 32);
        const float rinv = 1.f / sqrtf(ssq + kNormEps);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) kx[ks][e] *= rinv;
            kh[ks] = to_h8(kx[ks]);
            st_h8(&sK[row * LD16 + 32 * ks + 8 * lq], kh[ks]);
            if (writes_keys) st_h8(p.khat + cq * TILE + (size_t)row * 128 + 32 * ks + 8 * lq, kh[ks]);
        }
    }
    // ---- 1c. prefetch this head's v rows (16-byte pieces: row = e/16, cols 8*(e%16))
    float vv[4][8];
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int e_ = tid + 512 * n, row = e_ >> 4, cc = e_ & 15;
        if (row < r) load8(V + ((size_t)(t0 + row) * Nv + h) * 128 + 8 * cc, vv[n]);
        else {
#pragma unroll
            for (int e = 0; e < 8; ++e) vv[n][e] = 0.f;
        }
    }
    __syncthreads();

    // ---- 2. Gram k^ k^T on the lower tiles -> L (fp32); zero the upper tiles
    for (int n = wave; n < 36; n += 8) {
        int I, J;
        tri_tile(n, I, J);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = mma(ld_h8(&sK[(16 * I + lr) * LD16 + 32 * ks + 8 * lq]),
                      ld_h8(&sK[(16 * J + lr) * LD16 + 32 * ks + 8 * lq]), acc);
        const int j = 16 * J + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * lq + e;
            sT[i * LD32 + j] = i > j ? sBeta[i] * acc[e] * expf(sGc[i] - sGc[j]) : 0.f;
        }
    }
    for (int n = wave; n < 28; n += 8) {   // upper tiles (J > I)
        int I, J;
        tri_tile(n, I, J);   // enumerate pairs J' <= I' and map to (J', I' + 1)
        const int ui = J, uj = I + 1;
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[(16 * ui + 4 * lq + e) * LD32 + 16 * uj + lr] = 0.f;
    }
    __syncthreads();

    // ---- 2b. sK now holds k^T [dk][tok] (the Gram no longer reads it)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) sK[(32 * ks + 8 * lq + e) * LD16 + 16 * wave + lr] = kh[ks][e];

    // ---- 3. inverses of the eight 16x16 diagonal blocks: T_bb = (I + L_bb)^-1,
    //         one column per lane, forward substitution in fp32
    if (tid < 128) {
        const int bb = tid >> 4, j = tid & 15;
        float* Lb = &sT[(16 * bb) * LD32 + 16 * bb];
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) acc = fmaf(-Lb[i * LD32 + kk], t[kk], acc);
            t[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Lb[i * LD32 + j] = t[i];
    }
    __syncthreads();

    // k^T -> workspace (coalesced copy of sK)
    if (writes_keys) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int e_ = tid + 512 * n, row = e_ >> 4, cc = e_ & 15;
            st_h8(p.khatT + cq * TILE + (size_t)row * 128 + 8 * cc, ld_h8(&sK[row * LD16 + 8 * cc]));
        }
    }

    // ---- 4. block doubling: for blocks of size s = 16, 32, 64, merge pairs
    //         [[T11, 0], [L21, T22]] -> T21 = -T22 (L21 T11)
    for (int s = 16; s <= 64; s *= 2) {
        const int ts = s / 16, tpm = ts * ts, nt = (64 / s) * tpm, ldx = s + 4;
        for (int n = wave; n < nt; n += 8) {
            const int m = n / tpm, tt = n % tpm, ti = tt / ts, tj = tt % ts, pb = 2 * s * m;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < s; kk += 32) {
                const int kc = kk + 8 * lq;
                float a[8], bfr[8];
                if (kc < s) {
                    lds_row8(&sT[(pb + s + 16 * ti + lr) * LD32 + pb + kc], a);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bfr[e] = sT[(pb + kc + e) * LD32 + pb + 16 * tj + lr];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) { a[e] = 0.f; bfr[e] = 0.f; }
                }
                acc = mma_split(a, bfr, acc);
            }
            float* X = sX + m * s * ldx;
#pragma unroll
            for (int e = 0; e < 4; ++e) X[(16 * ti + 4 * lq + e) * ldx + 16 * tj + lr] = acc[e];
        }
        __syncthreads();
        for (int n = wave; n < nt; n += 8) {
            const int m = n / tpm, tt = n % tpm, ti = tt / ts, tj = tt % ts, pb = 2 * s * m;
            const float* X = sX + m * s * ldx;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int kk = 0; kk < s; kk += 32) {
                const int kc = kk + 8 * lq;
                float a[8], bfr[8];
                if (kc < s) {
                    lds_row8(&sT[(pb + s + 16 * ti + lr) * LD32 + pb + s + kc], a);
#pragma unroll
                    for (int e = 0; e < 8; ++e) bfr[e] = X[(kc + e) * ldx + 16 * tj + lr];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) { a[e] = 0.f; bfr[e] = 0.f; }
                }
                acc = mma_split(a, bfr, acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) sT[(pb + s + 16 * ti + 4 * lq + e) * LD32 + pb + 16 * tj + lr] = -acc[e];
        }
        __syncthreads();
    }

    // ---- 5. (v beta)^T [col][tok] into sV (the merge scratch is dead now)
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int e_ = tid + 512 * n, row = e_ >> 4, cc = e_ & 15;
        const float bt = sBeta[row];
#pragma unroll
        for (int e = 0; e < 8; ++e) sV[(8 * cc + e) * LD16 + row] = (_Float16)(vv[n][e] * bt);
    }
    __syncthreads();

    // ---- 6. u = T (v beta) -> uT [col][tok];  w^T = (k^ beta e^g)^T T^T -> w [tok][dk]
    //         lower-triangular K ranges; waves take row tiles {pr, 7 - pr} (balanced)
    const int pr = wave & 3, hsel = wave >> 2;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const int I = which ? 7 - pr : pr;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int J = 4 * hsel + jj;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks <= I / 2; ++ks) {
                float a[8];
                lds_row8(&sT[(16 * I + lr) * LD32 + 32 * ks + 8 * lq], a);
                acc = mma(to_h8(a), ld_h8(&sV[(16 * J + lr) * LD16 + 32 * ks + 8 * lq]), acc);
            }
            st_h4(p.uT + ch * TILE + (size_t)(16 * J + lr) * 128 + 16 * I + 4 * lq, to_h4(acc));
        }
    }
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const int Jt = which ? 7 - pr : pr;          // token tile (output columns of w^T)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int It = 4 * hsel + ii;             // dk tile (output rows of w^T)
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int ks = 0; ks <= Jt / 2; ++ks) {
                const half8 kt = ld_h8(&sK[(16 * It + lr) * LD16 + 32 * ks + 8 * lq]);
                float a[8], b[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] = (float)kt[e] * sBE[32 * ks + 8 * lq + e];
                lds_row8(&sT[(16 * Jt + lr) * LD32 + 32 * ks + 8 * lq], b);
                acc = mma(to_h8(a), to_h8(b), acc);
            }
            st_h4(p.w + ch * TILE + (size_t)(16 * Jt + lr) * 128 + 16 * It + 4 * lq, to_h4(acc));
        }
    }
}

// ------------------------------------------------------------------ K2: state scan
template <int DS>
__global__ __launch_bounds__(256) void scan_kernel(PrefillDev p) {
    constexpr int NS = 128 / DS, CT = DS / 16;
    __shared__ __align__(16) _Float16 sST[DS * LD16];   // S^T [col][dk] (fp16), current chunk's start state
    __shared__ __align__(16) _Float16 sVn[DS * LD16];   // scaled v_new^T [col][tok]

    // XCD-aware placement: the NS slices of one (sequence, head) stream read
    // the same w / k^T tiles, so they are given workgroup ids that the
    // hardware dispatches to the same XCD (id mod 8) and share its L2.
    const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
    const int slice = j % NS, stream = (j / NS) * 8 + xcd;
    if (stream >= p.B * p.Nv) return;
    const int Nv = p.Nv, Nqk = p.Nqk;
    const int b = stream / Nv, h = stream % Nv, hq = h / (Nv / Nqk);
    const int col0 = slice * DS;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;

    f32x4 S[2][CT];
    const size_t sbase = (size_t)stream * TILE;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dk = 32 * wv + 16 * rt + 4 * lq + e, col = col0 + 16 * ct + lr;
                S[rt][ct][e] = p.state_in ? p.state_in[sbase + (size_t)dk * 128 + col] : 0.f;
            }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
            st_h4(&sST[(16 * ct + lr) * LD16 + 32 * wv + 16 * rt + 4 * lq], to_h4(S[rt][ct]));
    __syncthreads();

    const int c0 = p.meta[b], c1 = p.meta[b + 1];
    for (int c = c0; c < c1; ++c) {
        const size_t ch = (size_t)c * Nv + h;
        const _Float16* W = p.w + ch * TILE;
        const _Float16* KT = p.khatT + ((size_t)c * Nqk + hq) * TILE;
        const _Float16* UT = p.uT + ch * TILE;
        const float* GC = p.gc + ch * 128;
        half8 aw[2][4], ak[2][4];
        half4 u4[2][CT];
        float gcr[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int row = 32 * wv + 16 * rt + lr;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                aw[rt][ks] = ld_h8(W + (size_t)row * 128 + 32 * ks + 8 * lq);
                ak[rt][ks] = ld_h8(KT + (size_t)row * 128 + 32 * ks + 8 * lq);
            }
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
                u4[rt][ct] = ld_h4(UT + (size_t)(col0 + 16 * ct + lr) * 128 + 32 * wv + 16 * rt + 4 * lq);
#pragma unroll
            for (int e = 0; e < 4; ++e) gcr[rt][e] = GC[32 * wv + 16 * rt + 4 * lq + e];
        }
        const float glast = GC[127];

        // the state at the start of this chunk, for the output kernel
        for (int e_ = tid; e_ < DS * 16; e_ += 256) {
            const int row = e_ >> 4, cc = e_ & 15;
            st_h8(p.ST + ch * TILE + (size_t)(col0 + row) * 128 + 8 * cc, ld_h8(&sST[row * LD16 + 8 * cc]));
        }
        // v_new = u - w S
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f32x4 vp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    vp = mma(aw[rt][ks], ld_h8(&sST[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), vp);
                f32x4 vn, vs;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vn[e] = (float)u4[rt][ct][e] - vp[e];
                    vs[e] = vn[e] * expf(glast - gcr[rt][e]);
                }
                const int tok = 32 * wv + 16 * rt + 4 * lq, col = 16 * ct + lr;
                st_h4(p.vnT + ch * TILE + (size_t)(col0 + col) * 128 + tok, to_h4(vn));
                st_h4(&sVn[col * LD16 + tok], to_h4(vs));
            }
        __syncthreads();
        // S <- exp(g_last) S + k^T (v_new exp(g_last - g_cum))
        const float dec = expf(glast);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                f32x4 acc = S[rt][ct] * dec;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    acc = mma(ak[rt][ks], ld_h8(&sVn[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), acc);
                S[rt][ct] = acc;
                st_h4(&sST[(16 * ct + lr) * LD16 + 32 * wv + 16 * rt + 4 * lq], to_h4(acc));
            }
        __syncthreads();
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dk = 32 * wv + 16 * rt + 4 * lq + e, col = col0 + 16 * ct + lr;
                p.state_out[sbase + (size_t)dk * 128 + col] = S[rt][ct][e];
            }
}

// ------------------------------------------------------------------ K3: output
template <typename ActT>
__global__ __launch_bounds__(256) void output_kernel(PrefillDev p) {
    __shared__ __align__(16) _Float16 sP[128 * LD16];
    __shared__ __align__(16) float sO[4][16 * LD32];

    const int Nv = p.Nv, Nqk = p.Nqk, G = Nv / Nqk;
    const int c = blockIdx.x / Nv, h = blockIdx.x % Nv, hq = h / G;
    if (c >= p.meta[p.B]) return;
    const int t0 = p.cmap[4 * c + 1], r = p.cmap[4 * c + 2];
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const ActT* Q = static_cast<const ActT*>(p.q);
    ActT* OUT = static_cast<ActT*>(p.out);
    const size_t ch = (size_t)c * Nv + h;
    const float* GC = p.gc + ch * 128;
    const _Float16* KH = p.khat + ((size_t)c * Nqk + hq) * TILE;
    const _Float16* STc = p.ST + ch * TILE;
    const _Float16* VNT = p.vnT + ch * TILE;

    // q^ (scaled) and q^ e^{g_cum} for this wave's row tiles {wv, 7 - wv}
    half8 qh[2][4], qe[2][4];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int I = it ? 7 - wv : wv, row = 16 * I + lr;
        float x[4][8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            if (row < r) load8(Q + ((size_t)(t0 + row) * Nqk + hq) * 128 + 32 * ks + 8 * lq, x[ks]);
            else {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[ks][e] = 0.f;
            }
        }
        float ssq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) ssq = fmaf(x[ks][e], x[ks][e], ssq);
        ssq += __shfl_xor(ssq, 16);
        ssq += __shfl_xor(ssq, 32);
        const float rinv = p.scale / sqrtf(ssq + kNormEps);
        const float eg = expf(GC[row]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float y[8], z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { y[e] = x[ks][e] * rinv; z[e] = y[e] * eg; }
            qh[it][ks] = to_h8(y);
            qe[it][ks] = to_h8(z);
        }
    }
    // P = (q^ k^T) . D on the inclusive lower triangle -> sP (fp16)
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int I = it ? 7 - wv : wv;
        for (int J = 0; J <= I; ++J) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = mma(qh[it][ks], ld_h8(KH + (size_t)(16 * J + lr) * 128 + 32 * ks + 8 * lq), acc);
            const int j = 16 * J + lr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * I + 4 * lq + e;
                sP[i * LD16 + j] = (_Float16)(i >= j ? acc[e] * expf(GC[i] - GC[j]) : 0.f);
            }
        }
        if ((I & 1) == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sP[(16 * I + 4 * lq + e) * LD16 + 16 * (I + 1) + lr] = (_Float16)0.f;
        }
    }
    __syncthreads();
    // o = (q^ e^g) S_c + P v_new, then rows < r -> out
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int I = it ? 7 - wv : wv;
        f32x4 o[8];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = mma(qe[it][ks], ld_h8(STc + (size_t)(16 * ct + lr) * 128 + 32 * ks + 8 * lq), acc);
            for (int ks = 0; ks <= I / 2; ++ks)
                acc = mma(ld_h8(&sP[(16 * I + lr) * LD16 + 32 * ks + 8 * lq]),
                          ld_h8(VNT + (size_t)(16 * ct + lr) * 128 + 32 * ks + 8 * lq), acc);
            o[ct] = acc;
        }
        float* so = sO[wv];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) so[(4 * lq + e) * LD32 + 16 * ct + lr] = o[ct][e];
        __syncthreads();
        const int row = lane >> 2, seg = lane & 3, tok = 16 * I + row;
        if (tok < r) {
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                float y[8];
                lds_row8(&so[row * LD32 + 32 * seg + 8 * n], y);
                store8(OUT + ((size_t)(t0 + tok) * Nv + h) * 128 + 32 * seg + 8 * n, y);
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t prefill_launch(const PrefillArgs& a, const PrefillLayout& lay, bool act_bf16, hipStream_t stream) {
    PrefillDev p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta;
    p.state_in = a.state_in; p.out = a.out; p.state_out = a.state_out;
    p.meta = reinterpret_cast<int32_t*>(a.ws + lay.off_meta);
    p.cmap = reinterpret_cast<int32_t*>(a.ws + lay.off_cmap);
    p.khat = reinterpret_cast<_Float16*>(a.ws + lay.off_khat);
    p.khatT = reinterpret_cast<_Float16*>(a.ws + lay.off_khatT);
    p.w = reinterpret_cast<_Float16*>(a.ws + lay.off_w);
    p.uT = reinterpret_cast<_Float16*>(a.ws + lay.off_uT);
    p.gc = reinterpret_cast<float*>(a.ws + lay.off_gc);
    p.vnT = reinterpret_cast<_Float16*>(a.ws + lay.off_vnT);
    p.ST = reinterpret_cast<_Float16*>(a.ws + lay.off_ST);
    p.T = a.T; p.nc = lay.nc; p.B = a.B; p.Nqk = a.Nqk; p.Nv = a.Nv; p.scale = a.scale;

    timing_begin(kChunkmap, stream);
    hipLaunchKernelGGL(chunkmap_kernel, dim3(1), dim3(256), 0, stream, a.cu, p);
    timing_end(kChunkmap, stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t nwg = (size_t)lay.nc * a.Nv;
    if (nwg > 0) {
        timing_begin(kIntra, stream);
        if (act_bf16) hipLaunchKernelGGL(intra_kernel<uint16_t>, dim3((unsigned)nwg), dim3(512), 0, stream, p);
        else hipLaunchKernelGGL(intra_kernel<float>, dim3((unsigned)nwg), dim3(512), 0, stream, p);
        timing_end(kIntra, stream);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    constexpr int DS = 32;
    const size_t nstream = (size_t)a.B * a.Nv;
    const size_t nscan = (nstream + 7) / 8 * 8 * (128 / DS);
    timing_begin(kScan, stream);
    hipLaunchKernelGGL(scan_kernel<DS>, dim3((unsigned)nscan), dim3(256), 0, stream, p);
    timing_end(kScan, stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (nwg > 0) {
        timing_begin(kOutput, stream);
        if (act_bf16) hipLaunchKernelGGL(output_kernel<uint16_t>, dim3((unsigned)nwg), dim3(256), 0, stream, p);
        else hipLaunchKernelGGL(output_kernel<float>, dim3((unsigned)nwg), dim3(256), 0, stream, p);
        timing_end(kOutput, stream);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gdr
