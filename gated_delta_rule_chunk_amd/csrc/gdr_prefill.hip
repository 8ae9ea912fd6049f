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
//             diagonal blocks of T, and u and w by block forward substitution
//             (T itself is never formed).  Fully parallel over chunks.
//   scan      K2, one workgroup (8 waves) per (sequence, value head, slice of
//             DS state columns).  Columns of S are independent in every step,
//             so the serial chunk loop is split over 128/DS workgroups.  S
//             stays in fp32 MFMA accumulators for the whole sequence; per
//             chunk it computes v_new = u - w S and the update, and records
//             v_new and the chunk's starting state for K3.
//   output    K3, one workgroup per (chunk, value head): o = (q^ e^g) S_c +
//             P v_new, fully parallel over chunks again.
//   With a per-key gate the intra kernel also stores the output's two A
//   operands (q^ e^G and P), and the one-level scan forms the output itself
//   (scan_gk_out): S_c and v_new never leave the chip and K3 does not run.
//
// Matrix products run on the gfx950 MFMA v_mfma_f32_16x16x32_f16 (fp16
// operands, fp32 accumulation).  fp16 rather than bf16 operands: at the
// tolerances these results are held to, bf16 rounding of the operands is too
// coarse, fp16's 11-bit significand is not, and both run at the same rate.
// The gates, the decays, the diagonal blocks of the triangular solve and the
// carried state stay fp32.
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
constexpr int TILE = 128 * 128;
constexpr float kNormEps = 1e-6f;
// Per-token log-decays (g, or g + gk[d] with a per-key gate) below
// -kLogDecayFloor act as -kLogDecayFloor.  exp(-80) = 1.8e-35, so a term that
// passes through such a decay is already below fp32 resolution next to any
// term that does not, and the result cannot change; the floor keeps the
// chunk-local prefix sums G small enough (|G| <= 128 * 80) that differences
// G_i - G_j of tokens behind a reset (a gate of, say, -1e4) keep fp32
// precision.
constexpr float kLogDecayFloor = 80.f;

// Update rules ("LinearAttention" page, update_rule; codes as in the C ABI):
// 0 gated_delta, 1 delta (no decay), 2 gated (no delta term), 3 linear
// (neither).  Only the intra kernel depends on the rule: without a gate the
// gates are zero; without the delta term L = 0 (so T = I), u = v and w = 0,
// which turns the scan's v_new = u - w S into v.
template <int RULE> struct Rule {
    static constexpr bool gated = RULE == 0 || RULE == 2;
    static constexpr bool delta = RULE == 0 || RULE == 1;
};

struct PrefillDev {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const void* beta;
    const float* state_in;
    void* out;
    float* state_out;
    const int32_t* cu;   // cu_seqlens [B+1]
    int32_t* meta;
    int32_t* cmap;
    _Float16* khatT;
    _Float16* w;
    _Float16* u;
    float* gc;
    _Float16* scvn;
    const float* gk;   // per-key gate [T][Nv][128] or NULL
    _Float16* qt;      // per-key gate: q^ exp(G) [NC][Nv] fragment order
    _Float16* pm;      // per-key gate: decayed scores P [NC][Nv] fragment order
    float* mb;       // two-level scan: segment maps [B][nseg][Nv] 128 x 256
    float* sstart;   // two-level scan: segment start states [B][nseg][Nv] 128 x 128
    int64_t T;
    int64_t nc;
    int32_t B, Nqk, Nv;
    int32_t nseg, seg_len;
    int32_t map_in_intra;   // the intra kernel builds the chunk map itself (no chunkmap_kernel launch)
    float scale;
};

__device__ __forceinline__ f32x4 mma(half8 a, half8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(half4 a, half4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ half8 ld_h8(const _Float16* p) { return *reinterpret_cast<const half8*>(p); }
__device__ __forceinline__ void st_h8(_Float16* p, half8 v) { *reinterpret_cast<half8*>(p) = v; }
__device__ __forceinline__ half4 ld_h4(const _Float16* p) { return *reinterpret_cast<const half4*>(p); }
__device__ __forceinline__ void st_h4(_Float16* p, half4 v) { *reinterpret_cast<half4*>(p) = v; }
// streaming store (evict-first in the caches): for results that no workgroup of
// the same kernel reads back, so they do not push shared operand tiles out of L2
__device__ __forceinline__ void st_h8_nt(_Float16* p, half8 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<half8*>(p));
}

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

// The same chunk map, built by every workgroup of the intra kernel into LDS
// when there are at most kMapSeqs sequences, which saves the chunkmap launch:
// per sequence b its first chunk, clamped first token and clamped length
// (sm[b], sm[kMapSeqs + 1 + b], sm[2 kMapSeqs + 1 + b]; sm[B] the chunk
// total; three more words for the scan's partial sums).  Workgroup 0 also
// writes meta, and the workgroups share out the cmap entries, for the
// kernels that follow.
constexpr int kMapSeqs = 168;
constexpr int kMapInts = 3 * kMapSeqs + 4;

__device__ void build_chunk_map(const PrefillDev& p, int32_t* sm, int tid) {
    int32_t* tmp = sm + 3 * kMapSeqs + 1;
    const int B = p.B;   // <= kMapSeqs
    const int64_t T = p.T;
    int32_t nb = 0;
    if (tid < B) {
        const int64_t s0 = min<int64_t>(max<int64_t>(p.cu[tid], 0), T);
        const int64_t e0 = min<int64_t>(max<int64_t>(p.cu[tid + 1], s0), T);
        nb = (int32_t)((e0 - s0 + kChunk - 1) / kChunk);
        sm[kMapSeqs + 1 + tid] = (int32_t)s0;
        sm[2 * kMapSeqs + 1 + tid] = (int32_t)(e0 - s0);
    }
    const int wave = tid >> 6, lane = tid & 63;
    int32_t incl = nb;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
    }
    if (lane == 63 && wave < 3) tmp[wave] = incl;
    __syncthreads();
    int32_t base = 0;
    for (int w = 0; w < wave && w < 3; ++w) base += tmp[w];
    const int32_t nc = (int32_t)p.nc;
    if (tid < B) sm[tid] = min(base + incl - nb, nc);
    if (tid == B - 1) sm[B] = min(base + incl, nc);
    __syncthreads();
    if (blockIdx.x == 0 && tid <= B) p.meta[tid] = sm[tid];
    const int32_t total = sm[B];
    for (int64_t c = blockIdx.x + (int64_t)gridDim.x * tid; c < total; c += (int64_t)gridDim.x * 512) {
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sm[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int32_t j = (int32_t)c - sm[lo];
        int4 e;
        e.x = lo;
        e.y = sm[kMapSeqs + 1 + lo] + kChunk * j;
        e.z = min(kChunk, sm[2 * kMapSeqs + 1 + lo] - kChunk * j);
        e.w = j;
        *reinterpret_cast<int4*>(&p.cmap[4 * c]) = e;
    }
}

// First token and valid rows of chunk c (wave-uniform) from the LDS map.
__device__ __forceinline__ void chunk_from_map(const int32_t* sm, int B, int c, int& t0, int& r) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (__builtin_amdgcn_readfirstlane(sm[mid]) <= c) lo = mid; else hi = mid - 1;
    }
    const int j = c - __builtin_amdgcn_readfirstlane(sm[lo]);
    t0 = __builtin_amdgcn_readfirstlane(sm[kMapSeqs + 1 + lo]) + kChunk * j;
    r = min(kChunk, __builtin_amdgcn_readfirstlane(sm[2 * kMapSeqs + 1 + lo]) - kChunk * j);
}

// Transposed fp16 tiles ([col][tok] or [dk][tok]) are stored with the 16-byte
// group index XOR-swizzled by the row's 8-row block, so that both the
// transposing 16-byte writes and the MFMA fragment reads are free of LDS bank
// conflicts.  Element (r, c) of such a tile:
__device__ __forceinline__ int sw(int r, int c) {
    return r * LD16 + ((((c >> 3) ^ (r >> 3)) & 15) << 3) + (c & 7);
}

// Workgroup ids are dispatched round-robin over the 8 XCDs (id mod 8), each
// with its own L2.  group_slot(id, G) renumbers them so that the G
// consecutive slots of one qk-head group -- items (chunk, value head) that
// read the same k and q rows -- run on one XCD, one after the other, and the
// second read hits that L2:
//   slot = ((id / 8) / G * 8 + id % 8) * G + (id / 8) % G,
// a bijection on [0, n) for n a multiple of 8 G (launches round up to one).
__device__ __forceinline__ int group_slot(int id, int G) {
    const int x = id & 7, j = id >> 3;
    return ((j / G) * 8 + x) * G + j % G;
}

// Workspace tiles that are written or read straight from MFMA registers are
// stored in the order of those registers, so that every such access is
// 512 B - 1 KiB contiguous (whole cache lines):
//  * A-fragment order (k^T [dk][tok], w [tok][dk]): element (r, k) sits at
//    16x32 block (r / 16, k / 32), lane 16 ((k / 8) % 4) + r % 16 of that
//    block, element k % 8 of the lane's 8.
//  * C-fragment order (u [tok][col]): element (r, c) sits at 16x16 block
//    (r / 16, c / 16), lane 16 ((r / 4) % 4) + c % 16, element r % 4.
//  * Paired C-fragment order (S_c [dk][col] with v_new [tok][col]): the two
//    tiles in C-fragment order with their lane runs interleaved -- the 4
//    elements of S_c at cfrag_off(r, c) and then the 4 of v_new at the same
//    offset form one 16-byte piece, at element 2 cfrag_off(r, c).
__device__ __forceinline__ int frag_off(int r, int k) {
    return (((r >> 4) * 4 + (k >> 5)) * 64 + ((k >> 3) & 3) * 16 + (r & 15)) * 8 + (k & 7);
}
__device__ __forceinline__ int cfrag_off(int r, int c) {
    return (((r >> 4) * 8 + (c >> 4)) * 64 + ((r >> 2) & 3) * 16 + (c & 15)) * 4 + (r & 3);
}
// Row and first column of the 8-element piece number e of an A-fragment tile
// (pieces in storage order).
__device__ __forceinline__ void frag_piece(int e, int& r, int& k) {
    const int blk = e >> 6, l = e & 63;
    r = 16 * (blk >> 2) + (l & 15);
    k = 32 * (blk & 3) + 8 * (l >> 4);
}

// ------------------------------------------------------------------ K1: intra-chunk
// 8 waves; LDS < 80 KiB so that two workgroups share a CU.
//   sA  fp16 [128][LD16]: k^ [tok][dk] (Gram) -> k^T [dk][tok] (swizzled, copied out)
//                         -> (k^ beta e^gcum)^T -> (v beta)^T [col][tok] (swizzled)
//   sL  fp16 [128][LD16]: L (strictly lower); then T_bb = (I + L_bb)^-1 on the
//                         diagonal blocks and M_ba = -T_bb L_ba below them
//   sD  fp32 8 x [16][17]: the diagonal 16x16 blocks L_bb
// w and u solve (I + L) X = R for R = k^ beta e^gcum and R = v beta by
// forward substitution over 16-row blocks, one 16-column tile per wave:
// X_b = T_bb R_b + sum_{a<b} M_ba X_a.  The 16x16x16 MFMA's accumulator
// layout equals its B-operand layout, so each solved block feeds the later
// blocks' products straight from registers; no barrier is needed inside the
// substitution.  Operands are plain fp16 with fp32 accumulation.
// Load of a lane-uniform int that the running kernel never writes (the chunk
// map), through the scalar unit: it waits on the scalar counter only, not on
// the vector-memory counter that also tracks this workgroup's pending stores.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* ptr) {
    return *(const __attribute__((address_space(4))) int32_t*)(ptr);
}

// Raw (unconverted) loads, so that a prefetch does not wait for its data
// until the data is used.
template <typename ActT> struct Raw8;
template <> struct Raw8<uint16_t> { u32x4 d; };
template <> struct Raw8<_Float16> { u32x4 d; };
template <> struct Raw8<float> { f32x4 a, b; };
template <typename ActT> struct Raw4;
template <> struct Raw4<uint16_t> { u32x2 d; };
template <> struct Raw4<_Float16> { u32x2 d; };
template <> struct Raw4<float> { f32x4 d; };

__device__ __forceinline__ void raw_load(Raw8<uint16_t>& x, const uint16_t* p) { x.d = *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void raw_load(Raw8<float>& x, const float* p) {
    x.a = *reinterpret_cast<const f32x4*>(p);
    x.b = *reinterpret_cast<const f32x4*>(p + 4);
}
__device__ __forceinline__ void raw_load(Raw4<uint16_t>& x, const uint16_t* p) { x.d = *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void raw_load(Raw8<_Float16>& x, const _Float16* p) { x.d = *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void raw_load(Raw4<_Float16>& x, const _Float16* p) { x.d = *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void raw_cvt(const Raw8<_Float16>& x, float (&y)[8]) {
    const half8 h = __builtin_bit_cast(half8, x.d);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (float)h[i];
}
__device__ __forceinline__ void raw_cvt(const Raw4<_Float16>& x, float (&y)[4]) {
    const half4 h = __builtin_bit_cast(half4, x.d);
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = (float)h[i];
}
__device__ __forceinline__ void raw_load(Raw4<float>& x, const float* p) { x.d = *reinterpret_cast<const f32x4*>(p); }
// Non-temporal (streaming) forms, for rows read exactly once in the whole
// call (an item's v rows): they do not displace from the caches the rows that
// two value heads or several scan slices share.
__device__ __forceinline__ void raw_load_nt(Raw8<uint16_t>& x, const uint16_t* p) {
    x.d = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void raw_load_nt(Raw8<_Float16>& x, const _Float16* p) {
    x.d = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void raw_load_nt(Raw8<float>& x, const float* p) {
    x.a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    x.b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
}
__device__ __forceinline__ void raw_zero(Raw8<uint16_t>& x) { x.d = u32x4{0u, 0u, 0u, 0u}; }
__device__ __forceinline__ void raw_zero(Raw8<float>& x) { x.a = f32x4{0.f, 0.f, 0.f, 0.f}; x.b = x.a; }
__device__ __forceinline__ void raw_zero(Raw4<uint16_t>& x) { x.d = u32x2{0u, 0u}; }
__device__ __forceinline__ void raw_zero(Raw4<float>& x) { x.d = f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ void raw_cvt(const Raw8<uint16_t>& x, float (&y)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        y[2 * i] = __uint_as_float(x.d[i] << 16);
        y[2 * i + 1] = __uint_as_float(x.d[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void raw_cvt(const Raw8<float>& x, float (&y)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { y[i] = x.a[i]; y[4 + i] = x.b[i]; }
}
__device__ __forceinline__ void raw_cvt(const Raw4<uint16_t>& x, float (&y)[4]) {
    y[0] = __uint_as_float(x.d[0] << 16);
    y[1] = __uint_as_float(x.d[0] & 0xffff0000u);
    y[2] = __uint_as_float(x.d[1] << 16);
    y[3] = __uint_as_float(x.d[1] & 0xffff0000u);
}
__device__ __forceinline__ void raw_cvt(const Raw4<float>& x, float (&y)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = x.d[i];
}

// Raw inputs of one (chunk, value head) item, held in registers so that the
// next item's loads are in flight while the current item computes.
//   k: row 16*wave + lr, key dims 32*ks + 8*lq .. +7 (A-fragment layout)
//   g0/g1, b0/b1: gate and beta of rows 2*lane, 2*lane+1 (used by wave 0)
// Rows past the chunk's end are loaded from its last row (every lane issues
// the same loads on every path, which keeps the compiler's memory-counter
// waits exact) and replaced by zeros when converted.
// (v is first needed late in the item, so each item loads its own v rows
// during its first steps.)
template <typename ActT>
struct IntraStage {
    Raw8<ActT> k[4];
    float g0, g1;
    ActT b0, b1;
    int c, h, t0, r;
};

// Where item (chunk c, value head h) lies: its first token and valid rows.
struct ItemPlace {
    int c, h, t0, r;
};
__device__ __forceinline__ ItemPlace place_item(const PrefillDev& p, const int32_t* smap, int item) {
    ItemPlace at;
    at.c = item / p.Nv;
    at.h = item % p.Nv;
    if (p.map_in_intra) {
        chunk_from_map(smap, p.B, at.c, at.t0, at.r);
    } else {
        at.t0 = ld_uniform(&p.cmap[4 * at.c + 1]);
        at.r = ld_uniform(&p.cmap[4 * at.c + 2]);
    }
    return at;
}

template <typename ActT, int RULE>
__device__ __forceinline__ void intra_load(IntraStage<ActT>& st, const PrefillDev& p, const ItemPlace& at, int wave,
                                           int lane, int lr, int lq, int c4, int tg, int part = 3) {
    // part 1: k dims 0..63; part 2: k dims 64..127, g and beta; 3: all
    const int Nv = p.Nv, Nqk = p.Nqk;
    const int h = at.h, hq = h / (Nv / Nqk), t0 = at.t0, r = at.r;
    st.c = at.c; st.h = h; st.t0 = t0; st.r = r;
    const ActT* K = static_cast<const ActT*>(p.k);
    const ActT* BETA = static_cast<const ActT*>(p.beta);
    const int last = max(r - 1, 0);   // every mapped chunk has r >= 1
    const int row = min(16 * wave + lr, last);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        if (((part & 1) && ks < 2) || ((part & 2) && ks >= 2))
            raw_load(st.k[ks], K + ((size_t)(t0 + row) * Nqk + hq) * 128 + 32 * ks + 8 * lq);
    if (!(part & 2)) return;
    // only wave 0 uses the gates; the other waves issue the same loads at one
    // lane-uniform address (a single cache line each)
    const int i0 = wave == 0 ? min(2 * lane, last) : 0, i1 = wave == 0 ? min(2 * lane + 1, last) : 0;
    if constexpr (Rule<RULE>::gated) {
        st.g0 = p.g[(size_t)(t0 + i0) * Nv + h];
        st.g1 = p.g[(size_t)(t0 + i1) * Nv + h];
    } else {
        st.g0 = st.g1 = 0.f;
    }
    if constexpr (Rule<RULE>::delta) {
        st.b0 = BETA[(size_t)(t0 + i0) * Nv + h];
        st.b1 = BETA[(size_t)(t0 + i1) * Nv + h];
    } else {
        (void)BETA;
        st.b0 = st.b1 = ActT(0);
    }
}

struct IntraSmem {
    const int32_t* sMap;
    _Float16* sA;
    _Float16* sL;
    float* sD;
    float* sGc;
    float* sBeta;
    float* sBE;
};

// Four 16x16 accumulator tiles acc[ii] of w (rows 16 Jt + lr, columns
// 16 (4 hsel + ii) + 4 lq + e) into the tile's fragment order.  A 16-byte piece
// there holds 8 consecutive columns of one row, which two lanes 16 apart (lq,
// lq ^ 1) hold half each; v_permlane16_swap over a pair of tiles (2m, 2m + 1)
// gives the even-row lane tile 2m's whole piece and the odd-row lane tile
// 2m + 1's, so each lane writes one 16-byte piece per pair.
__device__ __forceinline__ void store_w_tiles(_Float16* dst, const f32x4 (&acc)[4], int Jt, int hsel, int lr,
                                              int lq) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const half4 a = to_h4(acc[2 * m]), b = to_h4(acc[2 * m + 1]);
        const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
        u32x4 piece;
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const auto r = __builtin_amdgcn_permlane16_swap(ua[d], ub[d], false, false);
            piece[d] = r[0];
            piece[2 + d] = r[1];
        }
        const int ii = 2 * m + (lq & 1);
        st_h8(dst + frag_off(16 * Jt + lr, 16 * (4 * hsel + ii) + 8 * (lq >> 1)), __builtin_bit_cast(half8, piece));
    }
}

// Column block j of T = (I + L)^-1 by forward substitution over 16-row
// blocks: X_jj = T_jj, X_bj = -T_bb sum_{j <= a < b} L_ba X_aj.  Each solved
// block at once adds its term to every later block's sum (right-looking), so
// the L reads and most products are off the chain that runs from one solved
// block to the next; each sum still adds its terms in ascending a.  T_bb (the
// inverted diagonal blocks, fp32, row stride 17) is in sD, L (fp16) in sL.
// xh[b] receives X_bj in the 16x16x16 MFMA's accumulator (= B operand) layout.
__device__ __forceinline__ void block_column_solve(const float* sD, const _Float16* sL, int j, int lr, int lq,
                                                   half4 (&xh)[8]) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[b] = zero;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        if (a < j) continue;
        f32x4 x;
        if (a == j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = sD[(16 * a + 4 * lq + e) * 17 + lr];
        } else {
            half4 ta;
#pragma unroll
            for (int e = 0; e < 4; ++e) ta[e] = (_Float16)sD[(16 * a + lr) * 17 + 4 * lq + e];
            x = mma16(ta, to_h4(-acc[a]), zero);
        }
        xh[a] = to_h4(x);
#pragma unroll
        for (int b = a + 1; b < 8; ++b) acc[b] = mma16(ld_h4(&sL[(16 * b + lr) * LD16 + 16 * a + 4 * lq]), xh[a], acc[b]);
    }
}

// Block forward substitution for one 16-column tile of X = (I + L)^-1 R.
// acc[b] enters as T_bb R_b (T_bb = (I + L_bb)^-1) in the 16x16x16 MFMA's
// accumulator layout; sL holds M_ba = -T_bb L_ba (fp16) for b > a, so that
// X_b = T_bb R_b + sum_{a<b} M_ba X_a.  Each solved block X_a is rounded to
// fp16 once, handed to store(a, X_a), and at once adds its term to every later
// block (right-looking): the accumulator layout equals the B-operand layout, so
// the chain from one solved block to the next is one conversion and one
// product, and the other products come off it.
template <typename Store>
__device__ __forceinline__ void block_substitution(f32x4 (&acc)[8], const _Float16* sL, int lr, int lq, Store&& store) {
#pragma unroll
    for (int a = 0; a < 8; ++a) {
        const half4 xa = to_h4(acc[a]);
#pragma unroll
        for (int b = a + 1; b < 8; ++b) acc[b] = mma16(ld_h4(&sL[(16 * b + lr) * LD16 + 16 * a + 4 * lq]), xa, acc[b]);
        store(a, xa);
    }
}

// Two transposed 16x16 blocks of w, token blocks a0 and a0 + 1 of column tile
// ct (a lane holds token 16 a + lr, columns 16 ct + 4 lq ..), into the tile's
// fragment order.  The two lanes 16 apart (lq, lq ^ 1) that hold the halves of
// a 16-byte piece swap them with v_permlane16_swap over the pair, so each lane
// writes one whole piece: block a0 + (lq & 1), columns 16 ct + 8 (lq >> 1) ..
__device__ __forceinline__ void store_w_pair(_Float16* dst, half4 x0, half4 x1, int a0, int ct, int lr, int lq) {
    const u32x2 ua = __builtin_bit_cast(u32x2, x0), ub = __builtin_bit_cast(u32x2, x1);
    u32x4 piece;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const auto r = __builtin_amdgcn_permlane16_swap(ua[d], ub[d], false, false);
        piece[d] = r[0];
        piece[2 + d] = r[1];
    }
    const int a = a0 + (lq & 1);
    st_h8(dst + frag_off(16 * a + lr, 16 * ct + 8 * (lq >> 1)), __builtin_bit_cast(half8, piece));
}

template <typename ActT, int RULE>
__device__ __forceinline__ void intra_item(IntraStage<ActT>& st, int next, const PrefillDev& p, const IntraSmem& sm,
                                           int tid_in) {
    // The item loop would otherwise hoist every per-lane offset derived from
    // the thread index out of the loop and keep them all live; an opaque copy
    // of the index makes them per-item values instead.
    int tid = tid_in;
    asm volatile("" : "+v"(tid));
    _Float16* sA = sm.sA;
    _Float16* sL = sm.sL;
    float* sD = sm.sD;
    float* sGc = sm.sGc;
    float* sBeta = sm.sBeta;
    float* sBE = sm.sBE;
    const int Nv = p.Nv, Nqk = p.Nqk, G = Nv / Nqk;
    const int c = st.c, h = st.h, hq = h / G, r = st.r, t0 = st.t0;
    const int wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const size_t ch = (size_t)c * Nv + h;
    const size_t cq = (size_t)c * Nqk + hq;
    const bool writes_keys = (h % G) == 0;   // one value head per group stores k^T
    const int c4 = tid & 31, tg = tid >> 5;   // transposing layout: tokens 8*tg.., columns 4*c4..

    // v rows of this item, first used in step 7, loaded in two halves at steps
    // 2 and 4 (the workgroups' loads then come spread over the item, not in one
    // burst with the next item's k).  Rows past the chunk's end re-read its last
    // row: they are multiplied by beta = 0 there.
    Raw8<ActT> vr[4];   // rows 4 tq + i, columns 8 c8 .. 8 c8 + 7
    auto load_v = [&](int i0) {
        const ActT* V = static_cast<const ActT*>(p.v);
        const int c8 = tid & 15, tq = tid >> 4;
#pragma unroll
        for (int i = i0 / 2; i < i0 / 2 + 2; ++i) {
            const int row = min(4 * tq + i, max(r - 1, 0));
            raw_load_nt(vr[i], V + ((size_t)(t0 + row) * Nv + h) * 128 + 8 * c8);
        }
    };
    // where the next item lies, looked up now: its loads go out in steps 5 and 6
    const ItemPlace nxt = place_item(p, sm.sMap, next);
    __syncthreads();   // the previous item is done with the shared buffers
    // ---- 1. gate cumulative sum and beta (wave 0); k rows normalised -> sA (row-major)
    if (wave == 0) {   // lane owns rows 2l, 2l+1
        const int i0 = 2 * lane, i1 = i0 + 1;
        const float g0 = i0 < r ? fmaxf(st.g0, -kLogDecayFloor) : 0.f;
        const float g1 = i1 < r ? fmaxf(st.g1, -kLogDecayFloor) : 0.f;
        // without the delta term beta is 1 for u = T v and 0 for w (below)
        const float b0 = i0 < r ? (Rule<RULE>::delta ? load1(&st.b0) : 1.f) : 0.f;
        const float b1 = i1 < r ? (Rule<RULE>::delta ? load1(&st.b1) : 1.f) : 0.f;
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
        sBE[i0] = Rule<RULE>::delta ? b0 * __expf(gc0) : 0.f;
        sBE[i1] = Rule<RULE>::delta ? b1 * __expf(gc1) : 0.f;
        p.gc[ch * 128 + i0] = gc0;
        p.gc[ch * 128 + i1] = gc1;
    }
    {
        const int row = 16 * wave + lr;
        float kf[4][8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            raw_cvt(st.k[ks], kf[ks]);
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[ks][e] = row < r ? kf[ks][e] : 0.f;
        }
        float ssq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) ssq = fmaf(kf[ks][e], kf[ks][e], ssq);
        ssq += __shfl_xor(ssq, 16);
        ssq += __shfl_xor(ssq, 32);
        const float rinv = 1.f / sqrtf(ssq + kNormEps);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float kx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) kx[e] = kf[ks][e] * rinv;
            const half8 kh = to_h8(kx);
            st_h8(&sA[row * LD16 + 32 * ks + 8 * lq], kh);
        }
    }
    __syncthreads();

    load_v(0);
    // ---- 2. Gram k^ k^T on the lower 16-tiles -> L (fp16 in sL, diagonal
    //         blocks also fp32 in sD); k^ read back transposed (8 tokens x
    //         4 dk per thread).
    //         Waves take whole tile rows so that a row's A fragments load
    //         once: rows pair up as (pp, 7 - pp); wave 2 pp takes row pp and
    //         the first 4 - pp tiles of row 7 - pp, wave 2 pp + 1 the other
    //         four tiles of row 7 - pp (4 or 5 tiles per wave).  Row-major k^
    //         is already in the B-fragment layout of k^T.
    {
        // Each tile is computed transposed (A = rows j, B = rows i), so a
        // lane holds four consecutive columns 16 J + 4 lq .. of row
        // i = 16 I + lr: beta_i and g_cum_i are the lane's own, and the row
        // piece is one 8-byte store.
        auto gram_row = [&](int I, int J0, int J1) {
            half8 a[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) a[ks] = ld_h8(&sA[(16 * I + lr) * LD16 + 32 * ks + 8 * lq]);
            const int i = 16 * I + lr;
            const float bi = sBeta[i], gi = sGc[i];
            for (int J = J0; J < J1; ++J) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if constexpr (Rule<RULE>::delta) {
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        acc = mma(ld_h8(&sA[(16 * J + lr) * LD16 + 32 * ks + 8 * lq]), a[ks], acc);
                }
                const int j0 = 16 * J + 4 * lq;
                const f32x4 gj = *reinterpret_cast<const f32x4*>(&sGc[j0]);
                half4 o;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float Lij = (Rule<RULE>::delta && i > j0 + e) ? bi * acc[e] * __expf(gi - gj[e]) : 0.f;
                    o[e] = (_Float16)Lij;
                    if (I == J) sD[i * 17 + 4 * lq + e] = Lij;
                }
                st_h4(&sL[i * LD16 + j0], o);
            }
        };
        const int pp = wave >> 1;
        if (wave & 1) {
            gram_row(7 - pp, 4 - pp, 8 - pp);
        } else {
            gram_row(pp, 0, pp + 1);
            gram_row(7 - pp, 0, 4 - pp);
        }
    }
    half4 kt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kt[i] = ld_h4(&sA[(8 * tg + i) * LD16 + 4 * c4]);
    __syncthreads();

    // ---- 3. k^T into sA; inverses of the diagonal blocks T_bb = (I + L_bb)^-1
    //         (one column per lane, forward substitution in fp32), stored in
    //         fp16 over the diagonal blocks of sL
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        half8 col;
#pragma unroll
        for (int i = 0; i < 8; ++i) col[i] = kt[i][e];
        st_h8(&sA[sw(4 * c4 + e, 8 * tg)], col);
    }
    if (tid < 128) {
        const int bb = tid >> 4, j = tid & 15;
        const float* Lb = &sD[bb * 16 * 17];
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) acc = fmaf(-Lb[i * 17 + kk], t[kk], acc);
            t[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sL[(16 * bb + i) * LD16 + 16 * bb + j] = (_Float16)t[i];
    }
    __syncthreads();

    load_v(4);
    // ---- 4. unscaled k^T -> workspace (fragment order), and in place scaled
    //         to R = (k^ beta e^gcum)^T; M_ba = -T_bb L_ba over L_ba (b > a),
    //         28 blocks over the waves.  M_ba^T = L_ba^T T_bb^T is formed so
    //         that a lane holds four consecutive columns of one row of M_ba.
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int e_ = tid + 512 * n;
        int row, kc;
        frag_piece(e_, row, kc);
        _Float16* pk = &sA[sw(row, kc)];
        half8 x = ld_h8(pk);
        if (writes_keys) st_h8(p.khatT + cq * TILE + (size_t)e_ * 8, x);
        float be[8];
        lds_row8(&sBE[kc], be);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (_Float16)((float)x[e] * be[e]);
        st_h8(pk, x);
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const int n = wave + 8 * m;   // block (b, a), n = b (b - 1) / 2 + a
        if (n < 28) {
            const int b = 1 + (n >= 1) + (n >= 3) + (n >= 6) + (n >= 10) + (n >= 15) + (n >= 21);
            const int a = n - b * (b - 1) / 2;
            half4 lt;
#pragma unroll
            for (int e = 0; e < 4; ++e) lt[e] = sL[(16 * b + 4 * lq + e) * LD16 + 16 * a + lr];
            const f32x4 mt = mma16(lt, ld_h4(&sL[(16 * b + lr) * LD16 + 16 * b + 4 * lq]), zero);
            st_h4(&sL[(16 * b + lr) * LD16 + 16 * a + 4 * lq], to_h4(-mt));
        }
    }
    __syncthreads();

    // ---- 5. w = (I + L)^-1 R by block forward substitution, one 16-column
    //         tile ct = wave per wave: X_b = T_bb R_b + sum_{a<b} M_ba X_a.
    //         The next item's k, g and beta load into the stage in two parts,
    //         now and in step 6 (this item took its own in step 1); fp32
    //         inputs, twice the registers, load at the item's start
    if constexpr (sizeof(ActT) == 2) intra_load<ActT, RULE>(st, p, nxt, wave, lane, lr, lq, c4, tg, 1);
    const int ct = wave;
    f32x4 acc[8];
#pragma unroll
    for (int b = 0; b < 8; ++b)
        acc[b] = mma16(ld_h4(&sL[(16 * b + lr) * LD16 + 16 * b + 4 * lq]), ld_h4(&sA[sw(16 * ct + lr, 16 * b + 4 * lq)]),
                       zero);
    __syncthreads();   // R is read

    if constexpr (sizeof(ActT) == 2) intra_load<ActT, RULE>(st, p, nxt, wave, lane, lr, lq, c4, tg, 2);
    // ---- 6. (v beta)^T [col][tok] into sA; the substitution for w.  Each
    //         solved block goes to the store transposed (a product with I
    //         turns its accumulator layout, four tokens of one column, into
    //         four columns of one token) and pairs of blocks are stored as
    //         16-byte fragment pieces.
    {
        const int c8 = tid & 15, tq = tid >> 4;
        float vf[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) raw_cvt(vr[i], vf[i]);
        const f32x4 bt = *reinterpret_cast<const f32x4*>(&sBeta[4 * tq]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            half4 col;
#pragma unroll
            for (int i = 0; i < 4; ++i) col[i] = (_Float16)(vf[i][e] * bt[i]);
            st_h4(&sA[sw(8 * c8 + e, 4 * tq)], col);
        }
    }
    {
        half4 eye;
#pragma unroll
        for (int e = 0; e < 4; ++e) eye[e] = (_Float16)(4 * lq + e == lr ? 1.f : 0.f);
        half4 prev;
        block_substitution(acc, sL, lr, lq, [&](int a, half4 xa) {
            const half4 xt = to_h4(mma16(xa, eye, zero));   // token 16 a + lr, columns 16 ct + 4 lq ..
            if (a & 1) store_w_pair(p.w + ch * TILE, prev, xt, a - 1, ct, lr, lq);
            else prev = xt;
        });
    }
    __syncthreads();   // v beta is in sA

    // ---- 7. the same substitution for u = (I + L)^-1 (v beta), stored in
    //         C-fragment order straight from the accumulator layout
#pragma unroll
    for (int b = 0; b < 8; ++b)
        acc[b] = mma16(ld_h4(&sL[(16 * b + lr) * LD16 + 16 * b + 4 * lq]), ld_h4(&sA[sw(16 * ct + lr, 16 * b + 4 * lq)]),
                       zero);
    block_substitution(acc, sL, lr, lq, [&](int a, half4 xa) {
        st_h4(p.u + ch * TILE + cfrag_off(16 * a + 4 * lq, 16 * ct + lr), xa);
    });
}

// Persistent: each workgroup walks items blockIdx.x, blockIdx.x + gridDim.x, ...
// (item = chunk * Nv + value head), the next item's inputs loading while this
// one computes.
template <typename ActT, int RULE>
__global__ __launch_bounds__(512, 4) void intra_kernel(PrefillDev p) {
    __shared__ __align__(16) _Float16 sA[128 * LD16];
    __shared__ __align__(16) _Float16 sL[128 * LD16];
    __shared__ float sD[8 * 16 * 17];
    __shared__ __align__(16) float sGc[128];
    __shared__ __align__(16) float sBeta[128];
    __shared__ __align__(16) float sBE[128];
    __shared__ int32_t sMap[kMapInts];
    const IntraSmem sm{sMap, sA, sL, sD, sGc, sBeta, sBE};
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int c4 = tid & 31, tg = tid >> 5;
    int n_items;
    if (p.map_in_intra) {
        build_chunk_map(p, sMap, tid);
        n_items = __builtin_amdgcn_readfirstlane(sMap[p.B]) * p.Nv;
    } else {
        n_items = ld_uniform(&p.meta[p.B]) * p.Nv;
    }
    const int stride = gridDim.x;   // a multiple of 8 G
    int it = group_slot(blockIdx.x, p.Nv / p.Nqk);
    if (it >= n_items) return;
    // Wave priority per item.  Two workgroups share each CU, and the CU issues
    // the older one's ready waves first, so with equal priorities the second
    // workgroup dispatched to a CU (ids from gridDim.x / 2) ran its items about
    // a quarter slower and set the kernel's end.  That workgroup takes the
    // higher priority on every other item; a workgroup that has one item more
    // than the least loaded ones (the last, partial round) takes the highest on
    // all of its items.  Priorities change only the order of issue.
    const bool second = blockIdx.x >= stride / 2;
    const bool extra = (n_items - 1 - it) / stride + 1 > n_items / stride;
    int k_item = 0;
    auto item_priority = [&]() {
        if (extra) __builtin_amdgcn_s_setprio(2);
        else if (second && (k_item & 1) == 0) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        ++k_item;
    };
    // One register stage: the item loads the next one's k, g and beta into it
    // once it has used its own (after the last item they re-read the current
    // one, unused); with fp32 inputs each item loads its own at its start.
    IntraStage<ActT> st;
    if constexpr (sizeof(ActT) == 2) {
        // The first item is peeled off the loop, so that every entry into the
        // loop follows a whole item: the memory operations in flight at the
        // loop head are then the same on every path, and the compiler's
        // waits for the prefetched inputs stop at those loads instead of
        // also waiting for the previous item's stores.
        intra_load<ActT, RULE>(st, p, place_item(p, sMap, it), wave, lane, lr, lq, c4, tg);
        int nx = it + stride;
        item_priority();
        intra_item<ActT, RULE>(st, nx < n_items ? nx : it, p, sm, tid);
        while (nx < n_items) {
            it = nx;
            nx = it + stride;
            item_priority();
            intra_item<ActT, RULE>(st, nx < n_items ? nx : it, p, sm, tid);
        }
    } else {
        while (true) {
            intra_load<ActT, RULE>(st, p, place_item(p, sMap, it), wave, lane, lr, lq, c4, tg);
            const int nx = it + stride;
            item_priority();
            intra_item<ActT, RULE>(st, nx < n_items ? nx : it, p, sm, tid);
            if (nx >= n_items) break;
            it = nx;
        }
    }
}

// ------------------------------------------------------------------ K1 with a per-key gate
// Persistent workgroups of 8 waves, one per CU (LDS about 157 KiB), walking
// (chunk, value head) items.  With a per-key gate gk the decay from token j to
// token i >= j of state row d is exp(G_i[d] - G_j[d]), G the chunk-local
// inclusive prefix of g + gk[d] ("LinearAttention" page: per-key decay; the
// decode page's S <- S exp(g) exp(gk) at every token), so the decayed
// products q_i.k_j and k_i.k_j no longer factor through one scalar per
// token.  They are formed per pair of 16-token blocks (I, J):
//   J < I  through G at the token before block I, s = 16 I - 1:
//          exp(G_i - G_j) = exp(G_i - G_s) exp(G_s - G_j), both factors
//          <= 1, so the MFMA operands are scaled keys / queries (fp16);
//   J = I  through G at the block's middle row m = 16 I + 7: factors up to
//          exp(8 max|g + gk|); in fp16 when every |G_i - G_m| of the block
//          is within kDiagF16Range, in fp32 on the 16x16x4 fp32 MFMA when
//          within kDiagF32Range, and past that (a strong gate or a reset of
//          some keys) element by element, exp(G_i[d] - G_j[d]) <= 1 per
//          term, so nothing over- or underflows whatever the gates.
// The decay between blocks, exp(G_s(I) - G_e(J)), and the per-block factors
// come from running products of the block decays, not per element.
// The item stores k^T exp(G_last - G) (the scan's k^T, per value head),
// G_last (the chunk's decay of each state row), q^ exp(G) and the decayed
// scores P (the output kernel's two operands), and w, u as the intra kernel
// does, with w's scaling exp(g_cum) per token become exp(G[d]) per key.
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void ld_f8(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}
constexpr int LDG = 132;   // fp32 LDS row stride of G (elements): 528 B, 16-byte aligned rows

// Inputs an item holds in registers: the next item's k, q (this wave's rows),
// g and beta, and the item's own v; every thread issues the same loads on
// every pass (past the last item they re-read the current one, unused).
template <typename ActT>
struct GkStage {
    Raw8<ActT> k[4], q[4];   // rows 16 wave + lr, keys 32 ks + 8 lq ..
    Raw4<ActT> v[8];         // rows 8 tg + i, columns 4 c4 ..
    float g;                 // threads < 128: token tid
    ActT b;
    int c, h, t0, r;         // the item k, q, g, beta belong to
};

// The place of item `item` (chunk * Nv + value head) in the token stream
template <typename ActT>
__device__ __forceinline__ void gk_place(GkStage<ActT>& st, const ItemPlace& at) {
    st.c = at.c;
    st.h = at.h;
    st.t0 = at.t0;
    st.r = at.r;
}

// Parts of the item in st's place: what = 0: k, 1: q, 2: g and beta (issued
// at different points of the previous item, so that the loads of all
// workgroups do not come at once)
template <typename ActT, int RULE>
__device__ __forceinline__ void gk_load_in(GkStage<ActT>& st, const PrefillDev& p, int what, int tid) {
    const int Nv = p.Nv, Nqk = p.Nqk, hq = st.h / (Nv / Nqk), t0 = st.t0, last = max(st.r - 1, 0);
    const int wave = tid >> 6, lr = tid & 15, lq = (tid >> 4) & 3;
    const int lrow = min(16 * wave + lr, last);
    if (what < 2) {
        const ActT* X = static_cast<const ActT*>(what ? p.q : p.k);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            raw_load(what ? st.q[ks] : st.k[ks], X + ((size_t)(t0 + lrow) * Nqk + hq) * 128 + 32 * ks + 8 * lq);
    } else {
        const int tt = t0 + min(tid & 127, last);
        st.g = p.g[(size_t)tt * Nv + st.h];
        if constexpr (Rule<RULE>::delta) st.b = static_cast<const ActT*>(p.beta)[(size_t)tt * Nv + st.h];
        else st.b = ActT(0);
    }
}

// Rows 8 tg + 4 hv .. + 3 of v of the item at (t0, h, r)
template <typename ActT>
__device__ __forceinline__ void gk_load_v(GkStage<ActT>& st, const PrefillDev& p, int t0, int h, int r, int hv,
                                          int tid) {
    const int last = max(r - 1, 0), c4 = tid & 31, tg = tid >> 5;
    const ActT* V = static_cast<const ActT*>(p.v);
#pragma unroll
    for (int i = 4 * hv; i < 4 * hv + 4; ++i)
        raw_load(st.v[i], V + ((size_t)(t0 + min(8 * tg + i, last)) * p.Nv + h) * 128 + 4 * c4);
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16 B per lane from src straight into LDS at dst + 16 lane (dst uniform over
// the wave).  Written out so that the compiler, which would otherwise wait for
// it at the next access to the same shared array, leaves it in flight: the
// caller makes the data visible (s_waitcnt vmcnt(0), then a barrier) and
// touches the destination neither before that nor while it loads.  It has
// no register result.
// (M0 is set here and used by nothing else in this file.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_load16(const float* src, float* dst) {
    const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)dst);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

// The gate tile waits in G's region, unpadded [tok][128] fp32: tokens 0..63
// from float kGateHi on (behind KB, which takes the first 128 LD16 halves'
// rows), tokens 64..127 from 0 (free once KB is done).
constexpr int kGateHi = 128 * LD16 / 2;
// Largest |G_i - G_m| (G: the chunk-local log decay, m: a 16-token block's
// middle row) for which the block's diagonal tiles are taken in fp16: the
// scaled operands then stay within e^6, and a subnormal one errs by at most
// e^6 2^-25 in a product.
constexpr float kDiagF16Range = 6.f;
// Largest |G_i - G_m| for which the block's diagonal tiles are taken on the
// fp32 MFMA: both factors exp(+-(G_i - G_m)) then stay normal fp32 numbers
// (e^60 = 1.1e26); wider blocks are formed element by element.
constexpr float kDiagF32Range = 60.f;
static_assert(kGateHi + 64 * 128 <= 128 * LDG, "gate staging fits G's region");

// Quarter q4 of the gate tile of the item at (t0, h, r) (tokens 32 q4 ..
// 32 q4 + 31) straight from memory into LDS (rows past the end re-read the
// last row; the scan masks them): each wave 2 loads of two rows (1 KiB,
// lane l -> bytes 16 l .. 16 l + 15 of the destination).
__device__ __forceinline__ void gk_gate_dma(const PrefillDev& p, int t0, int h, int r, float* sG, int q4, int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, last = max(r - 1, 0);
    float* dst = sG + (q4 < 2 ? kGateHi + 32 * q4 * 128 : (32 * q4 - 64) * 128);
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int wi = 2 * wave + n, t = 32 * q4 + 2 * wi + (lane >> 5);
        const float* src = p.gk + ((size_t)(t0 + min(t, last)) * p.Nv + h) * 128 + 4 * (lane & 31);
        lds_load16(src, dst + wi * 256);
    }
}

// Thread indices taken afresh from a laundered copy of the thread id, so that
// the compiler recomputes a step's index arithmetic instead of keeping it
// live (and spilling it) from earlier steps.
#define GK_IDS()                                                                    \
    int tid = tid_in;                                                               \
    asm volatile("" : "+v"(tid));                                                   \
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;     \
    const int lr = lane & 15, lq = lane >> 4, c4 = tid & 31, tg = tid >> 5;         \
    (void)wave; (void)lr; (void)lq; (void)c4; (void)tg

template <typename ActT, int RULE>
__device__ __forceinline__ void gk_item(GkStage<ActT>& st, int next, const PrefillDev& p, float* sG, _Float16* sK,
                                        _Float16* sQL, float* sD, float* sEs, float* sTail, _Float16* sC, float* sGt,
                                        float* sBeta, float* sBw, int* sWide, const int32_t* sMap, int tid_in) {
    int tid = tid_in;
    asm volatile("" : "+v"(tid));
    constexpr bool kDelta = Rule<RULE>::delta;
    const int Nv = p.Nv;
    const int c = st.c, h = st.h, t0 = st.t0, r = st.r;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int c4 = tid & 31, tg = tid >> 5;
    const size_t ch = (size_t)c * Nv + h;
    _Float16* sKB = reinterpret_cast<_Float16*>(sG);   // KB takes G's place once G is done

    __syncthreads();   // the previous item is done with the shared buffers, the gate tile is in
    // ---- 0. g and beta per token; k^ (zero past the end) and q^ (scaled) of
    //         this wave's rows, row-major
    if (tid < 128) {
        const bool ok = tid < r;
        const float b = kDelta ? load1(&st.b) : 1.f;
        sGt[tid] = ok ? st.g : 0.f;
        sBeta[tid] = ok ? b : 0.f;                 // u = T (v beta)
        sBw[tid] = ok && kDelta ? b : 0.f;         // w = T (k^ beta exp(G))
    }
    {
        const int row = 16 * wave + lr;
        float kf[4][8], qf[4][8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            raw_cvt(st.k[ks], kf[ks]);
            raw_cvt(st.q[ks], qf[ks]);
        }
        float ksq = 0.f, qsq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                ksq = fmaf(kf[ks][e], kf[ks][e], ksq);
                qsq = fmaf(qf[ks][e], qf[ks][e], qsq);
            }
        ksq += __shfl_xor(ksq, 16);
        ksq += __shfl_xor(ksq, 32);
        qsq += __shfl_xor(qsq, 16);
        qsq += __shfl_xor(qsq, 32);
        const float kinv = row < r ? 1.f / sqrtf(ksq + kNormEps) : 0.f;
        const float qinv = p.scale / sqrtf(qsq + kNormEps);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float a[8], b[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { a[e] = kf[ks][e] * kinv; b[e] = qf[ks][e] * qinv; }
            st_h8(&sK[row * LD16 + 32 * ks + 8 * lq], to_h8(a));
            st_h8(&sQL[row * LD16 + 32 * ks + 8 * lq], to_h8(b));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's gate tile loads are in LDS
    __syncthreads();

    // ---- 1. G: inclusive prefix over tokens of g + gk[d], per key d (zero past
    //         the end); each thread scans 32 tokens of one key in registers,
    //         then the quarters are joined through sD and G overwrites the
    //         staged gate tile
    {
        const int d = tid & 127, qt = __builtin_amdgcn_readfirstlane(tid >> 7);
        const float* stg = sG + (qt < 2 ? kGateHi + 32 * qt * 128 : (32 * qt - 64) * 128) + d;
        float x[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = fmaxf(stg[i * 128] + sGt[32 * qt + i], -kLogDecayFloor);
        if (32 * qt + 31 >= r) {   // the chunk ends in this quarter
#pragma unroll
            for (int i = 0; i < 32; ++i) x[i] = 32 * qt + i < r ? x[i] : 0.f;
        }
#pragma unroll
        for (int i = 1; i < 32; ++i) x[i] += x[i - 1];
        sD[qt * 128 + d] = x[31];
        // blocks 2 qt, 2 qt + 1: is every |G_i - G_m| (m: the block's middle
        // row) within kDiagF16Range (tier 0), within kDiagF32Range (tier 1)
        // or neither (tier 2), for this wave's 64 keys?
        bool wide0 = false, wide1 = false, huge0 = false, huge1 = false;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float a0 = fabsf(x[i] - x[7]), a1 = fabsf(x[16 + i] - x[23]);
            wide0 |= !(a0 <= kDiagF16Range);
            wide1 |= !(a1 <= kDiagF16Range);
            huge0 |= !(a0 <= kDiagF32Range);
            huge1 |= !(a1 <= kDiagF32Range);
        }
        const bool w0 = __ballot(wide0) != 0, w1 = __ballot(wide1) != 0;
        const bool h0 = __ballot(huge0) != 0, h1 = __ballot(huge1) != 0;
        if ((tid & 63) == 0) {
            sWide[(2 * qt) * 2 + (d >> 6)] = h0 ? 2 : w0 ? 1 : 0;
            sWide[(2 * qt + 1) * 2 + (d >> 6)] = h1 ? 2 : w1 ? 1 : 0;
        }
        __syncthreads();
        float off = 0.f;
#pragma unroll
        for (int j = 0; j < 3; ++j) off += j < qt ? sD[j * 128 + d] : 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) sG[(32 * qt + i) * LDG + d] = x[i] + off;
    }
    __syncthreads();

    // ---- 2. with G at hand: per key d, from the block ends G_e[K] = G_{16K+15}
    //         and the block decays D[K] = exp(G_e[K] - G_e[K-1]), by running
    //         products: exp(G_s) of each block (sEs; s: the token before the
    //         block), exp(G_last - G_e) (sTail) and the decay between blocks
    //         J + 1 < I, c = exp(G_s(I) - G_e(J)) (sC, fp16: it only scales
    //         fp16 products); G_last -> workspace.  Then the diagonal blocks of
    //         P and L in fp32, and the scaled copies KA = k^ exp(G - G_s),
    //         KB = k^ exp(G_e - G), QA = q^ exp(G - G_s), with q^ exp(G) =
    //         QA exp(G_s) -> workspace
    if (tid < 128) {
        const int d = tid;
        float ge[8], D[8];
#pragma unroll
        for (int K = 0; K < 8; ++K) ge[K] = sG[(16 * K + 15) * LDG + d];
        p.gc[ch * 128 + d] = ge[7];
#pragma unroll
        for (int K = 1; K < 8; ++K) D[K] = __expf(ge[K] - ge[K - 1]);
        float es = 1.f, tl = 1.f;
        sEs[d] = 1.f;
#pragma unroll
        for (int I = 1; I < 8; ++I) {
            es = I == 1 ? __expf(ge[0]) : es * D[I - 1];
            sEs[I * 128 + d] = es;
        }
        sTail[7 * 128 + d] = 1.f;
#pragma unroll
        for (int J = 6; J >= 0; --J) {
            tl *= D[J + 1];
            sTail[J * 128 + d] = tl;
        }
#pragma unroll
        for (int J = 0; J < 6; ++J) {
            float cc = 1.f;
#pragma unroll
            for (int I = J + 2; I < 8; ++I) {
                cc *= D[I - 1];
                sC[((I - 2) * (I - 1) / 2 + J) * 128 + d] = (_Float16)cc;
            }
        }
    }
    // diagonal block Id of this wave (rows pair up as (pp, 7 - pp)), P and L
    // together through the block's middle row m: lane (lr, lq) supplies keys
    // d = 32 lq + 8 c8 + e of row 16 Id + lr to both operands, scaled by
    // exp(+-(G_row - G_m)).  In fp16 when every |G_row - G_m| of the block is
    // within kDiagF16Range (operands at most e^6, as precise as the other
    // tiles), in fp32 when within kDiagF32Range, else element by element.
    const int pp = wave >> 1;
    const int Id = (wave & 1) ? 7 - pp : pp;
    f32x4 pdiag = {0.f, 0.f, 0.f, 0.f}, ldiag = {0.f, 0.f, 0.f, 0.f};
    {
        const int rw = 16 * Id + lr, m = 16 * Id + 7;
        const int tier = __builtin_amdgcn_readfirstlane(max(sWide[2 * Id], sWide[2 * Id + 1]));
        if (tier == 0) {
#pragma unroll
            for (int c8 = 0; c8 < 4; ++c8) {
                const int d0 = 32 * lq + 8 * c8;
                const half8 kx = ld_h8(&sK[rw * LD16 + d0]), qx = ld_h8(&sQL[rw * LD16 + d0]);
                float gr[8], gm[8], kd[8], qu[8], ku[8];
                ld_f8(&sG[rw * LDG + d0], gr);
                ld_f8(&sG[m * LDG + d0], gm);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float up = __expf(gr[e] - gm[e]), dn = __expf(gm[e] - gr[e]);
                    kd[e] = (float)kx[e] * dn;
                    qu[e] = (float)qx[e] * up;
                    ku[e] = (float)kx[e] * up;
                }
                const half8 kdh = to_h8(kd);
                pdiag = mma(kdh, to_h8(qu), pdiag);                      // C[j][i] = P[i][j]
                if constexpr (kDelta) ldiag = mma(kdh, to_h8(ku), ldiag);   // C[j][i] = L[i][j]
            }
        } else if (tier == 1) {
#pragma unroll
            for (int c8 = 0; c8 < 4; ++c8) {
                const int d0 = 32 * lq + 8 * c8;
                const half8 kx = ld_h8(&sK[rw * LD16 + d0]), qx = ld_h8(&sQL[rw * LD16 + d0]);
                float gr[8], gm[8];
                ld_f8(&sG[rw * LDG + d0], gr);
                ld_f8(&sG[m * LDG + d0], gm);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float up = __expf(gr[e] - gm[e]), dn = __expf(gm[e] - gr[e]);
                    const float kd = (float)kx[e] * dn;
                    pdiag = mma_f32(kd, (float)qx[e] * up, pdiag);   // C[j][i] = P[i][j]
                    if constexpr (kDelta) ldiag = mma_f32(kd, (float)kx[e] * up, ldiag);   // C[j][i] = L[i][j]
                }
            }
        } else {
            // element by element: lane (lr, lq) forms P[i][j] and L[i][j] for
            // i = 16 Id + lr and j = 16 Id + 4 lq + e, the entries its
            // accumulators hold in the MFMA tiers, as sum_d q^_i[d] k^_j[d]
            // exp(G_i[d] - G_j[d]) (and k^_i for L); only j <= i are used, and
            // there each exponent is <= 0 (it is clamped to 0, so the
            // unused entries stay finite too)
            const int i = rw;
            for (int d0 = 0; d0 < 128; d0 += 8) {
                const half8 qi = ld_h8(&sQL[i * LD16 + d0]), ki = ld_h8(&sK[i * LD16 + d0]);
                float gi[8];
                ld_f8(&sG[i * LDG + d0], gi);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * Id + 4 * lq + e;
                    if (j > i) continue;
                    const half8 kj = ld_h8(&sK[j * LD16 + d0]);
                    float gj[8];
                    ld_f8(&sG[j * LDG + d0], gj);
#pragma unroll
                    for (int x = 0; x < 8; ++x) {
                        const float kf = (float)kj[x] * __expf(fminf(gi[x] - gj[x], 0.f));
                        pdiag[e] = fmaf((float)qi[x], kf, pdiag[e]);
                        if constexpr (kDelta) ldiag[e] = fmaf((float)ki[x], kf, ldiag[e]);
                    }
                }
            }
        }
    }
    __syncthreads();   // the diagonal tiles are done with the plain k^, q^
    half8 kb[4];
    {
        // each thread rescales its own pieces in place: rows 4 rg .. 4 rg + 3
        // (one block I), keys d0 .. d0 + 7
        const int d0 = 8 * (tid & 15), rg = tid >> 4, I = rg >> 2;
        float gs[8], ge[8], es[8];
        ld_f8(&sG[(16 * I + 15) * LDG + d0], ge);
        ld_f8(&sEs[I * 128 + d0], es);
        if (I > 0) ld_f8(&sG[(16 * I - 1) * LDG + d0], gs);
        else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gs[e] = 0.f;
        }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int t = 4 * rg + n;
        const half8 kx = ld_h8(&sK[t * LD16 + d0]), qx = ld_h8(&sQL[t * LD16 + d0]);
        float gt[8];
        ld_f8(&sG[t * LDG + d0], gt);
        float a[8], b[8], q8[8], qt8[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float fs = __expf(gt[e] - gs[e]);
            a[e] = (float)kx[e] * fs;
            q8[e] = (float)qx[e] * fs;
            qt8[e] = q8[e] * es[e];
            b[e] = (float)kx[e] * __expf(ge[e] - gt[e]);
        }
        st_h8(&sK[t * LD16 + d0], to_h8(a));
        st_h8(&sQL[t * LD16 + d0], to_h8(q8));
        st_h8(p.qt + ch * TILE + frag_off(t, d0), to_h8(qt8));
        kb[n] = to_h8(b);
    }
    }
    __syncthreads();   // G is done: KB takes its place, the next gate tile's first half goes behind it
    gk_place<ActT>(st, place_item(p, sMap, next));
    gk_gate_dma(p, st.t0, st.h, st.r, sG, 0, tid);
#pragma unroll
    for (int n = 0; n < 4; ++n) st_h8(&sKB[(4 * (tid >> 4) + n) * LD16 + 8 * (tid & 15)], kb[n]);
    __syncthreads();

    gk_load_in<ActT, RULE>(st, p, 0, tid);   // the next item's k
    // ---- 3. off-diagonal blocks J < I of P and L together: with KBc = KB_J c[I][J]
    //         (c = 1 when J = I - 1), P^T tile C[j][i] = sum_d KBc[j][d] QA[i][d]
    //         -> workspace; L^T tile C[j][i] = sum_d KBc[j][d] KA[i][d] (a lane
    //         then holds 4 consecutive columns of a row of L), kept in
    //         registers until QA is done
    const int J0A = (wave & 1) ? 4 - pp : 0, nA = Id - J0A;   // row Id: tiles J0A .. Id - 1
    const int rowB = 7 - pp, nT = nA + ((wave & 1) ? 0 : 4 - pp);   // even waves: row 7 - pp, tiles 0 ..
    f32x4 lacc[4];
    half8 qa[4], ka[4];   // QA and KA fragments of the current tile row, loaded once per row
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        lacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tt < nT) {
            const int I = tt < nA ? Id : rowB, J = tt < nA ? J0A + tt : tt - nA;
            if (tt == 0 || tt == nA) {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    qa[ks] = ld_h8(&sQL[(16 * I + lr) * LD16 + 32 * ks + 8 * lq]);
                    if constexpr (kDelta) ka[ks] = ld_h8(&sK[(16 * I + lr) * LD16 + 32 * ks + 8 * lq]);
                }
            }
            const _Float16* cIJ = &sC[((I - 2) * (I - 1) / 2 + J) * 128];
            f32x4 pacc = {0.f, 0.f, 0.f, 0.f}, la = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int d0 = 32 * ks + 8 * lq;
                half8 kb = ld_h8(&sKB[(16 * J + lr) * LD16 + d0]);
                if (J + 1 < I) kb = kb * ld_h8(&cIJ[d0]);
                pacc = mma(kb, qa[ks], pacc);
                if constexpr (kDelta) la = mma(kb, ka[ks], la);
            }
            st_h4(p.pm + ch * TILE + frag_off(16 * I + lr, 16 * J + 4 * lq), to_h4(pacc));
            lacc[tt] = la;
        }
    }
    {
        half4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (_Float16)(4 * lq + e <= lr ? pdiag[e] : 0.f);
        st_h4(p.pm + ch * TILE + frag_off(16 * Id + lr, 16 * Id + 4 * lq), o4);
        if ((Id & 1) == 0)   // the next block's columns, read by the output kernel's last k-step
            st_h4(p.pm + ch * TILE + frag_off(16 * Id + lr, 16 * (Id + 1) + 4 * lq), half4{0, 0, 0, 0});
    }
    __syncthreads();   // QA is done: sQL becomes L
    gk_gate_dma(p, st.t0, st.h, st.r, sG, 1, tid);

    // ---- 4. L = strictlower(beta_i sum_d k^_i k^_j exp(G_i - G_j)) -> sL (fp16,
    //         zeros above the block diagonal), diagonal blocks also fp32 in sD
    _Float16* sL = sQL;
    auto l_store = [&](int I, int J, const f32x4& acc) {   // acc[e] = L[16 I + lr][16 J + 4 lq + e]
        const int i = 16 * I + lr, j0 = 16 * J + 4 * lq;
        const float bi = sBw[i];
        half4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float Lij = (kDelta && i > j0 + e) ? bi * acc[e] : 0.f;
            o[e] = (_Float16)Lij;
            if (I == J) sD[i * 17 + 4 * lq + e] = Lij;
        }
        st_h4(&sL[i * LD16 + j0], o);
    };
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
        if (tt < nT) l_store(tt < nA ? Id : rowB, tt < nA ? J0A + tt : tt - nA, lacc[tt]);
    l_store(Id, Id, ldiag);
    {
        const int i = tid >> 2, I = i >> 4;
        const half8 z = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int gg = 2 * (I + 1) + (tid & 3); gg < 16; gg += 4) st_h8(&sL[i * LD16 + 8 * gg], z);
    }
    half4 kt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kt[i] = ld_h4(&sK[(8 * tg + i) * LD16 + 4 * c4]);
    __syncthreads();

    // ---- 5. KA^T into sK (swizzled); inverses of the diagonal blocks T_bb = (I + L_bb)^-1
    gk_load_in<ActT, RULE>(st, p, 1, tid);   // the next item's q
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        half8 col;
#pragma unroll
        for (int i = 0; i < 8; ++i) col[i] = kt[i][e];
        st_h8(&sK[sw(4 * c4 + e, 8 * tg)], col);
    }
    if (tid < 128) {
        const int bb = tid >> 4, j = tid & 15;
        float* Lb = &sD[bb * 16 * 17];
        float t[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) acc = fmaf(-Lb[i * 17 + kk], t[kk], acc);
            t[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Lb[i * 17 + j] = t[i];
    }
    __syncthreads();

    // ---- 6. k^T exp(G_last - G) = KB^T exp(G_last - G_e) -> workspace (fragment
    //         order, per value head: two adjacent pieces, keys dk and dk + 1,
    //         per thread and pass); column block j = wave of T by forward
    //         substitution
    gk_load_in<ActT, RULE>(st, p, 2, tid);   // the next item's g and beta
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int e_ = 2 * (tid + 512 * n);
        int dk, kc;
        frag_piece(e_, dk, kc);   // dk even; 8 tokens kc .. kc + 7, all in block kc / 16
        const float f0 = sTail[(kc >> 4) * 128 + dk], f1 = sTail[(kc >> 4) * 128 + dk + 1];
        float y0[8], y1[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const half2v x = *reinterpret_cast<const half2v*>(&sKB[(kc + e) * LD16 + dk]);
            y0[e] = (float)x[0] * f0;
            y1[e] = (float)x[1] * f1;
        }
        st_h8(p.khatT + ch * TILE + (size_t)e_ * 8, to_h8(y0));
        st_h8(p.khatT + ch * TILE + (size_t)e_ * 8 + 8, to_h8(y1));
    }
    half4 xh[8];
    block_column_solve(sD, sL, wave, lr, lq, xh);
    __syncthreads();   // KB is done
    gk_load_v<ActT>(st, p, t0, h, r, 0, tid);        // this item's v, used in step 9
    gk_gate_dma(p, st.t0, st.h, st.r, sG, 2, tid);   // the next gate tile's third quarter

    // ---- 7. T (fp16) into sL over L; sK scaled in place to (k^ beta exp(G))^T
    //         = KA^T beta exp(G_s) (8 tokens of one block per piece)
    {
    GK_IDS();
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        if (b < wave) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) sL[(16 * b + 4 * lq + e) * LD16 + 16 * wave + lr] = xh[b][e];
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int e_ = tid + 512 * n, dk = e_ >> 4, gg = e_ & 15, I = gg >> 1;
        _Float16* pk = &sK[sw(dk, 8 * gg)];
        half8 x = ld_h8(pk);
        const float f = sEs[I * 128 + dk];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (_Float16)((float)x[e] * sBw[8 * gg + e] * f);
        st_h8(pk, x);
    }
    }
    __syncthreads();

    // ---- 8. w^T = (k^ beta exp(G))^T T^T -> w [tok][dk], fragment order
    {
    GK_IDS();
    gk_load_v<ActT>(st, p, t0, h, r, 1, tid);
    const int pr = wave & 3, hsel = wave >> 2;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const int Jt = which ? 7 - pr : pr;
        f32x4 acc[4];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[ii] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks <= Jt / 2; ++ks) {
            const half8 b = ld_h8(&sL[(16 * Jt + lr) * LD16 + 32 * ks + 8 * lq]);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                acc[ii] = mma(ld_h8(&sK[sw(16 * (4 * hsel + ii) + lr, 32 * ks + 8 * lq)]), b, acc[ii]);
        }
        store_w_tiles(p.w + ch * TILE, acc, Jt, hsel, lr, lq);
    }
    }
    __syncthreads();

    // ---- 9. (v beta)^T [col][tok] into sK
    {
        GK_IDS();
        gk_gate_dma(p, st.t0, st.h, st.r, sG, 3, tid);   // the next gate tile's last quarter
        float vf[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) raw_cvt(st.v[i], vf[i]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            half8 col;
#pragma unroll
            for (int i = 0; i < 8; ++i) col[i] = (_Float16)(vf[i][e] * sBeta[8 * tg + i]);
            st_h8(&sK[sw(4 * c4 + e, 8 * tg)], col);
        }
    }
    __syncthreads();

    // ---- 10. u = T (v beta) -> u, fragment order
    {
    GK_IDS();
    const int pr = wave & 3, hsel = wave >> 2;
#pragma unroll
    for (int which = 0; which < 2; ++which) {
        const int I = which ? 7 - pr : pr;
        f32x4 acc[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int ks = 0; ks <= I / 2; ++ks) {
            const half8 a = ld_h8(&sL[(16 * I + lr) * LD16 + 32 * ks + 8 * lq]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                acc[jj] = mma(a, ld_h8(&sK[sw(16 * (4 * hsel + jj) + lr, 32 * ks + 8 * lq)]), acc[jj]);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            st_h4(p.u + ch * TILE + cfrag_off(16 * I + 4 * lq, 16 * (4 * hsel + jj) + lr), to_h4(acc[jj]));
    }
    }
}

// Persistent over items blockIdx.x, blockIdx.x + gridDim.x, ... (item =
// chunk * Nv + value head), one workgroup per CU.  Each item fetches the
// next one's inputs a little at a time over its own pass (the workgroups
// run in step, and a whole item's worth at once from all of them stalls on
// memory): the gate tile by quarters into LDS (the first half once G is
// done, the second once KB is done), k, q, g and beta into registers
// between; its own v in two halves before it is used.
template <typename ActT, int RULE>
__global__ __launch_bounds__(512) void intra_gk_kernel(PrefillDev p) {
    __shared__ __align__(16) float sG[128 * LDG];          // gate tile (staged) -> G [tok][dk]; then KB [tok][dk] fp16
    __shared__ __align__(16) _Float16 sK[128 * LD16];      // k^ -> KA -> KA^T (swizzled) -> (v beta)^T
    __shared__ __align__(16) _Float16 sQL[128 * LD16];     // q^ -> QA -> L / T
    __shared__ float sD[8 * 16 * 17];                      // (first: per-quarter prefix totals)
    __shared__ __align__(16) float sEs[8 * 128];           // exp(G) at the token before each block
    __shared__ __align__(16) float sTail[8 * 128];         // exp(G_last - G) at each block's last token
    __shared__ __align__(16) _Float16 sC[21 * 128];        // decay between blocks J + 1 < I
    __shared__ float sGt[128], sBeta[128], sBw[128];
    __shared__ int sWide[16];                              // per block and key half: tier of the diagonal tiles
    __shared__ int32_t sMap[kMapInts];                     // the chunk map, when built here
    const int tid = threadIdx.x;
    int n_items;
    if (p.map_in_intra) {
        build_chunk_map(p, sMap, tid);
        n_items = __builtin_amdgcn_readfirstlane(sMap[p.B]) * p.Nv;
    } else {
        n_items = ld_uniform(&p.meta[p.B]) * p.Nv;
    }
    const int stride = gridDim.x;   // a multiple of 8 G
    int it = group_slot(blockIdx.x, p.Nv / p.Nqk);
    if (it >= n_items) return;
    // Slot it holds item n_items - 1 - it: the last chunks first, so that the
    // first chunks, which the scan reads first, are the freshest in the
    // last-level cache when it starts (n_items is a multiple of G, so the G
    // value heads of a chunk keep consecutive slots).  Measured faster for
    // this scan, which also fetches q^ e^G and P each step; the intra kernel
    // without the gate keeps chunk order, which measured faster for its scan.
    GkStage<ActT> st;
    gk_place<ActT>(st, place_item(p, sMap, n_items - 1 - it));
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) gk_gate_dma(p, st.t0, st.h, st.r, sG, q4, tid);
    gk_load_in<ActT, RULE>(st, p, 0, tid);
    gk_load_in<ActT, RULE>(st, p, 1, tid);
    gk_load_in<ActT, RULE>(st, p, 2, tid);
    while (true) {
        const int nx = it + stride;
        gk_item<ActT, RULE>(st, n_items - 1 - (nx < n_items ? nx : it), p, sG, sK, sQL, sD, sEs, sTail, sC, sGt, sBeta,
                            sBw, sWide, sMap, tid);
        if (nx >= n_items) break;
        it = nx;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no load into LDS outlives the workgroup
}

// ------------------------------------------------------------------ K2: state scan
// 8 waves; wave wv owns rows 16*wv .. 16*wv+15 of w (tokens) and of k^T
// (key dims), i.e. one 16-row MFMA tile of each product, for DS columns.
// One chunk's operands for a scan wave:
template <int CT>
struct ScanOps {
    half8 aw[4], ak[4];
    half4 u4[CT];
    f32x4 gcr;
    float glast;
};

// Per-lane element offsets inside a chunk's tiles, fixed for the whole scan;
// each chunk only moves the (uniform) tile base pointers.
struct ScanLane {
    uint32_t a;    // fragment-order w / k^T: rows 16*wv + lr, columns 32*ks + 8*lq (+ 512 ks)
    uint32_t u;    // C-fragment-order u: tokens 16*wv + 4*lq, column col0 + lr (+ 256 ct)
    uint32_t g;    // g_cum: tokens 16*wv + 4*lq
};

// One chunk's operands, fetched in three parts: w (first needed by v_new),
// then u and the gates, then k^T (first needed by the state update).
template <int CT, int PART, bool GK = false>
__device__ __forceinline__ void scan_load_part(ScanOps<CT>& o, const PrefillDev& p, int c, int h, int hq,
                                               const ScanLane& ln) {
    const size_t ch = (size_t)c * p.Nv + h;
    if constexpr (PART == 0) {
        const _Float16* W = p.w + ch * TILE;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o.aw[ks] = ld_h8(W + ln.a + 512 * ks);
    } else if constexpr (PART == 1) {
        const _Float16* U = p.u + ch * TILE;
        const float* GC = p.gc + ch * 128;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o.u4[ct] = ld_h4(U + ln.u + 256 * ct);
        o.gcr = *reinterpret_cast<const f32x4*>(GC + ln.g);
        o.glast = GC[127];
    } else {
        const _Float16* KT = p.khatT + (GK ? (size_t)c * p.Nv + h : (size_t)c * p.Nqk + hq) * TILE;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o.ak[ks] = ld_h8(KT + ln.a + 512 * ks);
    }
}
template <int CT, bool GK>
__device__ __forceinline__ void scan_load(ScanOps<CT>& o, const PrefillDev& p, int c, int h, int hq,
                                          const ScanLane& ln) {
    scan_load_part<CT, 0, GK>(o, p, c, h, hq, ln);
    scan_load_part<CT, 1, GK>(o, p, c, h, hq, ln);
    scan_load_part<CT, 2, GK>(o, p, c, h, hq, ln);
}

// One chunk of the scan: record S_c and v_new for the output kernel, then
// S <- exp(g_last) S + k^T (v_new exp(g_last - g_cum)).  With LOAD, the
// operands of chunk cn are fetched into nx in three parts spread over the
// step (a burst of fetches would stall the waves' in-order issue behind the
// memory pipeline); scheduling barriers keep the parts where they are.
// MODE 1 (a segment's affine map, below) records nothing, and its u is
// scaled by umul (0 for the columns that carry M).  With the per-key gate
// (GK) the chunk's decays sit in k^T, and S decays row by row by
// exp(G_last[dk]) (the gate slot holds G_last of this lane's rows).
template <int DS, bool LOAD, int MODE = 0, bool GK = false>
__device__ __forceinline__ void scan_step(const ScanOps<DS / 16>& o, f32x4 (&S)[DS / 16], const PrefillDev& p,
                                          int c, int h, _Float16* sST, _Float16* sVn, int tid,
                                          int wv, int lr, int lq, int col0,
                                          ScanOps<DS / 16>& nx, int cn, int hq, const ScanLane& ln,
                                          float umul = 1.f) {
    constexpr int CT = DS / 16;
    const size_t ch = (size_t)c * p.Nv + h;
    if constexpr (LOAD) {
        scan_load_part<CT, 0, GK>(nx, p, cn, h, hq, ln);
        __builtin_amdgcn_sched_barrier(0);
    }
    // the state at the start of this chunk, for the output kernel; it is
    // stored below together with v_new (paired C-fragment order: straight
    // from the accumulators, one 16-byte piece per lane, 1 KiB per store)
    const int tok = 16 * wv + 4 * lq;
    half4 sc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) sc[ct] = to_h4(S[ct]);
    // v_new = u - w S for tokens 16*wv + 4*lq + e
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        f32x4 vp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) vp = mma(o.aw[ks], ld_h8(&sST[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), vp);
        f32x4 vn, vs;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vn[e] = (MODE == 0 ? (float)o.u4[ct][e] : umul * (float)o.u4[ct][e]) - vp[e];
            vs[e] = GK ? vn[e] : vn[e] * __expf(o.glast - o.gcr[e]);
        }
        const int col = 16 * ct + lr;
        if constexpr (MODE == 0) {
            const half4 vh = to_h4(vn);
            st_h8_nt(p.scvn + 2 * (ch * TILE + cfrag_off(tok, col0 + col)),
                     half8{sc[ct][0], sc[ct][1], sc[ct][2], sc[ct][3], vh[0], vh[1], vh[2], vh[3]});
        }
        st_h4(&sVn[col * LD16 + tok], to_h4(vs));
    }
    if constexpr (LOAD) {
        __builtin_amdgcn_sched_barrier(0);
        scan_load_part<CT, 1, GK>(nx, p, cn, h, hq, ln);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if constexpr (LOAD) {
        __builtin_amdgcn_sched_barrier(0);
        scan_load_part<CT, 2, GK>(nx, p, cn, h, hq, ln);
        __builtin_amdgcn_sched_barrier(0);
    }
    f32x4 dec;
    if constexpr (GK) {
#pragma unroll
        for (int e = 0; e < 4; ++e) dec[e] = __expf(o.gcr[e]);
    } else {
        const float d1 = __expf(o.glast);
        dec = f32x4{d1, d1, d1, d1};
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        f32x4 acc = S[ct] * dec;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mma(o.ak[ks], ld_h8(&sVn[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), acc);
        S[ct] = acc;
        st_h4(&sST[(16 * ct + lr) * LD16 + 16 * wv + 4 * lq], to_h4(acc));
    }
    __syncthreads();
}

// MODE 0: the scan proper.  Each (sequence, value head) stream -- or, with
//   two-level scanning, each segment of one -- carries its state from the
//   start state through its chunks, records S_c and v_new for the output
//   kernel, and the last segment writes the final state.
// MODE 1: the affine map of a segment that is not its sequence's last,
//   S_end = M S_start + B.  The scan runs over 256 columns: the first 128
//   start from I with u = 0 and end as M, the other 128 start from 0 with the
//   chunk's u and end as B; nothing is recorded.
template <int DS, int MODE, bool GK = false>
__global__ __launch_bounds__(512) void scan_kernel(PrefillDev p) {
    constexpr int NCOL = MODE == 0 ? 128 : 256;
    constexpr int NS = NCOL / DS, CT = DS / 16;
    __shared__ __align__(16) _Float16 sST[DS * LD16];   // S^T [col][dk] (fp16), current chunk's start state
    __shared__ __align__(16) _Float16 sVn[DS * LD16];   // scaled v_new^T [col][tok]

    // XCD-aware placement: the NS slices of a (sequence, segment, value head)
    // stream read the same w tiles, and the G value heads of one qk head read
    // the same k^T tiles, so all G*NS workgroups of a (sequence, segment, qk
    // head) group get ids the hardware dispatches to one XCD (id mod 8),
    // sharing its L2.
    const int Nv = p.Nv, Nqk = p.Nqk, G = Nv / Nqk, nseg = p.nseg;
    const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
    const int local = j % (G * NS), grp = (j / (G * NS)) * 8 + xcd;
    if (grp >= p.B * nseg * Nqk) return;
    const int hq = grp % Nqk, seg = (grp / Nqk) % nseg, b = grp / Nqk / nseg;
    const int slice = local % NS, h = hq * G + local / NS;
    const int stream = b * Nv + h;
    const int col0 = slice * DS;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;

    // this segment's chunks; a sequence has at least one segment (an empty
    // one passes its state through)
    const int cb = ld_uniform(&p.meta[b]), ce = ld_uniform(&p.meta[b + 1]);
    const int nsb = ce > cb ? (ce - cb + p.seg_len - 1) / p.seg_len : 1;
    if (MODE == 0 ? seg >= nsb : seg >= nsb - 1) return;
    const int c0 = cb + seg * p.seg_len;
    const int c1 = (int)min<int64_t>(ce, (int64_t)c0 + p.seg_len);
    const size_t sd = ((size_t)b * nseg + seg) * Nv + h;   // (sequence, segment, head) index

    // S rows 16*wv + 4*lq + e (key dims), columns col0 + 16*ct + lr
    // A sequence cut into several segments starts every segment from the
    // start state the combine pass wrote, segment 0's included (a copy of
    // the initial state): the last segment writes state_out during this same
    // launch, and state_out may alias state_in.  A sequence of one segment
    // reads state_in and writes state_out from the same threads.
    f32x4 S[CT];
    const float* sinit = MODE == 1 ? nullptr
                         : nsb > 1 ? p.sstart + sd * TILE
                                   : (p.state_in ? p.state_in + (size_t)stream * TILE : nullptr);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int dk = 16 * wv + 4 * lq + e, col = col0 + 16 * ct + lr;
            if constexpr (MODE == 1) S[ct][e] = col == dk ? 1.f : 0.f;
            else S[ct][e] = sinit ? sinit[(size_t)dk * 128 + col] : 0.f;
        }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) st_h4(&sST[(16 * ct + lr) * LD16 + 16 * wv + 4 * lq], to_h4(S[ct]));

    // the u columns of this slice (MODE 1: the columns that carry B; those
    // that carry M read the first columns of u, scaled by 0)
    const int ucol0 = MODE == 0 ? col0 : (col0 >= 128 ? col0 - 128 : 0);
    const float umul = MODE == 0 || col0 >= 128 ? 1.f : 0.f;
    const ScanLane ln{(uint32_t)(frag_off(16 * wv + lr, 8 * lq)), (uint32_t)(cfrag_off(16 * wv + 4 * lq, ucol0 + lr)),
                      (uint32_t)(16 * wv + 4 * lq)};
    // Register sets rotate between the chunk being computed and the ones being
    // fetched (no copies between them, so each chunk's compute waits only for
    // its own operands): three sets (two chunks of lookahead) up to 64 columns,
    // two sets at 128 columns, where a third would not fit in registers.
    // The compiler's memory-counter waits are exact only when every path into
    // a wait issued the same loads in the same order, so: every fetch is
    // issued unconditionally (past the last chunk it re-reads the last chunk,
    // unused), the prologue issues the sets whole and in loop order, and the
    // main loop runs whole rounds with one back edge; the last chunks that do
    // not fill a round are done after it, fetching nothing.
    const int cl = c1 - 1;
    __syncthreads();
    if (c0 < c1) {
        int c = c0;
        if constexpr (DS <= 64) {
            ScanOps<CT> A, B, C;
            scan_load<CT, GK>(A, p, c0, h, hq, ln);
            __builtin_amdgcn_sched_barrier(0);
            scan_load<CT, GK>(B, p, min(c0 + 1, cl), h, hq, ln);
            __builtin_amdgcn_sched_barrier(0);
            for (; c + 3 <= c1; c += 3) {
                scan_step<DS, true, MODE, GK>(A, S, p, c, h, sST, sVn, tid, wv, lr, lq, col0, C, min(c + 2, cl), hq,
                                          ln, umul);
                scan_step<DS, true, MODE, GK>(B, S, p, c + 1, h, sST, sVn, tid, wv, lr, lq, col0, A, min(c + 3, cl),
                                          hq, ln, umul);
                scan_step<DS, true, MODE, GK>(C, S, p, c + 2, h, sST, sVn, tid, wv, lr, lq, col0, B, min(c + 4, cl),
                                          hq, ln, umul);
            }
            if (c < c1)
                scan_step<DS, false, MODE, GK>(A, S, p, c, h, sST, sVn, tid, wv, lr, lq, col0, C, 0, hq, ln, umul);
            if (c + 1 < c1)
                scan_step<DS, false, MODE, GK>(B, S, p, c + 1, h, sST, sVn, tid, wv, lr, lq, col0, C, 0, hq, ln, umul);
        } else {
            ScanOps<CT> A, B;
            scan_load<CT, GK>(A, p, c0, h, hq, ln);
            __builtin_amdgcn_sched_barrier(0);
            for (; c + 2 <= c1; c += 2) {
                scan_step<DS, true, MODE, GK>(A, S, p, c, h, sST, sVn, tid, wv, lr, lq, col0, B, min(c + 1, cl), hq,
                                          ln, umul);
                scan_step<DS, true, MODE, GK>(B, S, p, c + 1, h, sST, sVn, tid, wv, lr, lq, col0, A, min(c + 2, cl),
                                          hq, ln, umul);
            }
            if (c < c1)
                scan_step<DS, false, MODE, GK>(A, S, p, c, h, sST, sVn, tid, wv, lr, lq, col0, B, 0, hq, ln, umul);
        }
    }
    if constexpr (MODE == 1) {
        // the map as one fp32 [dk][256] tile: M in columns 0..127, B in 128..255
        float* dst = p.mb + sd * (2 * TILE);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dk = 16 * wv + 4 * lq + e, col = col0 + 16 * ct + lr;
                dst[(size_t)dk * 256 + col] = S[ct][e];
            }
    } else if (seg == nsb - 1) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dk = 16 * wv + 4 * lq + e, col = col0 + 16 * ct + lr;
                p.state_out[(size_t)stream * TILE + (size_t)dk * 128 + col] = S[ct][e];
            }
    }
}

// Two-level scan, second level: the start state of every segment of a
// stream, S_0 = the stream's initial state, S_{s+1} = M_s S_s + B_s, in fp32.
// S_0 is written too, so that the scan proper reads no segment's start from
// state_in (state_out may alias it and is written by the last segment).
// One workgroup of 512 threads per (stream, 8 state columns).  Thread t owns
// row r = t / 4 of the product and the keys k = 16 i + 4 q + e (q = t % 4,
// i < 8, e < 4): its 32 entries of M_s sit in registers, fetched
// kCombineAhead maps ahead, so M never passes through LDS; the S slice does
// (double-buffered, one barrier per map), and the four threads of a row, one
// quad, add their partial sums with quad permutes.  Thread q then adds B and
// stores columns 2 q, 2 q + 1 of row r.
constexpr int kCombineCols = 8;    // state columns per workgroup
constexpr int kCombineAhead = 2;   // maps fetched ahead
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {   // x + (x of the lane CTRL selects within the DPP row)
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

__global__ __launch_bounds__(512) void combine_kernel(PrefillDev p) {
    constexpr int CW = kCombineCols, NPW = 128 / CW, CQ = CW / 4, NST = kCombineAhead + 1;
    constexpr int SLD = CW + 4;   // LDS row stride (floats): a quad's four rows fall in distinct banks
    __shared__ __align__(16) float sS[2][128 * SLD];
    const int Nv = p.Nv, nseg = p.nseg;
    const int stream = blockIdx.x / NPW, col0 = CW * (blockIdx.x % NPW);
    if (stream >= p.B * Nv) return;
    const int b = stream / Nv, h = stream % Nv;
    const int cb = ld_uniform(&p.meta[b]), ce = ld_uniform(&p.meta[b + 1]);
    const int nsb = ce > cb ? (ce - cb + p.seg_len - 1) / p.seg_len : 1;
    if (nsb < 2) return;
    const int tid = threadIdx.x, r = tid >> 2, q = tid & 3, cq = col0 + CQ * q;
    const size_t seg_stride = (size_t)Nv * TILE;
    float* sst = p.sstart + ((size_t)b * nseg * Nv + h) * TILE + (size_t)r * 128 + cq;   // segment 0, row r
    {
        float x[CQ];
#pragma unroll
        for (int j = 0; j < CQ; ++j)
            x[j] = p.state_in ? p.state_in[(size_t)stream * TILE + (size_t)r * 128 + cq + j] : 0.f;
#pragma unroll
        for (int j = 0; j < CQ; ++j) {
            sst[j] = x[j];
            sS[0][r * SLD + CQ * q + j] = x[j];
        }
    }
    const int last = nsb - 2;   // the last map used
    f32x4 m[NST][8];            // maps s .. s + NST - 1: M[r][16 i + 4 q .. + 3]
    float bb[NST][CQ];          //   and B[r][cq ..]
    auto fetch = [&](int slot, int s) {
        const float* MB = p.mb + (((size_t)b * nseg + min(s, last)) * Nv + h) * (2 * TILE) + (size_t)r * 256;
#pragma unroll
        for (int i = 0; i < 8; ++i) m[slot][i] = *reinterpret_cast<const f32x4*>(MB + 16 * i + 4 * q);
#pragma unroll
        for (int j = 0; j < CQ; ++j) bb[slot][j] = MB[128 + cq + j];
    };
    // one map: S_{s+1} = M_s S_s + B_s from sS[s & 1] into sS[(s + 1) & 1] and segment s + 1's start
    auto step = [&](int slot, int s) {
        const float* src = sS[s & 1];
        float acc[CW];
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[c] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float mk = m[slot][i][e];
                const float* row = src + (16 * i + 4 * q + e) * SLD;
#pragma unroll
                for (int c4 = 0; c4 < CW / 4; ++c4) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(row + 4 * c4);
#pragma unroll
                    for (int x = 0; x < 4; ++x) acc[4 * c4 + x] = fmaf(mk, v[x], acc[4 * c4 + x]);
                }
            }
#pragma unroll
        for (int c = 0; c < CW; ++c) acc[c] = dpp_add<0x4E>(dpp_add<0xB1>(acc[c]));   // lane ^ 1, then ^ 2
        float y[CQ];
#pragma unroll
        for (int j = 0; j < CQ; ++j) {
            const float a01 = q == 0 ? acc[j] : acc[CQ + j];
            const float a23 = q == 2 ? acc[2 * CQ + j] : acc[3 * CQ + j];
            y[j] = (q < 2 ? a01 : a23) + bb[slot][j];
        }
        float* dst = sst + (size_t)(s + 1) * seg_stride;
#pragma unroll
        for (int j = 0; j < CQ; ++j) {
            dst[j] = y[j];
            sS[(s + 1) & 1][r * SLD + CQ * q + j] = y[j];
        }
        __syncthreads();   // segment s + 1's start is in LDS; sS[s & 1] is free
    };
    static_assert(NST == 3, "the rounds below take three maps");
    fetch(0, 0);
    fetch(1, 1);
    fetch(2, 2);
    __syncthreads();   // S_0 is in LDS
    // Whole rounds of three maps, each issuing the same loads and stores, so
    // that the compiler's memory-counter waits at every step cover exactly
    // that step's map (fetches past the last map re-read it, unused); then
    // the last one or two maps.  (Written out: the same rounds as a loop
    // over the three slots let the compiler wait for later maps as well,
    // 75 against 54 us for one T=131072 stream group of four heads.)
    int s = 0;
    for (const int full = (last + 1) / NST * NST; s < full; s += NST) {
        step(0, s);
        fetch(0, s + 3);
        step(1, s + 1);
        fetch(1, s + 4);
        step(2, s + 2);
        fetch(2, s + 5);
    }
    if (s <= last) step(0, s);
    if (s + 1 <= last) step(1, s + 1);
}

// ------------------------------------------------------------------ K3: output
// 8 waves; wave w owns output rows 16w .. 16w+15.  The three operand tiles
// (k^, S_c^T, v_new^T) pass one after another through one LDS buffer.  The
// keys are normalised here from the input rows (each wave its own 16 rows);
// the S_c / v_new pair is fetched into registers up front, while k^ is in use.
// The pair is fetched in storage order: 16 B per lane, 1 KiB contiguous per
// wave; piece e holds the 4-row runs of S_c and of v_new at lane run e.  Each
// pair is read once, so the loads are non-temporal: together with the intra
// kernel's v rows (also read once) that took the T=8192 call from 190.4 to
// 183.8 us (same box; T=131072 unchanged); the same hint on rows that two
// value heads or several scan slices share (q, k; the scan's w and u) made
// the call slower (193-210 us).
__device__ __forceinline__ void pair_tile_fetch(u32x4 (&rg)[8], const _Float16* src, int tid) {
#pragma unroll
    for (int n = 0; n < 8; ++n)
        rg[n] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + (size_t)(tid + 512 * n) * 8));
}
// One tile of the pair (HALF 0: S_c, 1: v_new), X [row][col], placed
// transposed in LDS, X^T [col][row].
template <int HALF>
__device__ __forceinline__ void pair_tile_store_t(const u32x4 (&rg)[8], _Float16* dst, int tid) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int e = tid + 512 * n, blk = e >> 6, l = e & 63;
        const int r = 16 * (blk >> 3) + 4 * (l >> 4), c = 16 * (blk & 7) + (l & 15);
        *reinterpret_cast<u32x2*>(dst + c * LD16 + r) = u32x2{rg[n][2 * HALF], rg[n][2 * HALF + 1]};
    }
}

template <typename ActT>
__global__ __launch_bounds__(512, 4) void output_kernel(PrefillDev p) {
    __shared__ __align__(16) _Float16 sBuf[128 * LD16];
    __shared__ __align__(16) _Float16 sP[128 * LD16];
    __shared__ __align__(16) float sG[128];   // g_cum of the chunk

    const int Nv = p.Nv, Nqk = p.Nqk, G = Nv / Nqk;
    // the grid is a multiple of 8 G; items are taken last chunk first, the
    // ones whose S_c and v_new the scan wrote last and the last-level cache
    // most likely still holds
    const int item = (int)gridDim.x - 1 - group_slot(blockIdx.x, G);
    const int c = item / Nv, h = item % Nv, hq = h / G;
    if (c >= ld_uniform(&p.meta[p.B])) return;
    const int t0 = ld_uniform(&p.cmap[4 * c + 1]), r = ld_uniform(&p.cmap[4 * c + 2]);
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const ActT* Q = static_cast<const ActT*>(p.q);
    ActT* OUT = static_cast<ActT*>(p.out);
    const size_t ch = (size_t)c * Nv + h;
    const float* GC = p.gc + ch * 128;
    const int I = wv;

    // All of the item's tiles are fetched up front (one memory latency per
    // item rather than one per phase); the q rows follow the first.
    u32x4 stSV[8];
    Raw8<ActT> kr[4];
    {
        // k rows of this wave (rows past the chunk's end re-read its last row:
        // their entries of P lie above the diagonal or in rows never stored)
        const ActT* K = static_cast<const ActT*>(p.k);
        const int row = 16 * I + lr, lrow = min(row, max(r - 1, 0));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) raw_load(kr[ks], K + ((size_t)(t0 + lrow) * Nqk + hq) * 128 + 32 * ks + 8 * lq);
    }
    // q^ (scaled) and q^ e^{g_cum} for rows 16 I + lr
    half8 qh[4], qe[4];
    {
        // rows past the chunk's end re-read its last row (their outputs are
        // never stored, and P is zero above the diagonal)
        const int row = 16 * I + lr, lrow = min(row, max(r - 1, 0));
        Raw8<ActT> qr[4];   // held raw until used (as fp32 they would cost twice the registers)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) raw_load(qr[ks], Q + ((size_t)(t0 + lrow) * Nqk + hq) * 128 + 32 * ks + 8 * lq);
        const float eg = __expf(GC[row]);
        const float gmine = GC[tid & 127];
        __builtin_amdgcn_sched_barrier(0);
        pair_tile_fetch(stSV, p.scvn + 2 * ch * TILE, tid);
        __builtin_amdgcn_sched_barrier(0);
        if (tid < 128) sG[tid] = gmine;
        {
            // k^ = k / |k| -> sBuf rows of this wave, [tok][dk]
            float kx[4][8];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) raw_cvt(kr[ks], kx[ks]);
            float ksq = 0.f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int e = 0; e < 8; ++e) ksq = fmaf(kx[ks][e], kx[ks][e], ksq);
            ksq += __shfl_xor(ksq, 16);
            ksq += __shfl_xor(ksq, 32);
            const float kinv = 1.f / sqrtf(ksq + kNormEps);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] = kx[ks][e] * kinv;
                st_h8(&sBuf[(16 * I + lr) * LD16 + 32 * ks + 8 * lq], to_h8(y));
            }
        }
        float x[4][8];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) raw_cvt(qr[ks], x[ks]);
        float ssq = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) ssq = fmaf(x[ks][e], x[ks][e], ssq);
        ssq += __shfl_xor(ssq, 16);
        ssq += __shfl_xor(ssq, 32);
        const float rinv = p.scale / sqrtf(ssq + kNormEps);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float y[8], z[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) { y[e] = x[ks][e] * rinv; z[e] = y[e] * eg; }
            qh[ks] = to_h8(y);
            qe[ks] = to_h8(z);
        }
    }
    __syncthreads();

    // P = (q^ k^T) . D on the inclusive lower triangle -> sP rows of this wave.
    // Each tile is computed transposed (A = k^ rows j, B = q^ rows i), so a
    // lane holds four consecutive columns 16 J + 4 lq .. of row i = 16 I + lr.
    {
        const int i = 16 * I + lr;
        const float gi = sG[i];
        for (int J = 0; J <= I; ++J) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = mma(ld_h8(&sBuf[(16 * J + lr) * LD16 + 32 * ks + 8 * lq]), qh[ks], acc);
            const int j0 = 16 * J + 4 * lq;
            const f32x4 gj = *reinterpret_cast<const f32x4*>(&sG[j0]);
            half4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (_Float16)(i >= j0 + e ? acc[e] * __expf(gi - gj[e]) : 0.f);
            st_h4(&sP[i * LD16 + j0], o4);
        }
        // the next block's columns, read by the last k-step of P v_new
        if ((I & 1) == 0) st_h4(&sP[i * LD16 + 16 * (I + 1) + 4 * lq], half4{0, 0, 0, 0});
    }
    __syncthreads();
    pair_tile_store_t<0>(stSV, sBuf, tid);   // S_c^T [col][dk]
    __syncthreads();

    f32x4 o[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mma(qe[ks], ld_h8(&sBuf[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), acc);
        o[ct] = acc;
    }
    __syncthreads();
    pair_tile_store_t<1>(stSV, sBuf, tid);   // v_new^T [col][tok]
    __syncthreads();
    for (int ks = 0; ks <= I / 2; ++ks) {
        const half8 a = ld_h8(&sP[(16 * I + lr) * LD16 + 32 * ks + 8 * lq]);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) o[ct] = mma(a, ld_h8(&sBuf[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), o[ct]);
    }
    // rows < r -> out, staged through this wave's own rows of sP, 64 columns at a time
    float* so = reinterpret_cast<float*>(&sP[16 * I * LD16]);   // 16 x 68 floats
#pragma unroll
    for (int hx = 0; hx < 2; ++hx) {
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) so[(4 * lq + e) * 68 + 16 * ct + lr] = o[4 * hx + ct][e];
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        const int row = lane >> 2, seg = lane & 3, tok = 16 * I + row;
        if (tok < r) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                float y[8];
                lds_row8(&so[row * 68 + 16 * seg + 8 * n], y);
                store8(OUT + ((size_t)(t0 + tok) * Nv + h) * 128 + 64 * hx + 16 * seg + 8 * n, y);
            }
        }
    }
}

// ------------------------------------------------------------------ K3 with a per-key gate
// o = (q^ exp(G)) S_c + P v_new, both A operands stored by the intra kernel
// in fragment order (loaded straight into registers); S_c^T and v_new^T pass
// through LDS as in the output kernel.
template <typename ActT>
__global__ __launch_bounds__(512) void output_gk_kernel(PrefillDev p) {
    __shared__ __align__(16) _Float16 sBuf[128 * LD16];
    __shared__ __align__(16) float sStage[8 * 16 * 68];   // each wave's 16 output rows, 64 columns at a time
    const int Nv = p.Nv, Nqk = p.Nqk, G = Nv / Nqk;
    // the grid is a multiple of 8 G; items are taken last chunk first, the
    // ones whose S_c and v_new the scan wrote last and the last-level cache
    // most likely still holds
    const int item = (int)gridDim.x - 1 - group_slot(blockIdx.x, G);
    const int c = item / Nv, h = item % Nv;
    if (c >= ld_uniform(&p.meta[p.B])) return;
    const int t0 = ld_uniform(&p.cmap[4 * c + 1]), r = ld_uniform(&p.cmap[4 * c + 2]);
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const size_t ch = (size_t)c * Nv + h;
    const int I = wv;
    ActT* OUT = static_cast<ActT*>(p.out);

    half8 qe[4], pa[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        qe[ks] = ld_h8(p.qt + ch * TILE + frag_off(16 * I + lr, 32 * ks + 8 * lq));
        pa[ks] = ld_h8(p.pm + ch * TILE + frag_off(16 * I + lr, 32 * ks + 8 * lq));
    }
    u32x4 stSV[8];
    pair_tile_fetch(stSV, p.scvn + 2 * ch * TILE, tid);
    pair_tile_store_t<0>(stSV, sBuf, tid);   // S_c^T [col][dk]
    __syncthreads();
    f32x4 o[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) acc = mma(qe[ks], ld_h8(&sBuf[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), acc);
        o[ct] = acc;
    }
    __syncthreads();
    pair_tile_store_t<1>(stSV, sBuf, tid);   // v_new^T [col][tok]
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        if (ks > I / 2) break;   // P is zero past these columns
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            o[ct] = mma(pa[ks], ld_h8(&sBuf[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), o[ct]);
    }
    // rows < r -> out, staged through this wave's own rows of sStage, 64 columns at a time
    float* so = &sStage[I * 16 * 68];
#pragma unroll
    for (int hx = 0; hx < 2; ++hx) {
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int ct = 0; ct < 4; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) so[(4 * lq + e) * 68 + 16 * ct + lr] = o[4 * hx + ct][e];
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        const int row = lane >> 2, seg = lane & 3, tok = 16 * I + row;
        if (tok < r) {
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                float y[8];
                lds_row8(&so[row * 68 + 16 * seg + 8 * n], y);
                store8(OUT + ((size_t)(t0 + tok) * Nv + h) * 128 + 64 * hx + 16 * seg + 8 * n, y);
            }
        }
    }
}


// ------------------------------------------------------------------ K2 with K3 fused, per-key gate
// With a per-key gate the intra kernel stores both A operands of the output
// (q^ exp(G) and P, fragment order), so the one-level scan forms each chunk's
// output itself, where S_c and v_new are on chip: neither is written to
// memory and no output pass runs.  For this slice's columns
//   o^T = S_c^T (q^ e^G)^T + v_new^T P^T.
// Wave wv owns output rows i = 16 wv + lr.  Both products are taken
// transposed -- A = S^T or v_new^T fragments from LDS, B = the stored row
// fragments, whose A-operand layout is the B-operand layout of the transposed
// product -- so that a lane holds four consecutive columns of one row.  The
// first shares the S^T fragments that v_new = u - w S reads; the second reads
// the v_new^T tile that the state update reads (with this gate v_new enters
// the update unscaled: the chunk's decays sit in k^T).
template <int CT>
struct GkOutOps {
    ScanOps<CT> s;        // w, k^T (with its decays), u and G_last of the chunk
    half8 qe[4], pa[4];   // q^ e^G and P, rows 16 wv + lr (key blocks of 32)
    int t0, r;            // the chunk's first token and its number of rows
};

// Parts as in the scan (0: w, 1: u and the gates, 2: k^T), with q^ e^G in
// part 0 (needed first) and P in part 2 (needed after the first barrier).
// Key blocks of P past wv / 2 are zero and never used: their fetch re-reads
// block wv / 2.
template <int CT, int PART>
__device__ __forceinline__ void gk_out_load_part(GkOutOps<CT>& o, const PrefillDev& p, int c, int h, int hq,
                                                 const ScanLane& ln, int wvu) {
    const size_t ch = (size_t)c * p.Nv + h;
    if constexpr (PART == 0) {
        o.t0 = ld_uniform(&p.cmap[4 * c + 1]);
        o.r = ld_uniform(&p.cmap[4 * c + 2]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o.qe[ks] = ld_h8(p.qt + ch * TILE + ln.a + 512 * ks);
    }
    if constexpr (PART == 2) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) o.pa[ks] = ld_h8(p.pm + ch * TILE + ln.a + 512 * min(ks, wvu >> 1));
    }
    scan_load_part<CT, PART, true>(o.s, p, c, h, hq, ln);
}

template <int DS, bool LOAD, typename ActT>
__device__ __forceinline__ void scan_gk_out_step(const GkOutOps<DS / 16>& o, f32x4 (&S)[DS / 16],
                                                 const PrefillDev& p, int h, _Float16* sST, _Float16* sVn, int wv,
                                                 int wvu, int lr, int lq, int col0, GkOutOps<DS / 16>& nx, int cn,
                                                 int hq, const ScanLane& ln) {
    constexpr int CT = DS / 16;
    if constexpr (LOAD) {
        gk_out_load_part<CT, 0>(nx, p, cn, h, hq, ln, wvu);
        __builtin_amdgcn_sched_barrier(0);
    }
    // v_new = u - w S (tokens 16 wv + 4 lq + e) and (q^ e^G S_c)^T (rows
    // i = 16 wv + lr), from the same S^T fragments
    const int tok = 16 * wv + 4 * lq;
    f32x4 oT[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
        f32x4 vp = {0.f, 0.f, 0.f, 0.f}, oi = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const half8 b = ld_h8(&sST[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]);
            vp = mma(o.s.aw[ks], b, vp);
            oi = mma(b, o.qe[ks], oi);
        }
        oT[ct] = oi;
        f32x4 vn;
#pragma unroll
        for (int e = 0; e < 4; ++e) vn[e] = (float)o.s.u4[ct][e] - vp[e];
        st_h4(&sVn[(16 * ct + lr) * LD16 + tok], to_h4(vn));
    }
    if constexpr (LOAD) {
        __builtin_amdgcn_sched_barrier(0);
        gk_out_load_part<CT, 1>(nx, p, cn, h, hq, ln, wvu);
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if constexpr (LOAD) {
        __builtin_amdgcn_sched_barrier(0);
        gk_out_load_part<CT, 2>(nx, p, cn, h, hq, ln, wvu);
        __builtin_amdgcn_sched_barrier(0);
    }
    // S <- exp(G_last) S + k^T v_new, row by row (the gate slot holds G_last
    // of this lane's rows)
    {
        f32x4 dec;
#pragma unroll
        for (int e = 0; e < 4; ++e) dec[e] = __expf(o.s.gcr[e]);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            f32x4 acc = S[ct] * dec;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = mma(o.s.ak[ks], ld_h8(&sVn[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), acc);
            S[ct] = acc;
            st_h4(&sST[(16 * ct + lr) * LD16 + 16 * wv + 4 * lq], to_h4(acc));
        }
    }
    // o^T += v_new^T P^T over the key blocks ks <= wv / 2; rows < r -> out
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        if (ks > (wvu >> 1)) break;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
            oT[ct] = mma(ld_h8(&sVn[(16 * ct + lr) * LD16 + 32 * ks + 8 * lq]), o.pa[ks], oT[ct]);
    }
    const int i = 16 * wv + lr;
    if (i < o.r) {
        ActT* OUT = static_cast<ActT*>(p.out) + ((size_t)(o.t0 + i) * p.Nv + h) * 128 + col0 + 4 * lq;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) store4(OUT + 16 * ct, oT[ct]);
    }
    __syncthreads();
}

// One workgroup per (sequence, value head, slice of DS state columns), placed
// as the scan's.  Two register sets rotate between the chunk being computed
// and the one being fetched; every fetch is issued (past the last chunk it
// re-reads the last chunk, unused), as in the scan.
template <int DS, typename ActT>
__global__ __launch_bounds__(512) void scan_gk_out_kernel(PrefillDev p) {
    constexpr int NS = 128 / DS, CT = DS / 16;
    __shared__ __align__(16) _Float16 sST[DS * LD16];   // S^T [col][dk] (fp16), the chunk's start state
    __shared__ __align__(16) _Float16 sVn[DS * LD16];   // v_new^T [col][tok]

    const int Nv = p.Nv, Nqk = p.Nqk, G = Nv / Nqk;
    const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
    const int local = j % (G * NS), grp = (j / (G * NS)) * 8 + xcd;
    if (grp >= p.B * Nqk) return;
    const int hq = grp % Nqk, b = grp / Nqk;
    const int slice = local % NS, h = hq * G + local / NS;
    const int stream = b * Nv + h;
    const int col0 = slice * DS;
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63, lr = lane & 15, lq = lane >> 4;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int c0 = ld_uniform(&p.meta[b]), c1 = ld_uniform(&p.meta[b + 1]);

    f32x4 S[CT];
    const float* sinit = p.state_in ? p.state_in + (size_t)stream * TILE : nullptr;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            S[ct][e] = sinit ? sinit[(size_t)(16 * wv + 4 * lq + e) * 128 + col0 + 16 * ct + lr] : 0.f;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) st_h4(&sST[(16 * ct + lr) * LD16 + 16 * wv + 4 * lq], to_h4(S[ct]));

    const ScanLane ln{(uint32_t)(frag_off(16 * wv + lr, 8 * lq)), (uint32_t)(cfrag_off(16 * wv + 4 * lq, col0 + lr)),
                      (uint32_t)(16 * wv + 4 * lq)};
    __syncthreads();
    if (c0 < c1) {
        const int cl = c1 - 1;
        int c = c0;
        GkOutOps<CT> A, B;
        gk_out_load_part<CT, 0>(A, p, c0, h, hq, ln, wvu);
        gk_out_load_part<CT, 1>(A, p, c0, h, hq, ln, wvu);
        gk_out_load_part<CT, 2>(A, p, c0, h, hq, ln, wvu);
        __builtin_amdgcn_sched_barrier(0);
        for (; c + 2 <= c1; c += 2) {
            scan_gk_out_step<DS, true, ActT>(A, S, p, h, sST, sVn, wv, wvu, lr, lq, col0, B, min(c + 1, cl), hq, ln);
            scan_gk_out_step<DS, true, ActT>(B, S, p, h, sST, sVn, wv, wvu, lr, lq, col0, A, min(c + 2, cl), hq, ln);
        }
        if (c < c1) scan_gk_out_step<DS, false, ActT>(A, S, p, h, sST, sVn, wv, wvu, lr, lq, col0, B, 0, hq, ln);
    }
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            p.state_out[(size_t)stream * TILE + (size_t)(16 * wv + 4 * lq + e) * 128 + col0 + 16 * ct + lr] = S[ct][e];
}

}  // namespace

// Compute units of the current device (queried once per device).
static int compute_units() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

template <int RULE>
static void launch_intra_rule(int act, dim3 grid, hipStream_t stream, const PrefillDev& p) {
    if (act == kActBf16) GDR_LAUNCH(kIntra, (intra_kernel<uint16_t, RULE>), grid, dim3(512), 0, stream, p);
    else if (act == kActFp16) GDR_LAUNCH(kIntra, (intra_kernel<_Float16, RULE>), grid, dim3(512), 0, stream, p);
    else GDR_LAUNCH(kIntra, (intra_kernel<float, RULE>), grid, dim3(512), 0, stream, p);
}
template <int RULE>
static void launch_intra_gk_rule(int act, dim3 grid, hipStream_t stream, const PrefillDev& p) {
    if (act == kActBf16) GDR_LAUNCH(kIntra, (intra_gk_kernel<uint16_t, RULE>), grid, dim3(512), 0, stream, p);
    else if (act == kActFp16) GDR_LAUNCH(kIntra, (intra_gk_kernel<_Float16, RULE>), grid, dim3(512), 0, stream, p);
    else GDR_LAUNCH(kIntra, (intra_gk_kernel<float, RULE>), grid, dim3(512), 0, stream, p);
}
// The scan launch for a slice width, one- or two-level pass, with or without the per-key gate.
template <int DS, int MODE>
static void launch_scan(bool gk, dim3 grid, hipStream_t stream, const PrefillDev& p) {
    if (gk) GDR_LAUNCH(kScan, (scan_kernel<DS, MODE, true>), grid, dim3(512), 0, stream, p);
    else GDR_LAUNCH(kScan, (scan_kernel<DS, MODE, false>), grid, dim3(512), 0, stream, p);
}
// The per-key-gate scan with the output fused in, for a slice width.
template <int DS>
static void launch_scan_gk_out(int act, dim3 grid, hipStream_t stream, const PrefillDev& p) {
    if (act == kActBf16) GDR_LAUNCH(kScan, (scan_gk_out_kernel<DS, uint16_t>), grid, dim3(512), 0, stream, p);
    else if (act == kActFp16) GDR_LAUNCH(kScan, (scan_gk_out_kernel<DS, _Float16>), grid, dim3(512), 0, stream, p);
    else GDR_LAUNCH(kScan, (scan_gk_out_kernel<DS, float>), grid, dim3(512), 0, stream, p);
}
static void launch_intra(int rule, int act, dim3 grid, hipStream_t stream, const PrefillDev& p) {
    switch (rule) {
        case 1: launch_intra_rule<1>(act, grid, stream, p); break;
        case 2: launch_intra_rule<2>(act, grid, stream, p); break;
        case 3: launch_intra_rule<3>(act, grid, stream, p); break;
        default: launch_intra_rule<0>(act, grid, stream, p); break;
    }
}

hipError_t prefill_launch(const PrefillArgs& a, const PrefillLayout& lay, int act, hipStream_t stream) {
    const int ncu = compute_units();
    PrefillDev p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.g = a.g; p.beta = a.beta; p.cu = a.cu;
    p.state_in = a.state_in; p.out = a.out; p.state_out = a.state_out;
    p.meta = reinterpret_cast<int32_t*>(a.ws + lay.off_meta);
    p.cmap = reinterpret_cast<int32_t*>(a.ws + lay.off_cmap);
    p.khatT = reinterpret_cast<_Float16*>(a.ws + lay.off_khatT);
    p.w = reinterpret_cast<_Float16*>(a.ws + lay.off_w);
    p.u = reinterpret_cast<_Float16*>(a.ws + lay.off_u);
    p.gc = reinterpret_cast<float*>(a.ws + lay.off_gc);
    p.scvn = reinterpret_cast<_Float16*>(a.ws + lay.off_scvn);
    p.gk = a.gk;
    p.qt = reinterpret_cast<_Float16*>(a.ws + lay.off_qt);
    p.pm = reinterpret_cast<_Float16*>(a.ws + lay.off_pm);
    p.mb = reinterpret_cast<float*>(a.ws + lay.off_mb);
    p.sstart = reinterpret_cast<float*>(a.ws + lay.off_sstart);
    p.T = a.T; p.nc = lay.nc; p.B = a.B; p.Nqk = a.Nqk; p.Nv = a.Nv; p.scale = a.scale;
    p.nseg = lay.nseg; p.seg_len = lay.seg_len;

    const size_t nwg = (size_t)lay.nc * a.Nv;
    const bool gk = a.gk != nullptr;   // the API passes it only with a rule that decays
    // Few sequences: the intra kernel builds the chunk map itself.
    p.map_in_intra = (nwg > 0 && a.B <= kMapSeqs) ? 1 : 0;
    hipError_t e = hipSuccess;
    if (!p.map_in_intra) {
        GDR_LAUNCH(kChunkmap, chunkmap_kernel, dim3(1), dim3(256), 0, stream, a.cu, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (nwg > 0) {
        const size_t g8 = (size_t)8 * (a.Nv / a.Nqk);
        if (gk) {
            // persistent: one workgroup per CU (LDS about 157 KiB), each walking items
            const dim3 grid((unsigned)(((nwg < (size_t)ncu ? nwg : (size_t)ncu) + g8 - 1) / g8 * g8));
            if (a.rule == 2) launch_intra_gk_rule<2>(act, grid, stream, p);
            else launch_intra_gk_rule<0>(act, grid, stream, p);
        } else {
            // persistent: two workgroups per CU (LDS < 80 KiB each), each walking items
            const size_t nint = ((nwg < (size_t)2 * ncu ? nwg : (size_t)2 * ncu) + g8 - 1) / g8 * g8;
            launch_intra(a.rule, act, dim3((unsigned)nint), stream, p);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // State columns are split over NS = 128 / DS workgroups per (sequence,
    // segment, head) stream.  A narrower slice shortens each serial step (less
    // MFMA and LDS work per workgroup) but every slice fetches the chunk's
    // whole w and k^T tiles; on 256 CUs the best measured split keeps
    // streams x NS between 256 and about 1024 workgroups.  Launches cover
    // every (sequence, segment) pair of the bound; absent segments exit.
    const size_t G = (size_t)(a.Nv / a.Nqk);
    const size_t ngroup = ((size_t)a.B * lay.nseg * a.Nqk + 7) / 8 * 8;
    if (lay.nseg > 1) {
        // first level: the maps of all segments but each sequence's last
        launch_scan<128, 1>(gk, dim3((unsigned)(ngroup * G * 2)), stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // second level: the segments' start states
        GDR_LAUNCH(kScan, combine_kernel, dim3((unsigned)((size_t)a.B * a.Nv * (128 / kCombineCols))), dim3(512), 0,
                   stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // (segments have equal lengths, so there their slices are sized to fit
    // one workgroup per CU)
    const size_t nstream = (size_t)a.B * a.Nv * lay.nseg;
    int ns = nstream >= 512 ? 1 : nstream >= 256 ? 2 : nstream >= 64 ? 4 : 8;
    while (lay.nseg > 1 && ns > 1 && nstream * ns > (size_t)ncu) ns >>= 1;
    // With a per-key gate the one-level scan forms the output itself (slices
    // of at most 64 columns, which fit its registers); the other cases record
    // S_c and v_new for the output pass.
    const bool fused = gk && lay.nseg == 1;
    if (fused && ns == 1) ns = 2;
    const size_t nscan = ngroup * G * ns;
    if (fused) {
        switch (ns) {
            case 2: launch_scan_gk_out<64>(act, dim3((unsigned)nscan), stream, p); break;
            case 4: launch_scan_gk_out<32>(act, dim3((unsigned)nscan), stream, p); break;
            default: launch_scan_gk_out<16>(act, dim3((unsigned)nscan), stream, p); break;
        }
    } else {
        switch (ns) {
            case 1: launch_scan<128, 0>(gk, dim3((unsigned)nscan), stream, p); break;
            case 2: launch_scan<64, 0>(gk, dim3((unsigned)nscan), stream, p); break;
            case 4: launch_scan<32, 0>(gk, dim3((unsigned)nscan), stream, p); break;
            default: launch_scan<16, 0>(gk, dim3((unsigned)nscan), stream, p); break;
        }
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (nwg > 0 && !fused) {
        const size_t g8 = (size_t)8 * (a.Nv / a.Nqk);
        const unsigned nout = (unsigned)((nwg + g8 - 1) / g8 * g8);
        if (gk) {
            if (act == kActBf16) GDR_LAUNCH(kOutput, output_gk_kernel<uint16_t>, dim3(nout), dim3(512), 0, stream, p);
            else if (act == kActFp16)
                GDR_LAUNCH(kOutput, output_gk_kernel<_Float16>, dim3(nout), dim3(512), 0, stream, p);
            else GDR_LAUNCH(kOutput, output_gk_kernel<float>, dim3(nout), dim3(512), 0, stream, p);
        } else {
            if (act == kActBf16) GDR_LAUNCH(kOutput, output_kernel<uint16_t>, dim3(nout), dim3(512), 0, stream, p);
            else if (act == kActFp16) GDR_LAUNCH(kOutput, output_kernel<_Float16>, dim3(nout), dim3(512), 0, stream, p);
            else GDR_LAUNCH(kOutput, output_kernel<float>, dim3(nout), dim3(512), 0, stream, p);
        }
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gdr
