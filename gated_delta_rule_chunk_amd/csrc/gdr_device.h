// gdr_device.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct bf16_t { uint16_t bits; };

// ---- scalar conversions ----------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(uint32_t(b) << 16);
}
// Round to nearest even (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---- 8-element vector load / store in either activation dtype --------------
// bf16: one 16-byte access; fp32: two 16-byte accesses.
__device__ __forceinline__ void load8(const uint16_t* p, float (&x)[8]) {
    u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(r[i] << 16);
        x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float (&x)[8]) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8(uint16_t* p, const float (&x)[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = uint32_t(f32_to_bf16(x[2 * i])) | (uint32_t(f32_to_bf16(x[2 * i + 1])) << 16);
    *reinterpret_cast<u32x4*>(p) = r;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// 4-element vector store: bf16 one 8-byte access, fp32 one 16-byte access.
__device__ __forceinline__ void store4(uint16_t* p, f32x4 x) {
    u32x2 r;
    r[0] = uint32_t(f32_to_bf16(x[0])) | (uint32_t(f32_to_bf16(x[1])) << 16);
    r[1] = uint32_t(f32_to_bf16(x[2])) | (uint32_t(f32_to_bf16(x[3])) << 16);
    *reinterpret_cast<u32x2*>(p) = r;
}
__device__ __forceinline__ void store4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }

// 4-element vector load: bf16 one 8-byte access, fp32 one 16-byte access.
__device__ __forceinline__ void load4(const uint16_t* p, float (&x)[4]) {
    const u32x2 r = *reinterpret_cast<const u32x2*>(p);
    x[0] = __uint_as_float(r[0] << 16);
    x[1] = __uint_as_float(r[0] & 0xffff0000u);
    x[2] = __uint_as_float(r[1] << 16);
    x[3] = __uint_as_float(r[1] & 0xffff0000u);
}
__device__ __forceinline__ void load4(const float* p, float (&x)[4]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = a[i];
}

// Non-temporal 8-element load / store, for data streamed through exactly once
// (the decode state slabs): hints the caches not to keep the lines.
__device__ __forceinline__ void load8_nt(const uint16_t* p, float (&x)[8]) {
    const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(r[i] << 16);
        x[2 * i + 1] = __uint_as_float(r[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8_nt(const float* p, float (&x)[8]) {
    const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}
__device__ __forceinline__ void store8_nt(uint16_t* p, const float (&x)[8]) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        r[i] = uint32_t(f32_to_bf16(x[2 * i])) | (uint32_t(f32_to_bf16(x[2 * i + 1])) << 16);
    __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void store8_nt(float* p, const float (&x)[8]) {
    __builtin_nontemporal_store(f32x4{x[0], x[1], x[2], x[3]}, reinterpret_cast<f32x4*>(p));
    __builtin_nontemporal_store(f32x4{x[4], x[5], x[6], x[7]}, reinterpret_cast<f32x4*>(p + 4));
}

// Scalar load of one element of any activation dtype.
__device__ __forceinline__ float load1(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const _Float16* p) { return (float)*p; }

// ---- IEEE half (fp16) activations and state: one 16-byte access per 8 ----
__device__ __forceinline__ void load8(const _Float16* p, float (&x)[8]) {
    const half8 r = *reinterpret_cast<const half8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)r[i];
}
__device__ __forceinline__ void store4(_Float16* p, f32x4 x) {
    *reinterpret_cast<half4*>(p) = half4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]};
}
__device__ __forceinline__ void store8(_Float16* p, const float (&x)[8]) {
    half8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (_Float16)x[i];   // round to nearest even
    *reinterpret_cast<half8*>(p) = r;
}
__device__ __forceinline__ void load4(const _Float16* p, float (&x)[4]) {
    const half4 r = *reinterpret_cast<const half4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = (float)r[i];
}
__device__ __forceinline__ void load8_nt(const _Float16* p, float (&x)[8]) {
    const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const half8 h = __builtin_bit_cast(half8, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
}
__device__ __forceinline__ void store8_nt(_Float16* p, const float (&x)[8]) {
    half8 h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = (_Float16)x[i];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h), reinterpret_cast<u32x4*>(p));
}

}  // namespace gdr
