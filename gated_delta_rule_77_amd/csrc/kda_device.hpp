// Device-side helpers shared by the libkda kernels (gfx950 only).
//
// MFMA fragment conventions used throughout (wave64, 16x16 output tiles):
//   lane l = n + 16*g  (n = l & 15, g = l >> 4)
//   C/D tile: lane l element e holds D[4*g + e][n]                  (e = 0..3)
//   A operand: lane l holds row m = n and the lane group's k-slots
//   B operand: lane l holds column n and the lane group's k-slots
// A and B fragments pair their slots identically, so any consistent choice of
// which k index sits in which (g, e) slot gives the same product.  The
// kernels exploit this: a C/D tile, or two of them stacked, is reused as an
// operand whose k order follows the tile's own row order, with no shuffle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

// lower bound of the log-decay: alpha = exp(kGMin * sigmoid(.)) lies in (e^-5, 1)
constexpr float kGMin = -5.0f;

// sigma(x) = 1 / (1 + e^-x).  Saturates cleanly: e^-x overflows to +inf for
// very negative x (sigma -> 0) and underflows to 0 for very positive x.
template <bool kPrecise>
__device__ __forceinline__ float sigmoid_f(float x) {
    if constexpr (kPrecise) return 1.0f / (1.0f + expf(-x));
    else return 1.0f / (1.0f + __expf(-x));
}

template <bool kPrecise>
__device__ __forceinline__ float exp_f(float x) {
    if constexpr (kPrecise) return expf(x);
    else return __expf(x);
}

// log-decay g = kGMin * sigma(e^{A_h} z) for one channel; ea = e^{A_h}
template <bool kPrecise>
__device__ __forceinline__ float log_decay(float ea, float z) {
    return kGMin * sigmoid_f<kPrecise>(ea * z);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { f32x4 r = {0.f, 0.f, 0.f, 0.f}; return r; }

// two C tiles' lane elements (4 + 4) packed as one bf16 operand fragment
__device__ __forceinline__ bf16x8 pack_frag(f32x4 lo, f32x4 hi) {
    bf16x8 r;
    r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
    r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
    return r;
}

__device__ __forceinline__ bf16x8 pack_frag_neg(f32x4 lo, f32x4 hi) {
    bf16x8 r;
    r[0] = (bf16)(-lo[0]); r[1] = (bf16)(-lo[1]); r[2] = (bf16)(-lo[2]); r[3] = (bf16)(-lo[3]);
    r[4] = (bf16)(-hi[0]); r[5] = (bf16)(-hi[1]); r[6] = (bf16)(-hi[2]); r[7] = (bf16)(-hi[3]);
    return r;
}

__device__ __forceinline__ bf16x4 pack4(f32x4 x) {
    bf16x4 r;
    r[0] = (bf16)x[0]; r[1] = (bf16)x[1]; r[2] = (bf16)x[2]; r[3] = (bf16)x[3];
    return r;
}

__device__ __forceinline__ f32x4 unpack4(bf16x4 x) {
    f32x4 r = {(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    return r;
}

__device__ __forceinline__ bf16x8 concat44(bf16x4 a, bf16x4 b) {
    bf16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return r;
}

}  // namespace kda
