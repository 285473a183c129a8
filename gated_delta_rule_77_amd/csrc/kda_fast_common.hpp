// Device helpers shared by the intra-chunk kernels of the MFMA path (KDA and
// the general DPLR update): LDS strides, the per-channel decay-factor table,
// the tile-pair schedule and the fp32 unit-lower-triangular inverse.
#pragma once
#include "kda_device.hpp"

namespace kda {
namespace fastc {

// acc += A (16x16, row-major, lda) * B (16x16, row-major, ldb), fp32 MFMA.
// Step ks gives lane group g the index k = 4g + ks: a lane reads its four A
// values as one 16-byte piece of row n and its B values down column n, rows
// 4g..4g+3.  With a B row stride of 4 (mod 16) words (68 and 20 here) the B
// reads of one step fall on 64 distinct banks (bank = 16g + n + const).
__device__ __forceinline__ f32x4 mm16_f32(f32x4 acc, const float* A, int lda, const float* B,
                                          int ldb, int n16, int g4) {
    const float4 a = *reinterpret_cast<const float4*>(A + n16 * lda + 4 * g4);
    const float av[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) acc = mfma_f32(av[ks], B[(4 * g4 + ks) * ldb + n16], acc);
    return acc;
}

__device__ __forceinline__ void load8f(const float* p, float* out) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// LDS row strides (elements), padded so that 16-byte fragment reads whose
// rows vary across lanes fall on distinct banks: 528-byte fp32 rows of L and
// K.F, 272-byte bf16 rows, 272-byte rows of the 64x64 fp32 matrices.
constexpr int kLdG = 132;   // fp32 [64][kLdG]: L, then K.F in place
constexpr int kLdK = 136;   // bf16 row operands [64][kLdK]
constexpr int kLdA = 68;    // fp32 64x64 matrices [64][kLdA]
constexpr int kLdP = 20;    // the inverse's 16x16 fp32 partial products [16][kLdP]
constexpr int kInvScr = 4 * 16 * kLdP;   // floats of inverse scratch: a [16][kLdP] tile per wave
// per-channel factor rows (fp32 [128] each); L_s(r) = L at row 16r - 1
// (0 for r = 0), L_e(r) = L at row 16r + 15, L_C = L at row 63:
constexpr int kFX = 0;      // X(r,s) = 2^(L_s(r) - L_e(s)), row r(r+1)/2 + s, s <= r
constexpr int kFY = 10;     // Y(r) = 2^L_s(r)
constexpr int kFZ = 14;     // Z(r) = 2^(L_C - L_e(r))
constexpr int kFL = 18;     // L_e(r) itself
constexpr int kNFac = 22;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16x16 tile pairs (r, s), s <= r, numbered p = r(r+1)/2 + s; wave w takes
// p in [pair_beg(w), pair_beg(w + 1)): 3, 3, 2 and 2 tiles.
__device__ __forceinline__ int pair_beg(int w) { return w == 0 ? 0 : w == 1 ? 3 : w == 2 ? 6 : w == 3 ? 8 : 10; }
__device__ __forceinline__ int pair_row(int p) { return p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3; }

// N = (I + A)^{-1} for a strictly lower-triangular 64 x 64 fp32 A in LDS
// ([64][kLdA] rows), in fp32 by 16 x 16 blocks ([LA-KDA §8]: serial inside a
// 16-token tile, matrix products between tiles).  N must hold zeros on entry
// (its upper blocks stay zero); sP is kInvScr floats of scratch.  Every
// thread of the 256-thread workgroup calls it (it holds barriers).
__device__ __forceinline__ void unit_lower_inverse(const float* sA, float* sN, float* sP, int w,
                                                   int n16, int g4) {
    // diagonal blocks: forward substitution, lane = (block, column)
    if (w == 0) {
        const int rb = g4, cc = n16;
        const float* Ab = sA + (16 * rb) * kLdA + 16 * rb;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; i++) {
            float acc = (i == cc) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < i; m++) acc -= Ab[i * kLdA + m] * x[m];
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; i++) sN[(16 * rb + i) * kLdA + 16 * rb + cc] = x[i];
    }
    __syncthreads();
    // off-diagonal blocks by distance d: N_rs = -N_rr sum_{m=s}^{r-1} A_rm N_ms
    for (int d = 1; d < 4; d++) {
        const bool act = w < 4 - d;
        const int r = w + d, s = w;
        if (act) {
            f32x4 P = zero4();
            for (int m = s; m < r; m++)
                P = mm16_f32(P, sA + 16 * r * kLdA + 16 * m, kLdA, sN + 16 * m * kLdA + 16 * s, kLdA,
                             n16, g4);
#pragma unroll
            for (int e = 0; e < 4; e++) sP[w * 16 * kLdP + (4 * g4 + e) * kLdP + n16] = P[e];
        }
        __syncthreads();
        if (act) {
            const f32x4 R = mm16_f32(zero4(), sN + 16 * r * kLdA + 16 * r, kLdA, sP + w * 16 * kLdP, kLdP, n16, g4);
#pragma unroll
            for (int e = 0; e < 4; e++) sN[(16 * r + 4 * g4 + e) * kLdA + 16 * s + n16] = -R[e];
        }
        __syncthreads();
    }
}

}  // namespace fastc
}  // namespace kda
