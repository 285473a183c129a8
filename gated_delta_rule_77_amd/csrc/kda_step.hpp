// The single-token KDA step shared by the decode kernel, the replay fold and
// the fused layer step.
//
// Math ([K3-ATTN §2.2], three steps without a d_k x d_k matrix; order of
// [LA-KDA §5.2]: decay, erase, write, read).  With S' = Diag(alpha) S:
//   p = S'^T k,  r = S'^T q          (one pass over S)
//   u = beta (v - p)                  (the corrected value)
//   S <- S' + k u^T                   (erase + write)
//   o = S^T q = r + (q . k) u         (read after the update)
// Sources: [K3-ATTN] "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构";
//          [LA-KDA]  "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制".
//
// Layout: thread t owns rows [16*rg, 16*rg + 16) and columns [4*cg, 4*cg + 4)
// of the row-major [DK][DV] state (CG = DV/4 column groups, RG = DK/16 row
// groups), held in registers as 16 float4.
#pragma once
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

// One token for one (sequence, head): S (this thread's 16 x 4 block, in
// registers) advances by one step; with WITH_Q the output o = S^T q is also
// formed.  Every product that feeds an addition is an explicit fma and no
// other contraction is allowed, so the arithmetic of a step is fixed by this
// source: the decode kernel and the replay fold below run the same step and
// produce the same bits.
// MODE picks a row of the family table ([LA-KDA §4]): kModeGLA writes
// u = beta v without the erase (no p), kModeDeltaNet takes alpha = 1 without
// reading zt.
template <int DK, int DV, typename Tin, bool WITH_Q, int MODE = kModeKDA>
__device__ __forceinline__ void kda_token_step(float4 (&Sv)[16], const Tin* __restrict__ kt,
                                               const Tin* __restrict__ vt, const float* __restrict__ zt,
                                               float b_logit, float ea, const Tin* __restrict__ qt,
                                               Tin* __restrict__ ot, float* s_al, float* s_k,
                                               float* s_q, float (*s_red)[DK / 16][DV],
                                               float* s_qk = nullptr) {
#pragma clang fp contract(off)
    constexpr int CG = DV / 4, RG = DK / 16, NT = CG * RG;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    for (int i = t; i < DK; i += NT) {
        s_al[i] = MODE == kModeDeltaNet ? 1.f : expf(log_decay<true>(ea, zt[i]));
        s_k[i] = to_f32(kt[i]);
        if (WITH_Q) s_q[i] = to_f32(qt[i]);
    }
    const float beta = sigmoid_f<true>(b_logit);
    float vj[4];
#pragma unroll
    for (int c = 0; c < 4; c++) vj[c] = to_f32(vt[cg * 4 + c]);
    __syncthreads();

    // partial S'^T k (and S'^T q, q . k) over this thread's 16 rows
    float p[4] = {0.f, 0.f, 0.f, 0.f}, r4[4] = {0.f, 0.f, 0.f, 0.f}, qkp = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int i = rg * 16 + r;
        if (MODE != kModeGLA) {
            const float ka = s_al[i] * s_k[i];
            p[0] = __builtin_fmaf(ka, Sv[r].x, p[0]);
            p[1] = __builtin_fmaf(ka, Sv[r].y, p[1]);
            p[2] = __builtin_fmaf(ka, Sv[r].z, p[2]);
            p[3] = __builtin_fmaf(ka, Sv[r].w, p[3]);
        }
        if (WITH_Q) {
            const float qa = s_al[i] * s_q[i];
            r4[0] = __builtin_fmaf(qa, Sv[r].x, r4[0]);
            r4[1] = __builtin_fmaf(qa, Sv[r].y, r4[1]);
            r4[2] = __builtin_fmaf(qa, Sv[r].z, r4[2]);
            r4[3] = __builtin_fmaf(qa, Sv[r].w, r4[3]);
            qkp = __builtin_fmaf(s_q[i], s_k[i], qkp);
        }
    }
    *reinterpret_cast<float4*>(&s_red[0][rg][cg * 4]) = make_float4(p[0], p[1], p[2], p[3]);
    if (WITH_Q) {
        *reinterpret_cast<float4*>(&s_red[1][rg][cg * 4]) = make_float4(r4[0], r4[1], r4[2], r4[3]);
        if (cg == 0) s_qk[rg] = qkp;
    }
    __syncthreads();

    float P[4] = {0.f, 0.f, 0.f, 0.f}, R[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gidx = 0; gidx < RG; gidx++) {
        const float4 a = *reinterpret_cast<const float4*>(&s_red[0][gidx][cg * 4]);
        P[0] += a.x; P[1] += a.y; P[2] += a.z; P[3] += a.w;
        if (WITH_Q) {
            const float4 c = *reinterpret_cast<const float4*>(&s_red[1][gidx][cg * 4]);
            R[0] += c.x; R[1] += c.y; R[2] += c.z; R[3] += c.w;
        }
    }
    float u[4];
#pragma unroll
    for (int c = 0; c < 4; c++) u[c] = MODE == kModeGLA ? beta * vj[c] : beta * (vj[c] - P[c]);
    if (WITH_Q) {
        float qk = 0.f;       // row-group partials of q . k, summed in a fixed order
#pragma unroll
        for (int gidx = 0; gidx < RG; gidx++) qk += s_qk[gidx];
        if (rg == 0) {
#pragma unroll
            for (int c = 0; c < 4; c++) ot[cg * 4 + c] = from_f32<Tin>(__builtin_fmaf(qk, u[c], R[c]));
        }
    }
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int i = rg * 16 + r;
        const float al = s_al[i], ki = s_k[i];
        Sv[r].x = __builtin_fmaf(ki, u[0], al * Sv[r].x);
        Sv[r].y = __builtin_fmaf(ki, u[1], al * Sv[r].y);
        Sv[r].z = __builtin_fmaf(ki, u[2], al * Sv[r].z);
        Sv[r].w = __builtin_fmaf(ki, u[3], al * Sv[r].w);
    }
}

template <int DK, int DV>
__device__ __forceinline__ void load_state(float4 (&Sv)[16], const float* __restrict__ S) {
    constexpr int CG = DV / 4;
    const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
#pragma unroll
    for (int r = 0; r < 16; r++)
        Sv[r] = *reinterpret_cast<const float4*>(S + (size_t)(rg * 16 + r) * DV + cg * 4);
}

template <int DK, int DV>
__device__ __forceinline__ void store_state(const float4 (&Sv)[16], float* __restrict__ S) {
    constexpr int CG = DV / 4;
    const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
#pragma unroll
    for (int r = 0; r < 16; r++)
        *reinterpret_cast<float4*>(S + (size_t)(rg * 16 + r) * DV + cg * 4) = Sv[r];
}

}  // namespace kda
