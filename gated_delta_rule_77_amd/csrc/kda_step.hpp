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
// Layout: every thread owns a 16-row x 4-column block of the row-major
// [DK][DV] state, held in registers as 16 float4 (StateLayout below).  At
// d = 128 a wave owns 32 whole columns, so the sums over rows for p and r
// stay inside the wave (cross-lane adds, no LDS, no barrier); the smaller
// sizes of the fp32 path sum row groups through LDS.  The state is streamed
// with nontemporal loads and stores: it is read and written once per call,
// and a serving loop's states (64 KiB per layer and head) do not stay in the
// caches between a layer's steps.
#pragma once
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

// The state block of thread t: rows [row0, row0 + 16), columns [col0, col0 + 4).
//   d = 128 (kWave): wave w = t / 64 owns columns [32w, 32w + 32); lane l of
//     it holds columns 32w + 4 (l % 8) .. + 3 and rows 16 (l / 8) .. + 15, so
//     the 8 lanes that share a column group (l % 8) cover all 128 rows.
//   other sizes, and d = 128 with WAVE false: thread t holds columns
//     4 (t % CG) .. + 3 and rows 16 (t / CG) .. + 15 (CG = DV / 4 column
//     groups, DK / 16 row groups); a wave spans 2 row groups at d = 128.
template <int DK, int DV, bool WAVE = true> struct StateLayout {
    static constexpr bool kWave = WAVE && DK == 128 && DV == 128;
    static constexpr int CG = DV / 4, RG = DK / 16, NT = CG * RG;
    __device__ static int col0(int t) { return kWave ? 32 * (t >> 6) + 4 * (t & 7) : 4 * (t % CG); }
    __device__ static int row0(int t) { return kWave ? 16 * ((t & 63) >> 3) : 16 * (t / CG); }
};

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 load_nt(const float* p) {
    const f32x4v x = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    return make_float4(x.x, x.y, x.z, x.w);
}

__device__ __forceinline__ void store_nt(float* p, float4 v) {
    const f32x4v x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4v*>(p));
}

// What thread t reads of one token: the gate logit, key and query of the
// channels i = t, t + NT, ... (below DK), the beta logit, and the values of
// its 4 state columns.  Loaded apart from the step so that a caller can issue
// these small loads before the state stream and the gate arithmetic waits on
// them alone.
template <int DK, int DV> struct TokenIn {
    static constexpr int KPT = (DK + StateLayout<DK, DV>::NT - 1) / StateLayout<DK, DV>::NT;
    float z[KPT], k[KPT], q[KPT], v[4], b;
};

template <int DK, int DV, typename Tin, bool WITH_Q, int MODE = kModeKDA, bool WAVE = true>
__device__ __forceinline__ void load_token(TokenIn<DK, DV>& in, const Tin* __restrict__ kt,
                                           const Tin* __restrict__ vt, const float* __restrict__ zt,
                                           float b_logit, const Tin* __restrict__ qt) {
    using SL = StateLayout<DK, DV, WAVE>;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < TokenIn<DK, DV>::KPT; j++) {
        const int i = t + j * SL::NT;
        in.z[j] = in.k[j] = in.q[j] = 0.f;
        if (i < DK) {
            if (MODE != kModeDeltaNet) in.z[j] = zt[i];
            in.k[j] = to_f32(kt[i]);
            if (WITH_Q) in.q[j] = to_f32(qt[i]);
        }
    }
    const int c0 = SL::col0(t);
#pragma unroll
    for (int c = 0; c < 4; c++) in.v[c] = to_f32(vt[c0 + c]);
    in.b = b_logit;
}

// One token for one (sequence, head): S (this thread's 16 x 4 block, in
// registers) advances by one step; with WITH_Q the output o = S^T q is also
// formed.  Every product that feeds an addition is an explicit fma and no
// other contraction is allowed, so the arithmetic of a step is fixed by this
// source: the decode kernel, the replay fold, the verify pass and the fused
// layer step run the same step and produce the same bits.
// MODE picks a row of the family table ([LA-KDA §4]): kModeGLA writes
// u = beta v without the erase (no p), kModeDeltaNet takes alpha = 1 without
// a gate logit.  With STORE each updated row is also written to S_out (the
// thread's block of a row-major state) as soon as it is formed.  WAVE picks
// the state layout (StateLayout): at d = 128 the one-token kernels sum over
// row groups inside each wave with an xor butterfly (no barrier), while the
// multi-token loops of the fold and verify pass keep the row-group layout and
// sum through LDS.  Both add the 8 row groups' partial sums in the same
// pairwise order, ((g0 + g1) + (g2 + g3)) + ((g4 + g5) + (g6 + g7)), and
// every thread forms its partial over its 16 rows in row order, so both give
// the same bits.
template <int DK, int DV, typename Tin, bool WITH_Q, int MODE = kModeKDA, bool STORE = false,
          bool WAVE = true>
__device__ __forceinline__ void kda_token_step(float4 (&Sv)[16], const TokenIn<DK, DV>& in,
                                               float ea, Tin* __restrict__ ot, float* s_al,
                                               float* s_k, float* s_q,
                                               float (*s_red)[DK / 16][DV],
                                               float* s_qk = nullptr,
                                               float* __restrict__ S_out = nullptr) {
#pragma clang fp contract(off)
    using SL = StateLayout<DK, DV, WAVE>;
    constexpr int CG = SL::CG, RG = SL::RG, NT = SL::NT;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;           // the row-group layout (not kWave)
    const int col0 = SL::col0(t), row0 = SL::row0(t);
#pragma unroll
    for (int j = 0; j < TokenIn<DK, DV>::KPT; j++) {
        const int i = t + j * NT;
        if (i < DK) {
            s_al[i] = MODE == kModeDeltaNet ? 1.f : expf(log_decay<true>(ea, in.z[j]));
            s_k[i] = in.k[j];
            if (WITH_Q) s_q[i] = in.q[j];
        }
    }
    const float beta = sigmoid_f<true>(in.b);
    const float* vj = in.v;
    __syncthreads();

    // partial S'^T k (and S'^T q, q . k) over this thread's 16 rows
    float p[4] = {0.f, 0.f, 0.f, 0.f}, r4[4] = {0.f, 0.f, 0.f, 0.f}, qkp = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int i = row0 + r;
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
    float P[4] = {0.f, 0.f, 0.f, 0.f}, R[4] = {0.f, 0.f, 0.f, 0.f}, qk = 0.f;
    if constexpr (SL::kWave) {
        // the 8 lanes of a column group are 8, 16 and 32 apart: an xor
        // butterfly leaves the same sum (same bits) in all of them
#pragma unroll
        for (int c = 0; c < 4; c++) {
            P[c] = p[c];
            R[c] = r4[c];
        }
        qk = qkp;
#pragma unroll
        for (int m = 8; m < 64; m <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; c++) {
                if (MODE != kModeGLA) P[c] += __shfl_xor(P[c], m, 64);
                if (WITH_Q) R[c] += __shfl_xor(R[c], m, 64);
            }
            if (WITH_Q) qk += __shfl_xor(qk, m, 64);
        }
    } else {
        *reinterpret_cast<float4*>(&s_red[0][rg][cg * 4]) = make_float4(p[0], p[1], p[2], p[3]);
        if (WITH_Q) {
            *reinterpret_cast<float4*>(&s_red[1][rg][cg * 4]) = make_float4(r4[0], r4[1], r4[2], r4[3]);
            if (cg == 0) s_qk[rg] = qkp;
        }
        __syncthreads();
        // the RG row-group partials summed as a pairwise tree (the order of
        // the butterfly above when RG = 8)
        float a[4][RG], c[4][RG], qq[RG];
#pragma unroll
        for (int gidx = 0; gidx < RG; gidx++) {
            const float4 x = *reinterpret_cast<const float4*>(&s_red[0][gidx][cg * 4]);
            a[0][gidx] = x.x; a[1][gidx] = x.y; a[2][gidx] = x.z; a[3][gidx] = x.w;
            if (WITH_Q) {
                const float4 y = *reinterpret_cast<const float4*>(&s_red[1][gidx][cg * 4]);
                c[0][gidx] = y.x; c[1][gidx] = y.y; c[2][gidx] = y.z; c[3][gidx] = y.w;
                qq[gidx] = s_qk[gidx];
            }
        }
#pragma unroll
        for (int m = 1; m < RG; m <<= 1)
#pragma unroll
            for (int gidx = 0; gidx < RG; gidx += 2 * m) {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    a[e][gidx] += a[e][gidx + m];
                    if (WITH_Q) c[e][gidx] += c[e][gidx + m];
                }
                if (WITH_Q) qq[gidx] += qq[gidx + m];
            }
#pragma unroll
        for (int e = 0; e < 4; e++) {
            P[e] = a[e][0];
            R[e] = c[e][0];
        }
        if (WITH_Q) qk = qq[0];
    }
    float u[4];
#pragma unroll
    for (int c = 0; c < 4; c++) u[c] = MODE == kModeGLA ? beta * vj[c] : beta * (vj[c] - P[c]);
    if (WITH_Q && row0 == 0) {
#pragma unroll
        for (int c = 0; c < 4; c++) ot[col0 + c] = from_f32<Tin>(__builtin_fmaf(qk, u[c], R[c]));
    }
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int i = row0 + r;
        const float al = s_al[i], ki = s_k[i];
        Sv[r].x = __builtin_fmaf(ki, u[0], al * Sv[r].x);
        Sv[r].y = __builtin_fmaf(ki, u[1], al * Sv[r].y);
        Sv[r].z = __builtin_fmaf(ki, u[2], al * Sv[r].z);
        Sv[r].w = __builtin_fmaf(ki, u[3], al * Sv[r].w);
        if (STORE) store_nt(S_out + (size_t)i * DV + col0, Sv[r]);
    }
}

// NT: nontemporal loads and stores (the one-token kernels, bound by the state
// stream); plain ones for the multi-token loops, bound by their steps.
template <int DK, int DV, bool WAVE = true, bool NT = true>
__device__ __forceinline__ void load_state(float4 (&Sv)[16], const float* __restrict__ S) {
    using SL = StateLayout<DK, DV, WAVE>;
    const int c0 = SL::col0(threadIdx.x), r0 = SL::row0(threadIdx.x);
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const float* p = S + (size_t)(r0 + r) * DV + c0;
        Sv[r] = NT ? load_nt(p) : *reinterpret_cast<const float4*>(p);
    }
}

template <int DK, int DV, bool WAVE = true, bool NT = true>
__device__ __forceinline__ void store_state(const float4 (&Sv)[16], float* __restrict__ S) {
    using SL = StateLayout<DK, DV, WAVE>;
    const int c0 = SL::col0(threadIdx.x), r0 = SL::row0(threadIdx.x);
#pragma unroll
    for (int r = 0; r < 16; r++) {
        float* p = S + (size_t)(r0 + r) * DV + c0;
        if (NT) store_nt(p, Sv[r]);
        else *reinterpret_cast<float4*>(p) = Sv[r];
    }
}

}  // namespace kda
