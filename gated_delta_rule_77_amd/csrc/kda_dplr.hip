// General diagonal-plus-low-rank (DPLR) update, fp32 arithmetic: chunked
// prefill for every supported shape and the single-token step.
//
// [K3-ATTN §2.2] writes the KDA update as three steps (decay, a rank-1
// correction, the write) and credits binding the diagonal and low-rank terms
// to the same key k with halving the chunk matrices of the general form.
// The general form lifts that binding: per (sequence, head), S in R^{dk x dv},
//   S'  = Diag(alpha_t) S_{t-1}            alpha_t: the KDA gate of z_t ([LA-KDA §5.4])
//   S'' = S' + a_t (b_t^T S')              the low-rank pair (a_t, b_t)
//   S_t = S'' + k_t v_t^T,   o_t = S_t^T q_t.
// KDA is a = -beta k, b = k with write key beta k.
//
// Chunked form (G = in-chunk inclusive cumulative log-decay, Gamma = e^G,
// e_ij = e^{G_i - G_j} per channel; x_i = S'_i^T b_i the low-rank read):
//   A_ba[i,j] = sum_c b_ic a_jc e_ijc (j < i)    A_bk[i,j] = sum_c b_ic k_jc e_ijc (j < i)
//   A_qa[i,j] = sum_c q_ic a_jc e_ijc (j <= i)   A_qk[i,j] = sum_c q_ic k_jc e_ijc (j <= i)
//   T = (I - A_ba)^{-1},  Wb = T (B . Gamma),  Ub = (T A_bk) V
//   X = Wb S + Ub
//   O = (Q . Gamma) S + A_qa X + A_qk V
//   S <- Diag(Gamma_C) S + (A . e^{G_C - G})^T X + (K . e^{G_C - G})^T V
// Four C x C matrices where KDA forms two (A_kk, A_qk).
// Sources: [K3-ATTN] "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构" §2.2;
//          [LA-KDA] "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制" §5.4, §7.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

template <int DK, int DV, int C>
struct DplrRec {
    static constexpr size_t W = 0;                       // Wb [C][DK]
    static constexpr size_t U = W + (size_t)C * DK;      // Ub [C][DV]
    static constexpr size_t Q = U + (size_t)C * DV;      // Q . Gamma [C][DK]
    static constexpr size_t A = Q + (size_t)C * DK;      // A . e^{G_C - G} [C][DK]
    static constexpr size_t K = A + (size_t)C * DK;      // K . e^{G_C - G} [C][DK]
    static constexpr size_t AQA = K + (size_t)C * DK;    // A_qa [C][C]
    static constexpr size_t AQK = AQA + (size_t)C * C;   // A_qk [C][C]
    static constexpr size_t G = AQK + (size_t)C * C;     // Gamma_C [DK]
    static constexpr size_t FLOATS = G + DK;
};

// One workgroup per (chunk, head).  Positions past the end of the sequence
// read as zero inputs with g = 0, so they add nothing and decay nothing.
template <int DK, int DV, int C, typename Tin>
__global__ __launch_bounds__(256)
void gen_dplr_intra_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                           const Tin* __restrict__ v, const Tin* __restrict__ la,
                           const Tin* __restrict__ lb, const float* __restrict__ z,
                           const float* __restrict__ A, const int* __restrict__ hdr,
                           const int4* __restrict__ chunks, int H, float* __restrict__ recs)
{
    using R = DplrRec<DK, DV, C>;
    const int cid = blockIdx.x, h = blockIdx.y;
    if (cid >= hdr[0]) return;
    const int4 cd = chunks[cid];
    const int tok0 = cd.y, len = cd.z;
    const int tid = threadIdx.x;
    float* rec = recs + ((size_t)cid * H + h) * R::FLOATS;

    __shared__ float sG[C][DK];
    __shared__ float sAba[C][C];     // A_ba, then M = T A_bk
    __shared__ float sAbk[C][C];
    __shared__ float sN[C][C];       // T = (I - A_ba)^{-1}

    auto at = [&](const Tin* x, int i, int c) -> float {
        return i < len ? to_f32(x[((size_t)(tok0 + i) * H + h) * DK + c]) : 0.f;
    };

    const float ea = expf(A[h]);
    for (int c = tid; c < DK; c += 256) {
        float run = 0.f;
        for (int i = 0; i < C; i++) {
            if (i < len) run += log_decay<true>(ea, z[((size_t)(tok0 + i) * H + h) * DK + c]);
            sG[i][c] = run;
        }
    }
    __syncthreads();

    // the four chunk matrices; e^{G_i - G_j} <= 1 for j <= i
    for (int idx = tid; idx < C * C; idx += 256) {
        const int i = idx / C, j = idx % C;
        float aba = 0.f, abk = 0.f, aqa = 0.f, aqk = 0.f;
        if (j <= i) {
            for (int c = 0; c < DK; c++) {
                const float e = expf(sG[i][c] - sG[j][c]);
                const float aj = at(la, j, c) * e, kj = at(k, j, c) * e;
                const float bi = at(lb, i, c), qi = at(q, i, c);
                aba += bi * aj;
                abk += bi * kj;
                aqa += qi * aj;
                aqk += qi * kj;
            }
        }
        sAba[i][j] = j < i ? aba : 0.f;
        sAbk[i][j] = j < i ? abk : 0.f;
        rec[R::AQA + idx] = aqa;
        rec[R::AQK + idx] = aqk;
    }
    __syncthreads();

    // T = (I - A_ba)^{-1}: column j by forward substitution (unit diagonal)
    for (int j = tid; j < C; j += 256) {
        for (int i = 0; i < C; i++) {
            float acc = i == j ? 1.f : 0.f;
            for (int m = j; m < i; m++) acc += sAba[i][m] * sN[m][j];
            sN[i][j] = i < j ? 0.f : acc;
        }
    }
    __syncthreads();
    // M = T A_bk (strictly lower), into the A_ba buffer
    static_assert(C * C % 256 == 0, "whole passes over the C x C matrices");
    constexpr int kPass = C * C / 256;
    float mv[kPass];
#pragma unroll
    for (int u = 0; u < kPass; u++) {
        const int idx = tid + 256 * u, i = idx / C, m = idx % C;
        float acc = 0.f;
        for (int j = m + 1; j <= i; j++) acc += sN[i][j] * sAbk[j][m];
        mv[u] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPass; u++) sAba[(tid + 256 * u) / C][(tid + 256 * u) % C] = mv[u];
    __syncthreads();

    for (int idx = tid; idx < C * DK; idx += 256) {
        const int i = idx / DK, c = idx % DK;
        float acc = 0.f;
        for (int j = 0; j <= i; j++) acc += sN[i][j] * at(lb, j, c) * expf(sG[j][c]);
        rec[R::W + idx] = acc;
        rec[R::Q + idx] = at(q, i, c) * expf(sG[i][c]);
        const float dec = expf(sG[C - 1][c] - sG[i][c]);
        rec[R::A + idx] = at(la, i, c) * dec;
        rec[R::K + idx] = at(k, i, c) * dec;
    }
    for (int idx = tid; idx < C * DV; idx += 256) {
        const int i = idx / DV, c = idx % DV;
        float acc = 0.f;
        for (int m = 0; m < i; m++)
            acc += sAba[i][m] * (m < len ? to_f32(v[((size_t)(tok0 + m) * H + h) * DV + c]) : 0.f);
        rec[R::U + idx] = acc;
    }
    for (int c = tid; c < DK; c += 256) rec[R::G + c] = expf(sG[C - 1][c]);
}

// One workgroup per (sequence, head); the fp32 state lives in LDS.
template <int DK, int DV, int C, typename Tin>
__global__ __launch_bounds__(256)
void gen_dplr_chain_kernel(const float* __restrict__ recs, const int2* __restrict__ seqs,
                           const int4* __restrict__ chunks, const Tin* __restrict__ v,
                           const float* __restrict__ h0, int H, Tin* __restrict__ o,
                           float* __restrict__ hT)
{
    using R = DplrRec<DK, DV, C>;
    const int p = blockIdx.x;           // sequence * H + head
    const int n = p / H, h = p % H;
    const int tid = threadIdx.x;

    __shared__ float sS[DK][DV];
    __shared__ float sX[C][DV];

    for (int idx = tid; idx < DK * DV; idx += 256)
        sS[idx / DV][idx % DV] = h0 ? h0[(size_t)p * DK * DV + idx] : 0.f;

    const int2 sd = seqs[n];
    for (int ci = 0; ci < sd.y; ci++) {
        const int cid = sd.x + ci;
        const int4 cd = chunks[cid];
        const int tok0 = cd.y, len = cd.z;
        const float* rec = recs + ((size_t)cid * H + h) * R::FLOATS;
        auto vin = [&](int i, int j) -> float {
            return i < len ? to_f32(v[((size_t)(tok0 + i) * H + h) * DV + j]) : 0.f;
        };
        __syncthreads();
        for (int idx = tid; idx < C * DV; idx += 256) {
            const int i = idx / DV, j = idx % DV;
            float acc = rec[R::U + idx];
            for (int c = 0; c < DK; c++) acc += rec[R::W + i * DK + c] * sS[c][j];
            sX[i][j] = acc;
        }
        __syncthreads();
        for (int idx = tid; idx < C * DV; idx += 256) {
            const int i = idx / DV, j = idx % DV;
            if (i >= len) continue;
            float acc = 0.f;
            for (int c = 0; c < DK; c++) acc += rec[R::Q + i * DK + c] * sS[c][j];
            for (int m = 0; m <= i; m++)
                acc += rec[R::AQA + i * C + m] * sX[m][j] + rec[R::AQK + i * C + m] * vin(m, j);
            o[((size_t)(tok0 + i) * H + h) * DV + j] = from_f32<Tin>(acc);
        }
        __syncthreads();
        for (int idx = tid; idx < DK * DV; idx += 256) {
            const int c = idx / DV, j = idx % DV;
            float acc = rec[R::G + c] * sS[c][j];
            for (int i = 0; i < C; i++)
                acc += rec[R::A + i * DK + c] * sX[i][j] + rec[R::K + i * DK + c] * vin(i, j);
            sS[c][j] = acc;
        }
    }
    __syncthreads();
    if (hT)
        for (int idx = tid; idx < DK * DV; idx += 256)
            hT[(size_t)p * DK * DV + idx] = sS[idx / DV][idx % DV];
}

// One token per (sequence, head): thread (cg, rg) holds rows [16 rg, 16 rg + 16)
// and columns [4 cg, 4 cg + 4) of the state in registers.  One pass over
// S' = Diag(alpha) S forms x = S'^T b and r = S'^T q; then
// S = S' + a x^T + k v^T and o = S^T q = r + (q . a) x + (q . k) v.
template <int D, typename Tin>
__global__ __launch_bounds__((D / 4) * (D / 16))
void dplr_decode_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                        const Tin* __restrict__ v, const Tin* __restrict__ la,
                        const Tin* __restrict__ lb, const float* __restrict__ z,
                        const float* __restrict__ A, float* __restrict__ state,
                        Tin* __restrict__ o, int H)
{
    constexpr int CG = D / 4, RG = D / 16, NT = CG * RG;
    const int nh = blockIdx.x, t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    float* S = state + (size_t)nh * D * D;
    __shared__ float s_al[D], s_k[D], s_q[D], s_a[D], s_b[D];
    __shared__ __align__(16) float s_red[2][RG][D];
    float4 Sv[16];
#pragma unroll
    for (int r = 0; r < 16; r++)
        Sv[r] = *reinterpret_cast<const float4*>(S + (size_t)(rg * 16 + r) * D + cg * 4);
    const float ea = expf(A[nh % H]);
    const size_t base = (size_t)nh * D;
    for (int i = t; i < D; i += NT) {
        s_al[i] = expf(log_decay<true>(ea, z[base + i]));
        s_k[i] = to_f32(k[base + i]);
        s_q[i] = to_f32(q[base + i]);
        s_a[i] = to_f32(la[base + i]);
        s_b[i] = to_f32(lb[base + i]);
    }
    float vj[4];
#pragma unroll
    for (int c = 0; c < 4; c++) vj[c] = to_f32(v[base + cg * 4 + c]);
    __syncthreads();

    float x[4] = {0.f, 0.f, 0.f, 0.f}, r4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int i = rg * 16 + r;
        Sv[r].x *= s_al[i]; Sv[r].y *= s_al[i]; Sv[r].z *= s_al[i]; Sv[r].w *= s_al[i];
        const float bi = s_b[i], qi = s_q[i];
        x[0] += bi * Sv[r].x; x[1] += bi * Sv[r].y; x[2] += bi * Sv[r].z; x[3] += bi * Sv[r].w;
        r4[0] += qi * Sv[r].x; r4[1] += qi * Sv[r].y; r4[2] += qi * Sv[r].z; r4[3] += qi * Sv[r].w;
    }
    *reinterpret_cast<float4*>(&s_red[0][rg][cg * 4]) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(&s_red[1][rg][cg * 4]) = make_float4(r4[0], r4[1], r4[2], r4[3]);
    __syncthreads();
    float X[4] = {0.f, 0.f, 0.f, 0.f}, Rr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gi = 0; gi < RG; gi++) {
        const float4 p0 = *reinterpret_cast<const float4*>(&s_red[0][gi][cg * 4]);
        const float4 p1 = *reinterpret_cast<const float4*>(&s_red[1][gi][cg * 4]);
        X[0] += p0.x; X[1] += p0.y; X[2] += p0.z; X[3] += p0.w;
        Rr[0] += p1.x; Rr[1] += p1.y; Rr[2] += p1.z; Rr[3] += p1.w;
    }
    if (rg == 0) {
        float qa = 0.f, qk = 0.f;
        for (int i = 0; i < D; i++) {
            qa += s_q[i] * s_a[i];
            qk += s_q[i] * s_k[i];
        }
#pragma unroll
        for (int c = 0; c < 4; c++)
            o[base + cg * 4 + c] = from_f32<Tin>(Rr[c] + qa * X[c] + qk * vj[c]);
    }
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int i = rg * 16 + r;
        const float ai = s_a[i], ki = s_k[i];
        Sv[r].x += ai * X[0] + ki * vj[0];
        Sv[r].y += ai * X[1] + ki * vj[1];
        Sv[r].z += ai * X[2] + ki * vj[2];
        Sv[r].w += ai * X[3] + ki * vj[3];
        *reinterpret_cast<float4*>(S + (size_t)i * D + cg * 4) = Sv[r];
    }
}

template <int D, int C, typename Tin>
hipError_t launch_dplr_generic_t(const ChunkArgs& a) {
    const int* hdr = reinterpret_cast<const int*>(a.ws);
    const int4* chunks = reinterpret_cast<const int4*>(a.ws + a.L.off_chunks);
    const int2* seqs = reinterpret_cast<const int2*>(a.ws + a.L.off_seqs);
    float* recs = reinterpret_cast<float*>(a.ws + a.L.off_recs);
    hipLaunchKernelGGL((gen_dplr_intra_kernel<D, D, C, Tin>), dim3((unsigned)a.L.cap, (unsigned)a.H),
                       dim3(256), 0, a.stream, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v,
                       (const Tin*)a.la, (const Tin*)a.lb, a.z, a.A, hdr, chunks, a.H, recs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev && (e = hipEventRecord(a.ev[2], a.stream)) != hipSuccess) return e;
    hipLaunchKernelGGL((gen_dplr_chain_kernel<D, D, C, Tin>), dim3((unsigned)(a.N * a.H)), dim3(256),
                       0, a.stream, (const float*)recs, seqs, chunks, (const Tin*)a.v, a.h0, a.H,
                       (Tin*)a.o, a.hT);
    return hipGetLastError();
}

template <int D, typename Tin>
hipError_t launch_dplr_decode_t(const void* q, const void* k, const void* v, const void* la,
                                const void* lb, const float* z, const float* A, float* state,
                                void* o, int N, int H, hipStream_t s) {
    constexpr int NT = (D / 4) * (D / 16);
    hipLaunchKernelGGL((dplr_decode_kernel<D, Tin>), dim3((unsigned)N * H), dim3(NT), 0, s,
                       (const Tin*)q, (const Tin*)k, (const Tin*)v, (const Tin*)la, (const Tin*)lb,
                       z, A, state, (Tin*)o, H);
    return hipGetLastError();
}

}  // namespace

static_assert(DplrRec<128, 128, 64>::FLOATS == dplr_generic_rec_floats(128, 128, 64) &&
              DplrRec<16, 16, 16>::FLOATS == dplr_generic_rec_floats(16, 16, 16),
              "record size of the workspace layout");

hipError_t launch_dplr_generic(const ChunkArgs& a, int dtype_bf16) {
#define KDA_DPLR(D, CC)                                                                  \
    if (a.dk == D && a.C == CC)                                                          \
        return dtype_bf16 ? launch_dplr_generic_t<D, CC, bf16>(a) : launch_dplr_generic_t<D, CC, float>(a);
    KDA_DPLR(16, 16) KDA_DPLR(16, 64) KDA_DPLR(32, 16) KDA_DPLR(32, 64)
    KDA_DPLR(64, 16) KDA_DPLR(64, 64) KDA_DPLR(128, 16) KDA_DPLR(128, 64)
#undef KDA_DPLR
    return hipErrorInvalidValue;
}

hipError_t launch_dplr_decode(const void* q, const void* k, const void* v, const void* la,
                              const void* lb, const float* z, const float* A, float* state,
                              void* o, int N, int H, int d, int dtype_bf16, hipStream_t s) {
#define KDA_DPLR_DEC(D)                                                                          \
    if (d == D) return dtype_bf16                                                                \
        ? launch_dplr_decode_t<D, bf16>(q, k, v, la, lb, z, A, state, o, N, H, s)               \
        : launch_dplr_decode_t<D, float>(q, k, v, la, lb, z, A, state, o, N, H, s);
    KDA_DPLR_DEC(16) KDA_DPLR_DEC(32) KDA_DPLR_DEC(64) KDA_DPLR_DEC(128)
#undef KDA_DPLR_DEC
    return hipErrorInvalidValue;
}

}  // namespace kda
