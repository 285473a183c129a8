// Chunked KDA prefill with fp32 arithmetic throughout (any supported d_k =
// d_v and chunk size, fp32 or bf16 inputs).  Plain VALU code: it carries the
// fp32 configurations and every shape the MFMA path does not cover.
//
// Per chunk (local positions i, j; G = in-chunk inclusive cumulative
// log-decay; Gamma = e^G), the chunked form of [LA-KDA §7.2-§7.3] with the
// decay carried on the key side:
//   A_kk[i,j] = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}   (j < i)
//   A_qk[i,j] =        sum_c q_ic k_jc e^{G_ic - G_jc}   (j <= i)
//   T = (I + A_kk)^{-1} Diag(beta), W = T (K . Gamma), U = T V
//   V~ = U - W S,  O = (Q . Gamma) S + A_qk V~,  S <- Diag(Gamma_C) S + (K . e^{G_C - G})^T V~
// Here every decay factor is evaluated as e^{difference} with a non-positive
// exponent, so nothing can overflow whatever the chunk length.
// The family modes ([LA-KDA §4] table): kModeDeltaNet takes G = 0 without
// reading the gate logits; kModeGLA drops A_kk and stores W = 0, so that
// V~ = U = Diag(beta) V.
// Sources: [LA-KDA] "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制" §5.4, §7.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

namespace {

template <int DK, int DV, int C>
struct GenRec {
    static constexpr size_t W = 0;
    static constexpr size_t U = W + (size_t)C * DK;
    static constexpr size_t Q = U + (size_t)C * DV;
    static constexpr size_t K = Q + (size_t)C * DK;
    static constexpr size_t A = K + (size_t)C * DK;
    static constexpr size_t G = A + (size_t)C * C;
    static constexpr size_t FLOATS = G + DK;
};

template <int DK, int DV, int C, typename Tin>
__global__ __launch_bounds__(256)
void gen_intra_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                      const Tin* __restrict__ v, const float* __restrict__ z,
                      const float* __restrict__ bl, const float* __restrict__ A,
                      const int* __restrict__ hdr, const int4* __restrict__ chunks, int H,
                      float* __restrict__ recs, float* __restrict__ dbg, int mode)
{
    using R = GenRec<DK, DV, C>;
    const int cid = blockIdx.x, h = blockIdx.y;
    if (cid >= hdr[0]) return;
    const int4 cd = chunks[cid];
    const int tok0 = cd.y, len = cd.z;
    const int tid = threadIdx.x;
    float* rec = recs + ((size_t)cid * H + h) * R::FLOATS;

    __shared__ float sG[C][DK];
    __shared__ float sAkk[C][C];
    __shared__ float sN[C][C];
    __shared__ float sBeta[C];

    auto at_k = [&](int i, int c) -> float {
        return i < len ? to_f32(k[((size_t)(tok0 + i) * H + h) * DK + c]) : 0.f;
    };
    auto at_q = [&](int i, int c) -> float {
        return i < len ? to_f32(q[((size_t)(tok0 + i) * H + h) * DK + c]) : 0.f;
    };
    auto at_v = [&](int i, int c) -> float {
        return i < len ? to_f32(v[((size_t)(tok0 + i) * H + h) * DV + c]) : 0.f;
    };

    // gate [LA-KDA §5.4] and in-chunk cumulative sum; positions past the end
    // of the sequence get g = 0 (alpha = 1) and beta = 0 (no write)
    const bool gated = mode != kModeDeltaNet;
    const float ea = gated ? expf(A[h]) : 1.f;
    for (int c = tid; c < DK; c += 256) {
        float run = 0.f;
        for (int i = 0; i < C; i++) {
            if (gated && i < len) run += log_decay<true>(ea, z[((size_t)(tok0 + i) * H + h) * DK + c]);
            sG[i][c] = run;
        }
    }
    for (int i = tid; i < C; i += 256)
        sBeta[i] = i < len ? sigmoid_f<true>(bl[(size_t)(tok0 + i) * H + h]) : 0.f;
    __syncthreads();

    for (int idx = tid; idx < C * C; idx += 256) {
        const int i = idx / C, j = idx % C;
        float akk = 0.f, aqk = 0.f;
        if (j <= i) {
            for (int c = 0; c < DK; c++) {
                const float kj = at_k(j, c) * expf(sG[i][c] - sG[j][c]);
                akk += at_k(i, c) * kj;
                aqk += at_q(i, c) * kj;
            }
        }
        if (mode == kModeGLA) akk = 0.f;
        sAkk[i][j] = j < i ? sBeta[i] * akk : 0.f;
        rec[R::A + idx] = aqk;
        if (dbg) {
            float* d = dbg + ((size_t)cid * H + h) * ((size_t)C * DK + 3 * C * C);
            d[(size_t)C * DK + idx] = j < i ? sBeta[i] * akk : 0.f;
            d[(size_t)C * DK + C * C + idx] = aqk;
        }
    }
    __syncthreads();

    // N = (I + A_kk)^{-1}: column j by forward substitution (unit diagonal)
    for (int j = tid; j < C; j += 256) {
        for (int i = 0; i < C; i++) {
            float acc = i == j ? 1.f : 0.f;
            for (int m = j; m < i; m++) acc -= sAkk[i][m] * sN[m][j];
            sN[i][j] = i < j ? 0.f : acc;
        }
    }
    __syncthreads();

    for (int idx = tid; idx < C * DK; idx += 256) {
        const int i = idx / DK, c = idx % DK;
        float acc = 0.f;
        if (mode != kModeGLA)
            for (int j = 0; j <= i; j++) acc += sN[i][j] * sBeta[j] * at_k(j, c) * expf(sG[j][c]);
        rec[R::W + idx] = acc;
        rec[R::Q + idx] = at_q(i, c) * expf(sG[i][c]);
        rec[R::K + idx] = at_k(i, c) * expf(sG[C - 1][c] - sG[i][c]);
    }
    for (int idx = tid; idx < C * DV; idx += 256) {
        const int i = idx / DV, c = idx % DV;
        float acc = 0.f;
        for (int j = 0; j <= i; j++) acc += sN[i][j] * sBeta[j] * at_v(j, c);
        rec[R::U + idx] = acc;
    }
    for (int c = tid; c < DK; c += 256) rec[R::G + c] = expf(sG[C - 1][c]);
    if (dbg) {
        float* d = dbg + ((size_t)cid * H + h) * ((size_t)C * DK + 3 * C * C);
        for (int idx = tid; idx < C * DK; idx += 256) d[idx] = sG[idx / DK][idx % DK];
        for (int idx = tid; idx < C * C; idx += 256)
            d[(size_t)C * DK + 2 * C * C + idx] = sN[idx / C][idx % C] * sBeta[idx % C];
    }
}

// The chain over a sequence's chunks.  Columns of the state evolve
// independently (V~, O and the update of column j read only column j of S and
// of U), so one workgroup per (sequence, head, 16-column slice) carries its
// slice of S in LDS and reads the chunk's W, Q, Kbar, A and gamma rows whole
// (shared through L2 by the slices of one head).  Each thread produces four
// adjacent columns of a row; every sum runs in the same order as the plain
// definition: U - sum_c W S, sum_c Q S + sum_m A V~, gamma S + sum_i Kbar V~.
constexpr int kGenCS = 16;      // state columns per workgroup

template <int DK, int DV, int C, typename Tin>
__global__ __launch_bounds__(256)
void gen_chain_kernel(const float* __restrict__ recs, const int2* __restrict__ seqs,
                      const int4* __restrict__ chunks, const float* __restrict__ h0,
                      int H, Tin* __restrict__ o, float* __restrict__ hT,
                      float* __restrict__ dbgS)
{
    using R = GenRec<DK, DV, C>;
    constexpr int CS = DV < kGenCS ? DV : kGenCS, NSL = DV / CS, Q4 = CS / 4;
    const int p = blockIdx.x / NSL, j0 = (blockIdx.x % NSL) * CS;   // (sequence * H + head, slice)
    const int n = p / H, h = p % H;
    const int tid = threadIdx.x;

    __shared__ __align__(16) float sS[DK][CS];
    __shared__ __align__(16) float sVt[C][CS];

    for (int idx = tid; idx < DK * CS; idx += 256) {
        const int c = idx / CS, j = idx % CS;
        sS[c][j] = h0 ? h0[(size_t)p * DK * DV + (size_t)c * DV + j0 + j] : 0.f;
    }

    const int2 sd = seqs[n];
    for (int ci = 0; ci < sd.y; ci++) {
        const int cid = sd.x + ci;
        const int4 cd = chunks[cid];
        const int tok0 = cd.y, len = cd.z;
        const float* rec = recs + ((size_t)cid * H + h) * R::FLOATS;
        __syncthreads();
        if (dbgS)
            for (int idx = tid; idx < DK * CS; idx += 256) {
                const int c = idx / CS, j = idx % CS;
                dbgS[((size_t)cid * H + h) * DK * DV + (size_t)c * DV + j0 + j] = sS[c][j];
            }
        // V~ = U - W S (rows i, columns 4q .. 4q + 3 of the slice)
        for (int item = tid; item < C * Q4; item += 256) {
            const int i = item / Q4, jq = 4 * (item % Q4);
            const float* Ur = rec + R::U + (size_t)i * DV + j0 + jq;
            float4 acc = make_float4(Ur[0], Ur[1], Ur[2], Ur[3]);
            const float* Wr = rec + R::W + (size_t)i * DK;
            for (int c4 = 0; c4 < DK; c4 += 4) {
                const float4 w = *reinterpret_cast<const float4*>(Wr + c4);
                const float wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float4 sv = *reinterpret_cast<const float4*>(&sS[c4 + e][jq]);
                    acc.x -= wv[e] * sv.x; acc.y -= wv[e] * sv.y;
                    acc.z -= wv[e] * sv.z; acc.w -= wv[e] * sv.w;
                }
            }
            *reinterpret_cast<float4*>(&sVt[i][jq]) = acc;
        }
        __syncthreads();
        // O = (Q . Gamma) S + A_qk V~
        for (int item = tid; item < C * Q4; item += 256) {
            const int i = item / Q4, jq = 4 * (item % Q4);
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            const float* Qr = rec + R::Q + (size_t)i * DK;
            for (int c4 = 0; c4 < DK; c4 += 4) {
                const float4 qv = *reinterpret_cast<const float4*>(Qr + c4);
                const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const float4 sv = *reinterpret_cast<const float4*>(&sS[c4 + e][jq]);
                    acc.x += qa[e] * sv.x; acc.y += qa[e] * sv.y;
                    acc.z += qa[e] * sv.z; acc.w += qa[e] * sv.w;
                }
            }
            const float* Ar = rec + R::A + (size_t)i * C;
            for (int m = 0; m <= i; m++) {
                const float a = Ar[m];
                const float4 vv = *reinterpret_cast<const float4*>(&sVt[m][jq]);
                acc.x += a * vv.x; acc.y += a * vv.y; acc.z += a * vv.z; acc.w += a * vv.w;
            }
            if (i < len) {
                Tin* orow = o + ((size_t)(tok0 + i) * H + h) * DV + j0 + jq;
                orow[0] = from_f32<Tin>(acc.x); orow[1] = from_f32<Tin>(acc.y);
                orow[2] = from_f32<Tin>(acc.z); orow[3] = from_f32<Tin>(acc.w);
            }
        }
        __syncthreads();
        // S <- Diag(gamma_C) S + Kbar^T V~
        for (int item = tid; item < DK * Q4; item += 256) {
            const int c = item / Q4, jq = 4 * (item % Q4);
            const float g = rec[R::G + c];
            const float4 s0 = *reinterpret_cast<const float4*>(&sS[c][jq]);
            float4 acc = make_float4(g * s0.x, g * s0.y, g * s0.z, g * s0.w);
            for (int i = 0; i < C; i++) {
                const float kb = rec[R::K + (size_t)i * DK + c];
                const float4 vv = *reinterpret_cast<const float4*>(&sVt[i][jq]);
                acc.x += kb * vv.x; acc.y += kb * vv.y; acc.z += kb * vv.z; acc.w += kb * vv.w;
            }
            *reinterpret_cast<float4*>(&sS[c][jq]) = acc;
        }
    }
    __syncthreads();
    if (hT)
        for (int idx = tid; idx < DK * CS; idx += 256) {
            const int c = idx / CS, j = idx % CS;
            hT[(size_t)p * DK * DV + (size_t)c * DV + j0 + j] = sS[c][j];
        }
}

template <int D, int C, typename Tin>
hipError_t launch_generic_t(const ChunkArgs& a) {
    const int* hdr = reinterpret_cast<const int*>(a.ws);
    const int4* chunks = reinterpret_cast<const int4*>(a.ws + a.L.off_chunks);
    const int2* seqs = reinterpret_cast<const int2*>(a.ws + a.L.off_seqs);
    float* recs = reinterpret_cast<float*>(a.ws + a.L.off_recs);
    hipLaunchKernelGGL((gen_intra_kernel<D, D, C, Tin>), dim3((unsigned)a.L.cap, (unsigned)a.H),
                       dim3(256), 0, a.stream, (const Tin*)a.q, (const Tin*)a.k, (const Tin*)a.v,
                       a.z, a.b, a.A, hdr, chunks, a.H, recs, a.dbg_intra, a.mode);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev && (e = hipEventRecord(a.ev[2], a.stream)) != hipSuccess) return e;
    constexpr int NSL = D < kGenCS ? 1 : D / kGenCS;          // column slices per (sequence, head)
    if ((long long)a.N * a.H * NSL > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gen_chain_kernel<D, D, C, Tin>), dim3((unsigned)((long long)a.N * a.H * NSL)),
                       dim3(256), 0, a.stream, (const float*)recs, seqs, chunks, a.h0, a.H,
                       (Tin*)a.o, a.hT, a.dbg_state);
    return hipGetLastError();
}

}  // namespace

bool generic_supported(int dk, int dv, int C) {
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128) && (C == 16 || C == 64);
}

hipError_t launch_generic(const ChunkArgs& a, int dtype_bf16) {
#define KDA_GEN(D, CC)                                                                   \
    if (a.dk == D && a.C == CC)                                                          \
        return dtype_bf16 ? launch_generic_t<D, CC, bf16>(a) : launch_generic_t<D, CC, float>(a);
    KDA_GEN(16, 16) KDA_GEN(32, 16) KDA_GEN(64, 16) KDA_GEN(128, 16)
    KDA_GEN(16, 64) KDA_GEN(32, 64) KDA_GEN(64, 64) KDA_GEN(128, 64)
#undef KDA_GEN
    return hipErrorInvalidValue;
}

}  // namespace kda
