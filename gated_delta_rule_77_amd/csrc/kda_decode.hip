// Single-token KDA decode: one workgroup per (sequence, head) streams that
// head's fp32 state once in and once out.
//
// Math ([K3-ATTN §2.2], three steps without a d_k x d_k matrix; order of
// [LA-KDA §5.2]: decay, erase, write, read).  With S' = Diag(alpha) S:
//   p = S'^T k,  r = S'^T q          (one pass over S)
//   u = beta (v - p)                  (the corrected value)
//   S <- S' + k u^T                   (erase + write, in place)
//   o = S^T q = r + (q . k) u         (read after the update)
// Sources: [K3-ATTN] "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构";
//          [LA-KDA]  "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制".
//
// Layout: thread t owns rows [16*rg, 16*rg + 16) and columns [4*cg, 4*cg + 4)
// of the row-major [DK][DV] state (CG = DV/4 column groups, RG = DK/16 row
// groups).  A wave's loads cover whole 512-byte rows, so the stream is fully
// coalesced; every element is read and written by exactly one thread.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

template <int DK, int DV, typename Tin>
__global__ __launch_bounds__((DV / 4) * (DK / 16))
void decode_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                   const Tin* __restrict__ v, const float* __restrict__ z,
                   const float* __restrict__ bl, const float* __restrict__ A,
                   float* __restrict__ state, Tin* __restrict__ o, int H)
{
    constexpr int CG = DV / 4, RG = DK / 16, NT = CG * RG;
    const int nh = blockIdx.x;          // sequence * H + head
    const int h = nh % H;
    const int t = threadIdx.x;
    const int cg = t % CG, rg = t / CG;
    float* S = state + (size_t)nh * DK * DV;

    __shared__ float s_al[DK], s_k[DK], s_q[DK];
    __shared__ __align__(16) float s_red[2][RG][DV];

    // the state stream is the cost of this kernel: issue its loads first
    float4 Sv[16];
#pragma unroll
    for (int r = 0; r < 16; r++)
        Sv[r] = *reinterpret_cast<const float4*>(S + (size_t)(rg * 16 + r) * DV + cg * 4);

    const float ea = expf(A[h]);
    for (int i = t; i < DK; i += NT) {
        const size_t off = (size_t)nh * DK + i;
        s_al[i] = expf(log_decay<true>(ea, z[off]));
        s_k[i] = to_f32(k[off]);
        s_q[i] = to_f32(q[off]);
    }
    const float beta = sigmoid_f<true>(bl[nh]);
    float vj[4];
#pragma unroll
    for (int c = 0; c < 4; c++) vj[c] = to_f32(v[(size_t)nh * DV + cg * 4 + c]);
    __syncthreads();

    // partial S'^T k and S'^T q over this thread's 16 rows
    float p[4] = {0.f, 0.f, 0.f, 0.f}, r4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int i = rg * 16 + r;
        const float ka = s_al[i] * s_k[i], qa = s_al[i] * s_q[i];
        p[0] += ka * Sv[r].x; p[1] += ka * Sv[r].y; p[2] += ka * Sv[r].z; p[3] += ka * Sv[r].w;
        r4[0] += qa * Sv[r].x; r4[1] += qa * Sv[r].y; r4[2] += qa * Sv[r].z; r4[3] += qa * Sv[r].w;
    }
    *reinterpret_cast<float4*>(&s_red[0][rg][cg * 4]) = make_float4(p[0], p[1], p[2], p[3]);
    *reinterpret_cast<float4*>(&s_red[1][rg][cg * 4]) = make_float4(r4[0], r4[1], r4[2], r4[3]);
    __syncthreads();

    float P[4] = {0.f, 0.f, 0.f, 0.f}, R[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gidx = 0; gidx < RG; gidx++) {
        const float4 a = *reinterpret_cast<const float4*>(&s_red[0][gidx][cg * 4]);
        const float4 c = *reinterpret_cast<const float4*>(&s_red[1][gidx][cg * 4]);
        P[0] += a.x; P[1] += a.y; P[2] += a.z; P[3] += a.w;
        R[0] += c.x; R[1] += c.y; R[2] += c.z; R[3] += c.w;
    }
    float qk = 0.f;
#pragma unroll 8
    for (int i = 0; i < DK; i++) qk += s_q[i] * s_k[i];

    float u[4];
#pragma unroll
    for (int c = 0; c < 4; c++) u[c] = beta * (vj[c] - P[c]);
    if (rg == 0) {
#pragma unroll
        for (int c = 0; c < 4; c++)
            o[(size_t)nh * DV + cg * 4 + c] = from_f32<Tin>(R[c] + qk * u[c]);
    }
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int i = rg * 16 + r;
        const float al = s_al[i], ki = s_k[i];
        float4 n;
        n.x = al * Sv[r].x + ki * u[0];
        n.y = al * Sv[r].y + ki * u[1];
        n.z = al * Sv[r].z + ki * u[2];
        n.w = al * Sv[r].w + ki * u[3];
        *reinterpret_cast<float4*>(S + (size_t)i * DV + cg * 4) = n;
    }
}

bool decode_supported(int dk, int dv) {
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

template <int D, typename Tin>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* z,
                                  const float* b, const float* A, float* state, void* o,
                                  int N, int H, hipStream_t s) {
    constexpr int NT = (D / 4) * (D / 16);
    hipLaunchKernelGGL((decode_kernel<D, D, Tin>), dim3((unsigned)N * H), dim3(NT), 0, s,
                       (const Tin*)q, (const Tin*)k, (const Tin*)v, z, b, A, state, (Tin*)o, H);
    return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* z,
                         const float* b, const float* A, float* state, void* o,
                         int N, int H, int dk, int dv, int dtype_bf16, hipStream_t s) {
    (void)dv;
#define KDA_DEC(D)                                                                          \
    if (dk == D) return dtype_bf16                                                          \
        ? launch_decode_t<D, bf16>(q, k, v, z, b, A, state, o, N, H, s)                    \
        : launch_decode_t<D, float>(q, k, v, z, b, A, state, o, N, H, s);
    KDA_DEC(16) KDA_DEC(32) KDA_DEC(64) KDA_DEC(128)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

}  // namespace kda
