// The steps either side of the recurrence that act on one token-head row,
// and the decode step with them fused in.
//
//   [LA-KDA §5.3]  q, k = L2Norm(Swish(ShortConv(W x))),  v = Swish(ShortConv(W x))
//   [LA-KDA §5.5]  y = W_o [Sigmoid(W_g x) * RMSNorm(o)], RMSNorm per head ([K3-ATTN §2.3])
//   [K3-ATTN §6.3] the decode launch runs causal conv -> recurrent update ->
//                  gated RMSNorm as one kernel
// Sources: [LA-KDA] "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制";
//          [K3-ATTN] "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构".
// The projections W are the caller's: these kernels take their outputs.
// ShortConv is depthwise and causal with four taps per channel, oldest
// first, no bias; a sequence's first three taps read its carried convolution
// state (zeros without one).  Swish has unit slope.  L2Norm and RMSNorm add
// their epsilon under the square root; RMSNorm's weight is one per channel,
// shared by the heads.
//
// Convolution state layout: [N][3 (q, k, v)][3 (inputs t-3, t-2, t-1)][H][d],
// in the input dtype, so a carried state replays its inputs exactly.
#include "kda_device.hpp"
#include "kda_internal.hpp"
#include "kda_step.hpp"

namespace kda {
namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// sequence of packed token t (offsets clamped as in the chunk bookkeeping)
__device__ __forceinline__ void token_seq(const int* cu, int N, int Tfix, int Ttot, int t, int& n,
                                          int& start, int& end) {
    if (!cu) {
        n = t / Tfix;
        start = n * Tfix;
        end = start + Tfix;
        return;
    }
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (min(max(cu[mid], 0), Ttot) <= t) lo = mid; else hi = mid - 1;
    }
    n = lo;
    start = min(max(cu[lo], 0), Ttot);
    end = min(max(cu[lo + 1], start), Ttot);
}

// one convolution output: taps j = 0..3 over inputs t-3+j, fma in tap order
__device__ __forceinline__ float conv4(const float* __restrict__ w, float x0, float x1, float x2,
                                       float x3) {
    float y = 0.f;
    y = __builtin_fmaf(w[0], x0, y);
    y = __builtin_fmaf(w[1], x1, y);
    y = __builtin_fmaf(w[2], x2, y);
    y = __builtin_fmaf(w[3], x3, y);
    return y;
}

__device__ __forceinline__ float swish(float x) { return x * sigmoid_f<true>(x); }

// Convolution, Swish and (q, k) L2Norm: one wave per (token, head) row, lane
// c and c + 64 hold channels; rows outside every sequence are skipped.
template <typename T>
__global__ __launch_bounds__(256)
void layer_pre_kernel(const T* __restrict__ q_in, const T* __restrict__ k_in,
                      const T* __restrict__ v_in, const float* __restrict__ conv_w,
                      const T* __restrict__ cs0, const int* __restrict__ cu, int N, int Tfix,
                      int Ttot, int H, int d, float l2_eps, T* __restrict__ q_out,
                      T* __restrict__ k_out, T* __restrict__ v_out)
{
#pragma clang fp contract(off)
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= (long long)Ttot * H) return;
    const int t = (int)(row / H), h = (int)(row % H);
    int n, start, end;
    token_seq(cu, N, Tfix, Ttot, t, n, start, end);
    if (t < start || t >= end) return;
    const int p = t - start;
#pragma unroll
    for (int which = 0; which < 3; which++) {
        const T* x = which == 0 ? q_in : which == 1 ? k_in : v_in;
        T* out = which == 0 ? q_out : which == 1 ? k_out : v_out;
        float val[2] = {0.f, 0.f}, ss = 0.f;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int c = lane + 64 * i;
            if (c < d) {
                float xs[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int src = p - 3 + j;
                    if (src >= 0)
                        xs[j] = to_f32(x[((size_t)(start + src) * H + h) * d + c]);
                    else
                        xs[j] = cs0 ? to_f32(cs0[((((size_t)n * 3 + which) * 3 + (3 + src)) * H + h) * d + c])
                                    : 0.f;
                }
                const float y = swish(conv4(conv_w + (((size_t)which * H + h) * d + c) * 4, xs[0], xs[1],
                                            xs[2], xs[3]));
                val[i] = y;
                ss = __builtin_fmaf(y, y, ss);
            }
        }
        float scale = 1.f;
        if (which < 2) scale = 1.f / sqrtf(wave_sum(ss) + l2_eps);
#pragma unroll
        for (int i = 0; i < 2; i++) {
            const int c = lane + 64 * i;
            if (c < d) out[((size_t)t * H + h) * d + c] = from_f32<T>(val[i] * scale);
        }
    }
}

// Outgoing convolution states: per (sequence, head) the last three inputs of
// q, k, v, reaching into the incoming state for sequences shorter than three.
// All reads happen before any write, so cs_out may be cs0 (in place).
template <typename T>
__global__ __launch_bounds__(256)
void layer_convstate_kernel(const T* __restrict__ q_in, const T* __restrict__ k_in,
                            const T* __restrict__ v_in, const T* cs0, const int* __restrict__ cu,
                            int Tfix, int Ttot, int H, int d, T* cs_out)
{
    const int n = blockIdx.x / H, h = blockIdx.x % H;
    int start, len;
    if (cu) {
        start = min(max(cu[n], 0), Ttot);
        len = min(max(cu[n + 1], start), Ttot) - start;
    } else {
        start = n * Tfix;
        len = Tfix;
    }
    constexpr int kMax = 5;                  // 9 d / 256 <= 4.5 for d <= 128
    T vals[kMax];
#pragma unroll
    for (int r = 0; r < kMax; r++) {
        const int idx = threadIdx.x + 256 * r;
        vals[r] = from_f32<T>(0.f);
        if (idx < 9 * d) {
            const int which = idx / (3 * d), j = (idx / d) % 3, c = idx % d;
            const T* x = which == 0 ? q_in : which == 1 ? k_in : v_in;
            const int src = len - 3 + j;
            if (src >= 0) vals[r] = x[((size_t)(start + src) * H + h) * d + c];
            else if (cs0) vals[r] = cs0[((((size_t)n * 3 + which) * 3 + (3 + src)) * H + h) * d + c];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kMax; r++) {
        const int idx = threadIdx.x + 256 * r;
        if (idx < 9 * d) {
            const int which = idx / (3 * d), j = (idx / d) % 3, c = idx % d;
            cs_out[((((size_t)n * 3 + which) * 3 + j) * H + h) * d + c] = vals[r];
        }
    }
}

// Output gate: y = sigma(g) * o / sqrt(mean(o^2) + eps) * w, one wave per row.
template <typename T>
__global__ __launch_bounds__(256)
void layer_post_kernel(const T* __restrict__ o, const T* __restrict__ gate,
                       const float* __restrict__ norm_w, float rms_eps, long long rows, int d,
                       T* __restrict__ y)
{
#pragma clang fp contract(off)
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    float ov[2] = {0.f, 0.f}, ss = 0.f;
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int c = lane + 64 * i;
        if (c < d) {
            ov[i] = to_f32(o[row * d + c]);
            ss = __builtin_fmaf(ov[i], ov[i], ss);
        }
    }
    const float r = 1.f / sqrtf(wave_sum(ss) / (float)d + rms_eps);
#pragma unroll
    for (int i = 0; i < 2; i++) {
        const int c = lane + 64 * i;
        if (c < d)
            y[row * d + c] = from_f32<T>(sigmoid_f<true>(to_f32(gate[row * d + c])) * (ov[i] * r) * norm_w[c]);
    }
}

// sum over the NT threads of a block (every thread gets the total)
template <int NT>
__device__ __forceinline__ float block_sum(float x, float* s_tmp) {
    if constexpr (NT >= 64) {
        x = wave_sum(x);
        if ((threadIdx.x & 63) == 0) s_tmp[threadIdx.x >> 6] = x;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < NT / 64; w++) tot += s_tmp[w];
        __syncthreads();
        return tot;
    } else {
        s_tmp[threadIdx.x] = x;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < NT; w++) tot += s_tmp[w];
        __syncthreads();
        return tot;
    }
}

// Decode with the layer's steps fused: convolution (state updated in place),
// Swish, L2Norm, the recurrent step of the decode kernel, gated RMSNorm.
template <int D, typename Tin>
__global__ __launch_bounds__((D / 4) * (D / 16))
void layer_step_kernel(const Tin* __restrict__ q_in, const Tin* __restrict__ k_in,
                       const Tin* __restrict__ v_in, const float* __restrict__ conv_w,
                       Tin* __restrict__ conv_state, const float* __restrict__ z,
                       const float* __restrict__ bl, const float* __restrict__ A,
                       float* __restrict__ state, const Tin* __restrict__ gate,
                       const float* __restrict__ norm_w, float l2_eps, float rms_eps,
                       Tin* __restrict__ y, int H)
{
#pragma clang fp contract(off)
    constexpr int NT = (D / 4) * (D / 16);
    const int nh = blockIdx.x, n = nh / H, h = nh % H;
    const int tid = threadIdx.x;
    float* S = state + (size_t)nh * D * D;
    __shared__ float s_in[3][D], s_o[D];
    __shared__ float s_al[D], s_k[D], s_q[D], s_qk[D / 16];
    __shared__ __align__(16) float s_red[2][D / 16][D];
    __shared__ float s_tmp[NT >= 64 ? NT / 64 : NT];

    // the token's inputs first (the convolution's carried rows, new input and
    // taps, the gate and beta logits), then the state stream that is the cost
    // of this kernel: the convolution and the norms wait on the former alone
    constexpr int KPT = TokenIn<D, D>::KPT;
    Tin xr[3][KPT][4];
    float wt[3][KPT][4], zr[KPT];
#pragma unroll
    for (int j = 0; j < KPT; j++) {
        const int i = tid + j * NT;
        zr[j] = 0.f;
        if (i < D) {
#pragma unroll
            for (int which = 0; which < 3; which++) {
                const Tin* x = which == 0 ? q_in : which == 1 ? k_in : v_in;
                const Tin* cs = conv_state + ((size_t)n * 3 + which) * 3 * H * D;
#pragma unroll
                for (int r = 0; r < 3; r++) xr[which][j][r] = cs[((size_t)r * H + h) * D + i];
                xr[which][j][3] = x[(size_t)nh * D + i];
#pragma unroll
                for (int r = 0; r < 4; r++) wt[which][j][r] = conv_w[(((size_t)which * H + h) * D + i) * 4 + r];
            }
            zr[j] = z[(size_t)nh * D + i];
        }
    }
    const float b_logit = bl[nh], ea = expf(A[h]);
    float4 Sv[16];
    load_state<D, D>(Sv, S);
#pragma unroll
    for (int j = 0; j < KPT; j++) {
        const int i = tid + j * NT;
        if (i < D) {
#pragma unroll
            for (int which = 0; which < 3; which++) {
                Tin* cs = conv_state + ((size_t)n * 3 + which) * 3 * H * D;
                s_in[which][i] = swish(conv4(wt[which][j], to_f32(xr[which][j][0]), to_f32(xr[which][j][1]),
                                             to_f32(xr[which][j][2]), to_f32(xr[which][j][3])));
#pragma unroll
                for (int r = 0; r < 3; r++) cs[((size_t)r * H + h) * D + i] = xr[which][j][r + 1];
            }
        }
    }
    __syncthreads();
    float sq = 0.f, sk = 0.f;
    for (int i = tid; i < D; i += NT) {
        sq = __builtin_fmaf(s_in[0][i], s_in[0][i], sq);
        sk = __builtin_fmaf(s_in[1][i], s_in[1][i], sk);
    }
    const float inv_q = 1.f / sqrtf(block_sum<NT>(sq, s_tmp) + l2_eps);
    const float inv_k = 1.f / sqrtf(block_sum<NT>(sk, s_tmp) + l2_eps);
    for (int i = tid; i < D; i += NT) {
        s_in[0][i] *= inv_q;
        s_in[1][i] *= inv_k;
    }
    __syncthreads();
    TokenIn<D, D> in;
#pragma unroll
    for (int j = 0; j < KPT; j++) {
        const int i = tid + j * NT;
        in.z[j] = in.k[j] = in.q[j] = 0.f;
        if (i < D) {
            in.z[j] = zr[j];
            in.k[j] = s_in[1][i];
            in.q[j] = s_in[0][i];
        }
    }
    const int c0 = StateLayout<D, D>::col0(tid);
#pragma unroll
    for (int c = 0; c < 4; c++) in.v[c] = s_in[2][c0 + c];
    in.b = b_logit;
    // each updated state row is stored as soon as it is formed
    kda_token_step<D, D, float, true, kModeKDA, true>(Sv, in, ea, s_o, s_al, s_k, s_q, s_red, s_qk, S);
    __syncthreads();
    float so = 0.f;
    for (int i = tid; i < D; i += NT) so = __builtin_fmaf(s_o[i], s_o[i], so);
    const float r = 1.f / sqrtf(block_sum<NT>(so, s_tmp) / (float)D + rms_eps);
    for (int i = tid; i < D; i += NT)
        y[(size_t)nh * D + i] =
            from_f32<Tin>(sigmoid_f<true>(to_f32(gate[(size_t)nh * D + i])) * (s_o[i] * r) * norm_w[i]);
}

}  // namespace

hipError_t launch_layer_pre(const void* q_in, const void* k_in, const void* v_in,
                            const float* conv_w, const void* cs0, const int* cu, int N, int Tfix,
                            int Ttot, int H, int d, float l2_eps, void* q_out, void* k_out,
                            void* v_out, int dtype_bf16, hipStream_t s) {
    const long long rows = (long long)Ttot * H;
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4));
#define KDA_PRE(T)                                                                          \
    hipLaunchKernelGGL(layer_pre_kernel<T>, grid, dim3(256), 0, s, (const T*)q_in,         \
                       (const T*)k_in, (const T*)v_in, conv_w, (const T*)cs0, cu, N, Tfix,   \
                       Ttot, H, d, l2_eps, (T*)q_out, (T*)k_out, (T*)v_out)
    if (dtype_bf16) KDA_PRE(bf16); else KDA_PRE(float);
#undef KDA_PRE
    return hipGetLastError();
}

hipError_t launch_layer_convstate(const void* q_in, const void* k_in, const void* v_in,
                                  const void* cs0, const int* cu, int N, int Tfix, int Ttot,
                                  int H, int d, void* cs_out, int dtype_bf16, hipStream_t s) {
    const dim3 grid((unsigned)((long long)N * H));
#define KDA_CS(T)                                                                           \
    hipLaunchKernelGGL(layer_convstate_kernel<T>, grid, dim3(256), 0, s, (const T*)q_in,   \
                       (const T*)k_in, (const T*)v_in, (const T*)cs0, cu, Tfix, Ttot, H,     \
                       d, (T*)cs_out)
    if (dtype_bf16) KDA_CS(bf16); else KDA_CS(float);
#undef KDA_CS
    return hipGetLastError();
}

hipError_t launch_layer_post(const void* o, const void* gate, const float* norm_w, float rms_eps,
                             long long rows, int d, void* y, int dtype_bf16, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4));
#define KDA_POST(T)                                                                         \
    hipLaunchKernelGGL(layer_post_kernel<T>, grid, dim3(256), 0, s, (const T*)o,           \
                       (const T*)gate, norm_w, rms_eps, rows, d, (T*)y)
    if (dtype_bf16) KDA_POST(bf16); else KDA_POST(float);
#undef KDA_POST
    return hipGetLastError();
}

hipError_t launch_layer_step(const void* q_in, const void* k_in, const void* v_in,
                             const float* conv_w, void* conv_state, const float* z, const float* b,
                             const float* A, float* state, const void* gate, const float* norm_w,
                             float l2_eps, float rms_eps, void* y, int N, int H, int d,
                             int dtype_bf16, hipStream_t s) {
#define KDA_LSTEP(D, T)                                                                     \
    hipLaunchKernelGGL((layer_step_kernel<D, T>), dim3((unsigned)N * H),                   \
                       dim3((D / 4) * (D / 16)), 0, s, (const T*)q_in, (const T*)k_in,      \
                       (const T*)v_in, conv_w, (T*)conv_state, z, b, A, state,               \
                       (const T*)gate, norm_w, l2_eps, rms_eps, (T*)y, H)
#define KDA_LSTEP_D(D)                                                                      \
    if (d == D) {                                                                           \
        if (dtype_bf16) KDA_LSTEP(D, bf16); else KDA_LSTEP(D, float);                       \
        return hipGetLastError();                                                           \
    }
    KDA_LSTEP_D(16) KDA_LSTEP_D(32) KDA_LSTEP_D(64) KDA_LSTEP_D(128)
#undef KDA_LSTEP_D
#undef KDA_LSTEP
    return hipErrorInvalidValue;
}

}  // namespace kda
