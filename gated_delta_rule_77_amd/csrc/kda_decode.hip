// Single-token KDA decode: one workgroup per (sequence, head) streams that
// head's fp32 state once in and once out.
//
// The step itself (kda_token_step) and the state's thread layout are in
// kda_step.hpp.  A wave's state loads cover whole 512-byte rows, so the
// stream is fully coalesced; every element is read and written by exactly
// one thread.
#include "kda_device.hpp"
#include "kda_internal.hpp"
#include "kda_step.hpp"

namespace kda {

template <int DK, int DV, typename Tin, int MODE>
__global__ __launch_bounds__((DV / 4) * (DK / 16))
void decode_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k,
                   const Tin* __restrict__ v, const float* __restrict__ z,
                   const float* __restrict__ bl, const float* __restrict__ A,
                   float* __restrict__ state, Tin* __restrict__ o, int H)
{
    const int nh = blockIdx.x;          // sequence * H + head
    float* S = state + (size_t)nh * DK * DV;
    __shared__ float s_al[DK], s_k[DK], s_q[DK], s_qk[DK / 16];
    __shared__ __align__(16) float s_red[2][DK / 16][DV];
    // the token's few inputs first, then the state stream that is the cost
    // of this kernel; the gate arithmetic waits on the former alone
    TokenIn<DK, DV> in;
    load_token<DK, DV, Tin, true, MODE>(in, k + (size_t)nh * DK, v + (size_t)nh * DV,
                                        MODE == kModeDeltaNet ? z : z + (size_t)nh * DK, bl[nh],
                                        q + (size_t)nh * DK);
    const float ea = MODE == kModeDeltaNet ? 1.f : expf(A[nh % H]);
    float4 Sv[16];
    load_state<DK, DV>(Sv, S);
    kda_token_step<DK, DV, Tin, true, MODE, true>(Sv, in, ea, o + (size_t)nh * DV, s_al, s_k, s_q,
                                                  s_red, s_qk, S);
}

// Replay fold ([K3-ATTN §6.2], ReplaySSM): advance each (sequence, head)
// state over the first n_accept[s] tokens of its stored window with exactly
// the decode step above, keeping the state in registers between tokens: one
// state read and one write for the whole window instead of one per token.
// Window layout: k, z [N, W, H, DK]; v [N, W, H, DV]; b [N, W, H].
template <int DK, int DV, typename Tin>
__global__ __launch_bounds__((DV / 4) * (DK / 16))
void fold_kernel(const Tin* __restrict__ k, const Tin* __restrict__ v, const float* __restrict__ z,
                 const float* __restrict__ bl, const float* __restrict__ A,
                 const int* __restrict__ n_accept, float* __restrict__ state, int W, int H)
{
    const int nh = blockIdx.x;          // sequence * H + head
    const int n = nh / H, h = nh % H;
    const int cnt = min(max(n_accept[n], 0), W);
    if (cnt == 0) return;
    float* S = state + (size_t)nh * DK * DV;
    __shared__ float s_al[DK], s_k[DK];
    __shared__ __align__(16) float s_red[2][DK / 16][DV];
    float4 Sv[16];
    load_state<DK, DV, false>(Sv, S);
    const float ea = expf(A[h]);
    for (int t = 0; t < cnt; t++) {
        const size_t tok = ((size_t)n * W + t) * H + h;
        if (t > 0) __syncthreads();     // the previous step's readers of s_al, s_k, s_red are done
        TokenIn<DK, DV> in;
        load_token<DK, DV, Tin, false, kModeKDA, false>(in, k + tok * DK, v + tok * DV, z + tok * DK,
                                                        bl[tok], (const Tin*)nullptr);
        kda_token_step<DK, DV, Tin, false, kModeKDA, false, false>(Sv, in, ea, (Tin*)nullptr, s_al,
                                                                   s_k, (float*)nullptr, s_red);
    }
    store_state<DK, DV, false>(Sv, S);
}

// One window token as loaded for a multi-token loop: the raw elements of
// TokenIn (converted when the step needs them), so that a token loaded a
// step ahead is waited for only where it is used.  Every thread loads
// (channel indices past DK are clamped and their values zeroed at use), so
// the loads are unconditional and the compiler's wait counts exact.
template <int DK, int DV, typename Tin> struct TokenRaw {
    static constexpr int KPT = TokenIn<DK, DV>::KPT;
    Tin k[KPT], q[KPT], v[4];
    float z[KPT], b;
};

template <int DK, int DV, typename Tin, bool WITH_Q>
__device__ __forceinline__ void load_token_raw(TokenRaw<DK, DV, Tin>& r, const Tin* __restrict__ kt,
                                               const Tin* __restrict__ vt, const float* __restrict__ zt,
                                               const float* __restrict__ bt, const Tin* __restrict__ qt) {
    using SL = StateLayout<DK, DV, false>;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < TokenRaw<DK, DV, Tin>::KPT; j++) {
        const int i = min(t + j * SL::NT, DK - 1);
        r.z[j] = zt[i];
        r.k[j] = kt[i];
        if (WITH_Q) r.q[j] = qt[i];
    }
    const int c0 = SL::col0(t);
#pragma unroll
    for (int c = 0; c < 4; c++) r.v[c] = vt[c0 + c];
    r.b = *bt;
}

template <int DK, int DV, typename Tin, bool WITH_Q>
__device__ __forceinline__ void cook_token(const TokenRaw<DK, DV, Tin>& r, TokenIn<DK, DV>& in) {
    using SL = StateLayout<DK, DV, false>;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < TokenIn<DK, DV>::KPT; j++) {
        const bool live = t + j * SL::NT < DK;
        in.z[j] = live ? r.z[j] : 0.f;
        in.k[j] = live ? to_f32(r.k[j]) : 0.f;
        in.q[j] = live && WITH_Q ? to_f32(r.q[j]) : 0.f;
    }
#pragma unroll
    for (int c = 0; c < 4; c++) in.v[c] = to_f32(r.v[c]);
    in.b = r.b;
}

// s_waitcnt immediate for "no vector memory operation outstanding" (vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
constexpr int kWaitVm0 = (7 << 4) | (15 << 8);

// Verify pass of the same draft window ([K3-ATTN §6.2]): from the checkpoint
// state, the outputs of every window token, with exactly the decode step
// above, the state held in registers and never written back (the accepted
// prefix is committed afterwards by the fold).  Window layout: q, k, z
// [N, W, H, DK]; v, o [N, W, H, DV]; b [N, W, H].  Token t + 1 is loaded
// during step t into the other of two register sets (the loop runs two
// tokens per turn, so no set is copied), and the state and token 0 have
// landed before the loop: the loop never waits on a load it does not use.
template <int DK, int DV, typename Tin>
__global__ __launch_bounds__((DV / 4) * (DK / 16))
void verify_kernel(const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
                   const float* __restrict__ z, const float* __restrict__ bl,
                   const float* __restrict__ A, const float* __restrict__ state,
                   Tin* __restrict__ o, int W, int H)
{
    const int nh = blockIdx.x;          // sequence * H + head
    const int n = nh / H, h = nh % H;
    if (W <= 0) return;
    __shared__ float s_al[DK], s_k[DK], s_q[DK], s_qk[DK / 16];
    __shared__ __align__(16) float s_red[2][DK / 16][DV];
    auto token = [&](TokenRaw<DK, DV, Tin>& r, int t) {     // index clamped into the window
        const size_t tok = ((size_t)n * W + min(t, W - 1)) * H + h;
        load_token_raw<DK, DV, Tin, true>(r, k + tok * DK, v + tok * DV, z + tok * DK, bl + tok, q + tok * DK);
    };
    TokenRaw<DK, DV, Tin> ra, rb;
    token(ra, 0);
    float4 Sv[16];
    load_state<DK, DV, false>(Sv, state + (size_t)nh * DK * DV);
    const float ea = expf(A[h]);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    for (int t = 0;; t += 2) {
        token(rb, t + 1);
        {
            if (t > 0) __syncthreads();
            TokenIn<DK, DV> in;
            cook_token<DK, DV, Tin, true>(ra, in);
            kda_token_step<DK, DV, Tin, true, kModeKDA, false, false>(Sv, in, ea,
                                                                      o + (((size_t)n * W + t) * H + h) * DV,
                                                                      s_al, s_k, s_q, s_red, s_qk);
        }
        if (t + 1 >= W) break;
        token(ra, t + 2);
        {
            __syncthreads();
            TokenIn<DK, DV> in;
            cook_token<DK, DV, Tin, true>(rb, in);
            kda_token_step<DK, DV, Tin, true, kModeKDA, false, false>(Sv, in, ea,
                                                                      o + (((size_t)n * W + t + 1) * H + h) * DV,
                                                                      s_al, s_k, s_q, s_red, s_qk);
        }
        if (t + 2 >= W) break;
    }
}

bool decode_supported(int dk, int dv) {
    return dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128);
}

template <int D, typename Tin>
static hipError_t launch_decode_t(const void* q, const void* k, const void* v, const float* z,
                                  const float* b, const float* A, float* state, void* o,
                                  int N, int H, hipStream_t s, int mode) {
    constexpr int NT = (D / 4) * (D / 16);
#define KDA_DEC_MODE(M)                                                                     \
    hipLaunchKernelGGL((decode_kernel<D, D, Tin, M>), dim3((unsigned)N * H), dim3(NT), 0, s, \
                       (const Tin*)q, (const Tin*)k, (const Tin*)v, z, b, A, state, (Tin*)o, H)
    if (mode == kModeGLA) KDA_DEC_MODE(kModeGLA);
    else if (mode == kModeDeltaNet) KDA_DEC_MODE(kModeDeltaNet);
    else KDA_DEC_MODE(kModeKDA);
#undef KDA_DEC_MODE
    return hipGetLastError();
}

hipError_t launch_decode(const void* q, const void* k, const void* v, const float* z,
                         const float* b, const float* A, float* state, void* o,
                         int N, int H, int dk, int dv, int dtype_bf16, hipStream_t s, int mode) {
    (void)dv;
#define KDA_DEC(D)                                                                          \
    if (dk == D) return dtype_bf16                                                          \
        ? launch_decode_t<D, bf16>(q, k, v, z, b, A, state, o, N, H, s, mode)              \
        : launch_decode_t<D, float>(q, k, v, z, b, A, state, o, N, H, s, mode);
    KDA_DEC(16) KDA_DEC(32) KDA_DEC(64) KDA_DEC(128)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

template <int D, typename Tin>
static hipError_t launch_verify_t(const void* q, const void* k, const void* v, const float* z,
                                  const float* b, const float* A, const float* state, void* o,
                                  int N, int W, int H, hipStream_t s) {
    constexpr int NT = (D / 4) * (D / 16);
    hipLaunchKernelGGL((verify_kernel<D, D, Tin>), dim3((unsigned)N * H), dim3(NT), 0, s,
                       (const Tin*)q, (const Tin*)k, (const Tin*)v, z, b, A, state, (Tin*)o, W, H);
    return hipGetLastError();
}

hipError_t launch_verify(const void* q, const void* k, const void* v, const float* z,
                         const float* b, const float* A, const float* state, void* o, int N,
                         int W, int H, int dk, int dv, int dtype_bf16, hipStream_t s) {
    (void)dv;
#define KDA_VER(D)                                                                          \
    if (dk == D) return dtype_bf16                                                          \
        ? launch_verify_t<D, bf16>(q, k, v, z, b, A, state, o, N, W, H, s)                 \
        : launch_verify_t<D, float>(q, k, v, z, b, A, state, o, N, W, H, s);
    KDA_VER(16) KDA_VER(32) KDA_VER(64) KDA_VER(128)
#undef KDA_VER
    return hipErrorInvalidValue;
}

template <int D, typename Tin>
static hipError_t launch_fold_t(const void* k, const void* v, const float* z, const float* b,
                                const float* A, const int* n_accept, float* state, int N, int W,
                                int H, hipStream_t s) {
    constexpr int NT = (D / 4) * (D / 16);
    hipLaunchKernelGGL((fold_kernel<D, D, Tin>), dim3((unsigned)N * H), dim3(NT), 0, s,
                       (const Tin*)k, (const Tin*)v, z, b, A, n_accept, state, W, H);
    return hipGetLastError();
}

hipError_t launch_fold(const void* k, const void* v, const float* z, const float* b,
                       const float* A, const int* n_accept, float* state, int N, int W, int H,
                       int dk, int dv, int dtype_bf16, hipStream_t s) {
    (void)dv;
#define KDA_FOLD(D)                                                                         \
    if (dk == D) return dtype_bf16                                                          \
        ? launch_fold_t<D, bf16>(k, v, z, b, A, n_accept, state, N, W, H, s)               \
        : launch_fold_t<D, float>(k, v, z, b, A, n_accept, state, N, W, H, s);
    KDA_FOLD(16) KDA_FOLD(32) KDA_FOLD(64) KDA_FOLD(128)
#undef KDA_FOLD
    return hipErrorInvalidValue;
}

}  // namespace kda
