// C ABI of libkda: argument validation, workspace sizing and dispatch.
// Declarations and the contract of every entry point are in include/kda.h.
#include <initializer_list>
#include "../../include/kda.h"
#include "kda_internal.hpp"

#include <mutex>

using namespace kda;

// Scratch memory of kda_chunk_fwd_noalloc, for callers that cannot allocate:
// a file-scope device array, so that every GPU the library runs on holds its
// own copy from the module's load until the process ends.  In host code the
// name `scratch` is a host-side stand-in, never a device address: the device
// address of each GPU's copy comes from hipGetSymbolAddress (noalloc_scratch
// below) and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {

// per device: the address of that device's `scratch`, looked up once with
// the device current (guarded by a mutex; later calls only read the table)
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

hipError_t noalloc_scratch(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

bool dtype_ok(kda_dtype_t d) { return d == KDA_F32 || d == KDA_BF16; }

// every pointer given that is not NULL is 16-byte aligned, as the header
// requires of tensor pointers: the kernels move rows with 16-byte loads,
// stores and direct-to-LDS copies, so a misaligned tensor is refused here,
// before anything is enqueued
bool aligned16(std::initializer_list<const void*> ps) {
    for (const void* p : ps)
        if (reinterpret_cast<uintptr_t>(p) & 15) return false;
    return true;
}

bool mode_ok(int m) { return m == kModeKDA || m == kModeGLA || m == kModeDeltaNet; }
static_assert(KDA_MODE_KDA == kModeKDA && KDA_MODE_GLA == kModeGLA &&
              KDA_MODE_DELTANET == kModeDeltaNet, "mode numbering of the ABI and the kernels");

bool chunk_shape_supported(int dk, int dv, int chunk) { return generic_supported(dk, dv, chunk); }

// A dispatch's grid size (workgroups x threads) is a 32-bit work-item count.
constexpr long long kMaxWorkItems = 0xFFFFFFFFLL;
bool items_ok(long long blocks, long long threads) { return blocks * threads <= kMaxWorkItems; }

// sizes shared by the prefill entry points; false on invalid arguments
bool prefill_sizes_ok(int B, int T, int H, int dk, int dv, int N, int chunk) {
    if (B < 1 || T < 0 || H < 1 || dk < 1 || dv < 1 || N < 0 || chunk < 1) return false;
    if ((long long)B * T > 0x7fffffffLL) return false;            // token index fits int32
    if ((long long)N * H > 0x7fffffffLL) return false;
    const int cap = chunk_capacity(B, T, N, chunk);
    if (cap < 0) return false;
    // one workgroup per (chunk, head) (256 threads) and per (segment, head)
    // (at most 512 threads; at most twice as many segments as chunks); per
    // (sequence, head) the fp32 chain runs up to 8 column slices and the
    // composition 8 of 256 threads
    if (!items_ok((long long)cap * H, 1024) || !items_ok((long long)N * H, 2048)) return false;
    // the intra kernels address a chunk's rows with 32-bit offsets
    return (long long)H * (dk > dv ? dk : dv) * chunk <= kMaxWorkItems;
}

// decode-type launches: one workgroup of at most 256 threads per (sequence, head)
bool nh_ok(int N, int H) { return items_ok((long long)N * H, 256); }

kda_status_t run_prefill(const void* q, const void* k, const void* v, const float* z,
                         const float* b, const float* A, const float* h0, const int* cu,
                         int B, int T, int H, int dk, int dv, int N, int chunk,
                         kda_dtype_t dtype, void* o, float* hT, void* ws, size_t ws_bytes,
                         float* dbg_intra, float* dbg_state, hipEvent_t* ev, int n_ev,
                         void* stream, const void* gate = nullptr, const float* norm_w = nullptr,
                         float rms_eps = 0.f, const float* conv_w = nullptr,
                         const void* conv_state0 = nullptr, float l2_eps = 0.f,
                         int mode = kModeKDA) {
    if (!dtype_ok(dtype) || !mode_ok(mode)) return KDA_ERR_INVALID_ARG;
    if (!prefill_sizes_ok(B, T, H, dk, dv, N, chunk)) return KDA_ERR_INVALID_ARG;
    if (cu) {
        if (B != 1) return KDA_ERR_INVALID_ARG;
    } else if (N != B) {
        return KDA_ERR_INVALID_ARG;
    }
    if (!chunk_shape_supported(dk, dv, chunk)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    const long long tokens = (long long)B * T;
    const bool gated = mode != kModeDeltaNet;    // DeltaNet reads no gate logits
    if (tokens > 0 && (!q || !k || !v || (gated && !z) || !b || !o)) return KDA_ERR_INVALID_ARG;
    if (gated && !A) return KDA_ERR_INVALID_ARG;
    if (!aligned16({q, k, v, z, o, h0, hT, gate, conv_w, conv_state0})) return KDA_ERR_INVALID_ARG;
    const bool fast = use_fast_path(dk, dv, chunk, dtype == KDA_BF16);
    const WsLayout L = ws_layout(B, T, H, dk, dv, N, chunk, fast);
    if (L.total == 0) return KDA_ERR_INVALID_ARG;
    if (!ws || ws_bytes < L.total) return KDA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return KDA_ERR_WORKSPACE;

    ChunkArgs a{};
    a.q = q; a.k = k; a.v = v; a.z = z; a.b = b; a.A = A; a.h0 = h0; a.cu = cu;
    a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv; a.N = N; a.C = chunk;
    a.o = o; a.hT = hT; a.ws = static_cast<uint8_t*>(ws); a.L = L;
    a.dbg_intra = dbg_intra; a.dbg_state = dbg_state; a.ev = ev;
    a.ev5 = (ev && n_ev >= 6) ? ev + 4 : nullptr;
    a.stream = static_cast<hipStream_t>(stream);
    a.gate = fast ? gate : nullptr;
    a.norm_w = norm_w;
    a.rms_eps = rms_eps;
    a.conv_w = fast ? conv_w : nullptr;
    a.conv_state0 = conv_state0;
    a.l2_eps = l2_eps;
    a.mode = mode;
    // equal-length sequences on the MFMA path: the bookkeeping is planned here
    // and written by the intra launch (no launch of its own)
    if (fast && !cu) a.fx = plan_fixed(N, T, chunk, H, L, a.ws);
    hipError_t e = ev ? hipEventRecord(ev[0], a.stream) : hipSuccess;
    if (e == hipSuccess && !a.fx.on) e = launch_prep(a);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], a.stream);
    if (e == hipSuccess) e = fast ? launch_fast(a) : launch_generic(a, dtype == KDA_BF16);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[3], a.stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// workspace of the layer entry point: the core's, then q, k, v after the
// convolution and o before the output gate (dtype, [B*T, H, d] each)
struct LayerWs {
    size_t core, row_bytes, total;
};

LayerWs layer_ws(int B, int T, int H, int d, int N, int chunk, kda_dtype_t dtype) {
    LayerWs w{0, 0, 0};
    if (!dtype_ok(dtype) || !prefill_sizes_ok(B, T, H, d, d, N, chunk)) return w;
    if (!chunk_shape_supported(d, d, chunk)) return w;
    const bool fast = use_fast_path(d, d, chunk, dtype == KDA_BF16);
    // the fp32 path's convolution and output-gate passes: 64 threads per row
    if (!fast && !items_ok(((long long)B * T * H + 3) / 4, 256)) return w;
    const WsLayout L = ws_layout(B, T, H, d, d, N, chunk, fast);
    if (L.total == 0) return w;
    w.core = align256(L.total);
    w.row_bytes = align256((size_t)B * T * H * d * (dtype == KDA_BF16 ? 2 : 4));
    w.total = w.core + 4 * w.row_bytes;
    return w;
}

bool eps_ok(float e) { return e >= 0.f && e < 1e30f; }

}  // namespace

extern "C" {

const char* kda_status_string(kda_status_t s) {
    switch (s) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG: invalid argument (a NULL or misaligned pointer, or a size out of range)";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: shape or dtype not supported";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing, too small or misaligned";
        case KDA_ERR_HIP: return "KDA_ERR_HIP: kernel launch failed";
        case KDA_ERR_SCRATCH:
            return "KDA_ERR_SCRATCH: the call needs more scratch than kda_chunk_fwd_noalloc holds "
                   "(KDA_NOALLOC_SCRATCH_BYTES); use kda_chunk_fwd with a workspace";
    }
    return "KDA_ERR_UNKNOWN";
}

int kda_chunk_fwd_supported(int dk, int dv, int chunk, kda_dtype_t dtype) {
    return dtype_ok(dtype) && chunk_shape_supported(dk, dv, chunk) ? 1 : 0;
}

int kda_recurrent_step_supported(int dk, int dv, kda_dtype_t dtype) {
    return dtype_ok(dtype) && decode_supported(dk, dv) ? 1 : 0;
}

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N, int chunk,
                                     kda_dtype_t dtype) {
    if (!dtype_ok(dtype) || !prefill_sizes_ok(B, T, H, dk, dv, N, chunk)) return 0;
    if (!chunk_shape_supported(dk, dv, chunk)) return 0;
    const bool fast = use_fast_path(dk, dv, chunk, dtype == KDA_BF16);
    return ws_layout(B, T, H, dk, dv, N, chunk, fast).total;
}

size_t kda_chunk_fwd_debug_floats(int B, int T, int H, int dk, int dv, int N, int chunk,
                                  size_t* dbg_state_floats, int* chunk_capacity_out) {
    if (!prefill_sizes_ok(B, T, H, dk, dv, N, chunk)) return 0;
    const int cap = chunk_capacity(B, T, N, chunk);
    if (dbg_state_floats) *dbg_state_floats = (size_t)cap * H * dk * dv;
    if (chunk_capacity_out) *chunk_capacity_out = cap;
    return (size_t)cap * H * ((size_t)chunk * dk + 3 * (size_t)chunk * chunk);
}

kda_status_t kda_chunk_fwd(const void* q, const void* k, const void* v, const float* g_logits,
                           const float* beta_logits, const float* A, const float* h0,
                           const int* cu_seqlens, int B, int T, int H, int dk, int dv, int N,
                           int chunk, kda_dtype_t dtype, void* o, float* hT, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return run_prefill(q, k, v, g_logits, beta_logits, A, h0, cu_seqlens, B, T, H, dk, dv, N,
                       chunk, dtype, o, hT, workspace, workspace_bytes, nullptr, nullptr, nullptr, 0,
                       stream);
}

kda_status_t kda_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                   const float* g_logits, const float* beta_logits, const float* A,
                                   const float* h0, const int* cu_seqlens, int B, int T, int H,
                                   int dk, int dv, int N, int chunk, kda_dtype_t dtype, void* o,
                                   float* hT, void* stream) {
    // the workspace the same call of kda_chunk_fwd would need (0: the sizes
    // are invalid or unsupported, which run_prefill reports before it looks
    // at the scratch)
    const size_t need = kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, chunk, dtype);
    if (need > KDA_NOALLOC_SCRATCH_BYTES) return KDA_ERR_SCRATCH;
    void* ws = nullptr;
    if (need > 0 && N > 0 && noalloc_scratch(&ws) != hipSuccess) return KDA_ERR_HIP;
    return run_prefill(q, k, v, g_logits, beta_logits, A, h0, cu_seqlens, B, T, H, dk, dv, N,
                       chunk, dtype, o, hT, ws, ws ? (size_t)KDA_NOALLOC_SCRATCH_BYTES : 0,
                       nullptr, nullptr, nullptr, 0, stream);
}

kda_status_t kda_chunk_fwd_debug(const void* q, const void* k, const void* v,
                                 const float* g_logits, const float* beta_logits, const float* A,
                                 const float* h0, const int* cu_seqlens, int B, int T, int H,
                                 int dk, int dv, int N, int chunk, kda_dtype_t dtype, void* o,
                                 float* hT, void* workspace, size_t workspace_bytes,
                                 float* dbg_intra, float* dbg_state, void* stream) {
    return run_prefill(q, k, v, g_logits, beta_logits, A, h0, cu_seqlens, B, T, H, dk, dv, N,
                       chunk, dtype, o, hT, workspace, workspace_bytes, dbg_intra, dbg_state,
                       nullptr, 0, stream);
}

kda_status_t kda_chunk_fwd_timed(const void* q, const void* k, const void* v,
                                 const float* g_logits, const float* beta_logits, const float* A,
                                 const float* h0, const int* cu_seqlens, int B, int T, int H,
                                 int dk, int dv, int N, int chunk, kda_dtype_t dtype, void* o,
                                 float* hT, void* workspace, size_t workspace_bytes,
                                 void* const* events, int n_events, void* stream) {
    if (!events || n_events < 4) return KDA_ERR_INVALID_ARG;
    const int n = n_events >= 6 ? 6 : 4;
    hipEvent_t ev[6];
    for (int i = 0; i < n; i++) {
        if (!events[i]) return KDA_ERR_INVALID_ARG;
        ev[i] = static_cast<hipEvent_t>(events[i]);
    }
    return run_prefill(q, k, v, g_logits, beta_logits, A, h0, cu_seqlens, B, T, H, dk, dv, N,
                       chunk, dtype, o, hT, workspace, workspace_bytes, nullptr, nullptr, ev, n,
                       stream);
}

kda_status_t kda_recurrent_step_mode(const void* q, const void* k, const void* v,
                                     const float* g_logits, const float* beta_logits,
                                     const float* A, float* state, void* o, int N, int H, int dk,
                                     int dv, kda_dtype_t dtype, kda_mode_t mode, void* stream) {
    if (!dtype_ok(dtype) || !mode_ok(mode)) return KDA_ERR_INVALID_ARG;
    if (N < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_INVALID_ARG;
    if (!nh_ok(N, H)) return KDA_ERR_INVALID_ARG;
    if (!decode_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    const bool gated = mode != KDA_MODE_DELTANET;
    if (!q || !k || !v || (gated && (!g_logits || !A)) || !beta_logits || !state || !o)
        return KDA_ERR_INVALID_ARG;
    if (!aligned16({q, k, v, g_logits, state, o})) return KDA_ERR_INVALID_ARG;
    hipError_t e = launch_decode(q, k, v, g_logits, beta_logits, A, state, o, N, H, dk, dv,
                                 dtype == KDA_BF16, static_cast<hipStream_t>(stream), mode);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_recurrent_step(const void* q, const void* k, const void* v, const float* g_logits,
                                const float* beta_logits, const float* A, float* state, void* o,
                                int N, int H, int dk, int dv, kda_dtype_t dtype, void* stream) {
    return kda_recurrent_step_mode(q, k, v, g_logits, beta_logits, A, state, o, N, H, dk, dv,
                                   dtype, KDA_MODE_KDA, stream);
}

kda_status_t kda_chunk_fwd_mode(const void* q, const void* k, const void* v,
                                const float* g_logits, const float* beta_logits, const float* A,
                                const float* h0, const int* cu_seqlens, int B, int T, int H,
                                int dk, int dv, int N, int chunk, kda_dtype_t dtype,
                                kda_mode_t mode, void* o, float* hT, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return run_prefill(q, k, v, g_logits, beta_logits, A, h0, cu_seqlens, B, T, H, dk, dv, N,
                       chunk, dtype, o, hT, workspace, workspace_bytes, nullptr, nullptr, nullptr, 0,
                       stream, nullptr, nullptr, 0.f, nullptr, nullptr, 0.f, mode);
}

size_t kda_dplr_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int N, int chunk,
                                          kda_dtype_t dtype) {
    if (!dtype_ok(dtype) || !prefill_sizes_ok(B, T, H, dk, dv, N, chunk)) return 0;
    if (!chunk_shape_supported(dk, dv, chunk)) return 0;
    const bool fast = use_fast_path(dk, dv, chunk, dtype == KDA_BF16);
    return ws_layout(B, T, H, dk, dv, N, chunk, fast, true).total;
}

namespace {
kda_status_t run_dplr(const void* q, const void* k, const void* v, const void* a, const void* b,
                      const float* g_logits, const float* A, const float* h0,
                      const int* cu_seqlens, int B, int T, int H, int dk, int dv, int N, int chunk,
                      kda_dtype_t dtype, void* o, float* hT, void* workspace,
                      size_t workspace_bytes, hipEvent_t* ev, int n_ev, void* stream) {
    if (!dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
    if (!prefill_sizes_ok(B, T, H, dk, dv, N, chunk)) return KDA_ERR_INVALID_ARG;
    if (cu_seqlens ? B != 1 : N != B) return KDA_ERR_INVALID_ARG;
    if (!chunk_shape_supported(dk, dv, chunk)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    if ((long long)B * T > 0 && (!q || !k || !v || !a || !b || !g_logits || !o))
        return KDA_ERR_INVALID_ARG;
    if (!A) return KDA_ERR_INVALID_ARG;
    if (!aligned16({q, k, v, a, b, g_logits, o, h0, hT})) return KDA_ERR_INVALID_ARG;
    const bool fast = use_fast_path(dk, dv, chunk, dtype == KDA_BF16);
    const WsLayout L = ws_layout(B, T, H, dk, dv, N, chunk, fast, true);
    if (L.total == 0) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < L.total) return KDA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return KDA_ERR_WORKSPACE;
    ChunkArgs c{};
    c.q = q; c.k = k; c.v = v; c.la = a; c.lb = b; c.z = g_logits; c.A = A; c.h0 = h0;
    c.cu = cu_seqlens;
    c.B = B; c.T = T; c.H = H; c.dk = dk; c.dv = dv; c.N = N; c.C = chunk;
    c.o = o; c.hT = hT; c.ws = static_cast<uint8_t*>(workspace); c.L = L;
    c.stream = static_cast<hipStream_t>(stream);
    c.ev = ev;
    c.ev5 = (ev && n_ev >= 6) ? ev + 4 : nullptr;
    hipError_t e = ev ? hipEventRecord(ev[0], c.stream) : hipSuccess;
    if (e == hipSuccess) e = launch_prep(c);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[1], c.stream);
    if (e == hipSuccess) e = fast ? launch_fast_dplr(c) : launch_dplr_generic(c, dtype == KDA_BF16);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[3], c.stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}
}  // namespace

kda_status_t kda_dplr_chunk_fwd(const void* q, const void* k, const void* v, const void* a,
                                const void* b, const float* g_logits, const float* A,
                                const float* h0, const int* cu_seqlens, int B, int T, int H,
                                int dk, int dv, int N, int chunk, kda_dtype_t dtype, void* o,
                                float* hT, void* workspace, size_t workspace_bytes, void* stream) {
    return run_dplr(q, k, v, a, b, g_logits, A, h0, cu_seqlens, B, T, H, dk, dv, N, chunk, dtype,
                    o, hT, workspace, workspace_bytes, nullptr, 0, stream);
}

kda_status_t kda_dplr_chunk_fwd_timed(const void* q, const void* k, const void* v, const void* a,
                                      const void* b, const float* g_logits, const float* A,
                                      const float* h0, const int* cu_seqlens, int B, int T, int H,
                                      int dk, int dv, int N, int chunk, kda_dtype_t dtype, void* o,
                                      float* hT, void* workspace, size_t workspace_bytes,
                                      void* const* events, int n_events, void* stream) {
    if (!events || n_events < 4) return KDA_ERR_INVALID_ARG;
    const int n = n_events >= 6 ? 6 : 4;
    hipEvent_t ev[6];
    for (int i = 0; i < n; i++) {
        if (!events[i]) return KDA_ERR_INVALID_ARG;
        ev[i] = static_cast<hipEvent_t>(events[i]);
    }
    return run_dplr(q, k, v, a, b, g_logits, A, h0, cu_seqlens, B, T, H, dk, dv, N, chunk, dtype,
                    o, hT, workspace, workspace_bytes, ev, n, stream);
}

kda_status_t kda_dplr_recurrent_step(const void* q, const void* k, const void* v, const void* a,
                                     const void* b, const float* g_logits, const float* A,
                                     float* state, void* o, int N, int H, int dk, int dv,
                                     kda_dtype_t dtype, void* stream) {
    if (!dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
    if (N < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_INVALID_ARG;
    if (!nh_ok(N, H)) return KDA_ERR_INVALID_ARG;
    if (!decode_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !a || !b || !g_logits || !A || !state || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned16({q, k, v, a, b, g_logits, state, o})) return KDA_ERR_INVALID_ARG;
    hipError_t e = launch_dplr_decode(q, k, v, a, b, g_logits, A, state, o, N, H, dk,
                                      dtype == KDA_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

size_t kda_layer_fwd_workspace_bytes(int B, int T, int H, int d, int N, int chunk,
                                     kda_dtype_t dtype) {
    return layer_ws(B, T, H, d, N, chunk, dtype).total;
}

kda_status_t kda_layer_fwd(const void* q_in, const void* k_in, const void* v_in,
                           const float* conv_w, const void* conv_state0, void* conv_stateT,
                           const float* g_logits, const float* beta_logits, const float* A,
                           const float* h0, const int* cu_seqlens, const void* gate,
                           const float* norm_w, float l2_eps, float rms_eps, int B, int T, int H,
                           int d, int N, int chunk, kda_dtype_t dtype, void* y, float* hT,
                           void* workspace, size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
    if (!prefill_sizes_ok(B, T, H, d, d, N, chunk)) return KDA_ERR_INVALID_ARG;
    if (cu_seqlens ? B != 1 : N != B) return KDA_ERR_INVALID_ARG;
    if (!eps_ok(l2_eps) || !eps_ok(rms_eps)) return KDA_ERR_INVALID_ARG;
    if (!chunk_shape_supported(d, d, chunk)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    const long long tokens = (long long)B * T;
    if (tokens > 0 && (!q_in || !k_in || !v_in || !g_logits || !beta_logits || !gate || !y))
        return KDA_ERR_INVALID_ARG;
    if (!A || !conv_w || !norm_w) return KDA_ERR_INVALID_ARG;
    if (!aligned16({q_in, k_in, v_in, conv_w, conv_state0, conv_stateT, g_logits, gate, y, h0, hT}))
        return KDA_ERR_INVALID_ARG;
    const LayerWs W = layer_ws(B, T, H, d, N, chunk, dtype);
    if (W.total == 0) return KDA_ERR_INVALID_ARG;
    if (!workspace || workspace_bytes < W.total) return KDA_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return KDA_ERR_WORKSPACE;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    void* qw = ws + W.core;
    void* kw = ws + W.core + W.row_bytes;
    void* vw = ws + W.core + 2 * W.row_bytes;
    void* ow = ws + W.core + 3 * W.row_bytes;
    const int bf = dtype == KDA_BF16;
    const int Ttot = (int)tokens;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // The MFMA path runs the steps before the core in its intra kernel and the
    // output gate in its output kernel; the fp32 path runs them as passes of
    // their own around the core.
    const bool fused = use_fast_path(d, d, chunk, bf);
    hipError_t e = hipSuccess;
    if (!fused)
        e = launch_layer_pre(q_in, k_in, v_in, conv_w, conv_state0, cu_seqlens, N, T, Ttot, H, d,
                             l2_eps, qw, kw, vw, bf, s);
    if (e != hipSuccess) return KDA_ERR_HIP;
    const kda_status_t st =
        fused ? run_prefill(q_in, k_in, v_in, g_logits, beta_logits, A, h0, cu_seqlens, B, T, H, d,
                            d, N, chunk, dtype, y, hT, ws, W.core, nullptr, nullptr, nullptr, 0,
                            stream, gate, norm_w, rms_eps, conv_w, conv_state0, l2_eps)
              : run_prefill(qw, kw, vw, g_logits, beta_logits, A, h0, cu_seqlens, B, T, H, d, d, N,
                            chunk, dtype, ow, hT, ws, W.core, nullptr, nullptr, nullptr, 0, stream);
    if (st != KDA_OK) return st;
    if (!fused) e = launch_layer_post(ow, gate, norm_w, rms_eps, tokens * H, d, y, bf, s);
    // after the core: conv_stateT may be conv_state0, which the intra kernel reads
    if (e == hipSuccess && conv_stateT)
        e = launch_layer_convstate(q_in, k_in, v_in, conv_state0, cu_seqlens, N, T, Ttot, H, d,
                                   conv_stateT, bf, s);
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_layer_step(const void* q_in, const void* k_in, const void* v_in,
                            const float* conv_w, void* conv_state, const float* g_logits,
                            const float* beta_logits, const float* A, float* state,
                            const void* gate, const float* norm_w, float l2_eps, float rms_eps,
                            void* y, int N, int H, int d, kda_dtype_t dtype, void* stream) {
    if (!dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
    if (N < 0 || H < 1 || d < 1) return KDA_ERR_INVALID_ARG;
    if (!nh_ok(N, H)) return KDA_ERR_INVALID_ARG;
    if (!eps_ok(l2_eps) || !eps_ok(rms_eps)) return KDA_ERR_INVALID_ARG;
    if (!decode_supported(d, d)) return KDA_ERR_UNSUPPORTED;
    if (N == 0) return KDA_OK;
    if (!q_in || !k_in || !v_in || !conv_w || !conv_state || !g_logits || !beta_logits || !A ||
        !state || !gate || !norm_w || !y)
        return KDA_ERR_INVALID_ARG;
    if (!aligned16({q_in, k_in, v_in, conv_w, conv_state, g_logits, state, gate, y}))
        return KDA_ERR_INVALID_ARG;
    hipError_t e = launch_layer_step(q_in, k_in, v_in, conv_w, conv_state, g_logits, beta_logits, A,
                                     state, gate, norm_w, l2_eps, rms_eps, y, N, H, d,
                                     dtype == KDA_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_recurrent_verify(const void* q, const void* k, const void* v,
                                  const float* g_logits, const float* beta_logits, const float* A,
                                  const float* state, void* o, int N, int W, int H, int dk, int dv,
                                  kda_dtype_t dtype, void* stream) {
    if (!dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
    if (N < 0 || W < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_INVALID_ARG;
    if (!nh_ok(N, H) || (long long)N * W * H > 0x7fffffffLL)
        return KDA_ERR_INVALID_ARG;
    if (!decode_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (N == 0 || W == 0) return KDA_OK;
    if (!q || !k || !v || !g_logits || !beta_logits || !A || !state || !o) return KDA_ERR_INVALID_ARG;
    if (!aligned16({q, k, v, g_logits, state, o})) return KDA_ERR_INVALID_ARG;
    hipError_t e = launch_verify(q, k, v, g_logits, beta_logits, A, state, o, N, W, H, dk, dv,
                                 dtype == KDA_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

kda_status_t kda_recurrent_fold(const void* k, const void* v, const float* g_logits,
                                const float* beta_logits, const float* A, const int* n_accept,
                                float* state, int N, int W, int H, int dk, int dv,
                                kda_dtype_t dtype, void* stream) {
    if (!dtype_ok(dtype)) return KDA_ERR_INVALID_ARG;
    if (N < 0 || W < 0 || H < 1 || dk < 1 || dv < 1) return KDA_ERR_INVALID_ARG;
    if (!nh_ok(N, H)) return KDA_ERR_INVALID_ARG;
    if (!decode_supported(dk, dv)) return KDA_ERR_UNSUPPORTED;
    if (N == 0 || W == 0) return KDA_OK;
    if (!k || !v || !g_logits || !beta_logits || !A || !n_accept || !state) return KDA_ERR_INVALID_ARG;
    if (!aligned16({k, v, g_logits, state})) return KDA_ERR_INVALID_ARG;
    hipError_t e = launch_fold(k, v, g_logits, beta_logits, A, n_accept, state, N, W, H, dk, dv,
                               dtype == KDA_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? KDA_OK : KDA_ERR_HIP;
}

}  // extern "C"
