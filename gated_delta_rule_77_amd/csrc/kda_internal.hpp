// Host-side declarations shared by the libkda translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// ---------------------------------------------------------------- workspace
//
// Chunks are numbered sequence by sequence in token order; `cap` bounds their
// number for both layouts: B*ceil(T/C) + N.  The full layout is given with
// ws_layout below.
struct WsLayout {
    int cap;                 // chunk capacity
    int seg_chunks;          // smallest chunks per segment of the MFMA chain (0 on the fp32 path)
    int seg_cap;             // segment capacity
    size_t off_chunks, off_seqs, off_seqsegs, off_segs, off_recs, rec_bytes;
    size_t off_sstart, off_rm, total;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline int chunk_capacity(int B, int T, int N, int C) {
    long long per = (T + (long long)C - 1) / C;
    long long cap = (long long)B * per + N;
    return cap > 0x7fffffffLL ? -1 : (int)cap;
}

// fp32 record of the generic path: W [C][DK], U [C][DV], Qg [C][DK],
// Kb [C][DK], Aqk [C][C], gamma_C [DK]
inline size_t generic_rec_floats(int dk, int dv, int C) {
    return (size_t)C * dk * 3 + (size_t)C * dv + (size_t)C * C + dk;
}

// fp32 record of the general DPLR path: Wb, Q . Gamma, A . dec, K . dec
// [C][DK] each, Ub [C][DV], A_qa and A_qk [C][C], gamma_C [DK]
constexpr size_t dplr_generic_rec_floats(int dk, int dv, int C) {
    return (size_t)C * dk * 4 + (size_t)C * dv + 2 * (size_t)C * C + dk;
}

// record of the MFMA path (bf16 operand fragments + fp32 gamma_C); offsets in
// bytes, see kda_chunk_fast.hip for the fragment orders
namespace fast {
constexpr int C = 64, DK = 128, DV = 128;
constexpr int REC_W = 0;        // -W^T fragments [4 token block][4 kstep][64 lane][8] bf16
constexpr int REC_Q = 16384;    // (Q . Gamma)^T fragments, same layout
constexpr int REC_K = 32768;    // Kbar^T fragments [4 row block][2 half][2 kstep][64 lane][8] bf16
constexpr int REC_U = 49152;    // U tiles [8 slice][4 token block][64 lane][4] bf16
constexpr int REC_A = 65536;    // A_qk row fragments [6 nonzero (token block, kstep)][64 lane][8] bf16
constexpr int REC_G = 71680;    // gamma_C [128] fp32
constexpr int REC_BYTES = 72192;
// A_qk is causal: token blocks 0 and 1 (rows 0..31) have no entry in k-step 1
// (columns 32..63), so only six of the eight row fragments are stored, in the
// order (0,0) (1,0) (2,0) (2,1) (3,0) (3,1)
__host__ __device__ constexpr int rec_a_frag(int tb, int kb) { return tb < 2 ? tb : 2 * tb - 2 + kb; }
__host__ __device__ constexpr bool rec_a_stored(int tb, int kb) { return tb >= 2 || kb == 0; }
static_assert(rec_a_frag(3, 1) == 5 && REC_A + 6 * 1024 == REC_G, "A_qk fragments fill the gap");
}  // namespace fast

// record of the MFMA path of the general DPLR update: what the chain needs
// with the S-independent terms folded in, X = Wb S, O = Q' S + Uo,
// S <- Diag(gamma_C) S + Abar^T X + Cs
namespace fast_dplr {
constexpr int RD_W = 0;         // Wb^T fragments, layout of REC_W (not negated)
constexpr int RD_Q = 16384;     // Q'^T fragments, layout of REC_Q
constexpr int RD_K = 32768;     // Abar^T fragments, layout of REC_K
constexpr int RD_U = 49152;     // Uo tiles, layout of REC_U
constexpr int RD_C = 65536;     // Cs tiles [8 row tile][8 slice][64 lane][4] bf16
constexpr int RD_G = 98304;     // gamma_C [128] fp32
constexpr int RD_BYTES = 98816;
}  // namespace fast_dplr

// record offsets by kind, for the chain kernels shared by both updates
template <bool DPLR> struct RecLayout;
template <> struct RecLayout<false> {
    static constexpr int W = fast::REC_W, Q = fast::REC_Q, K = fast::REC_K, U = fast::REC_U,
                         A = fast::REC_A, C = -1, G = fast::REC_G, BYTES = fast::REC_BYTES;
};
template <> struct RecLayout<true> {
    static constexpr int W = fast_dplr::RD_W, Q = fast_dplr::RD_Q, K = fast_dplr::RD_K,
                         U = fast_dplr::RD_U, A = -1, C = fast_dplr::RD_C, G = fast_dplr::RD_G,
                         BYTES = fast_dplr::RD_BYTES;
};

inline bool use_fast_path(int dk, int dv, int C, int dtype_bf16) {
    return dtype_bf16 && dk == 128 && dv == 128 && C == 64;
}

// Segments of the MFMA chain.  Both chain launches run one workgroup per
// (segment, head) and one workgroup fills a CU, so the segments of all
// sequences together should number about 256 / H: one full round of 256 CUs.
inline int seg_target(int H) { return H >= 256 ? 1 : 256 / H; }

// Smallest segment length (chunks) the device may pick: the target count on
// the whole capacity, and at least 8 chunks (512 tokens), below which the
// serial composition of segment starts costs more than the shorter chains
// save.  The device picks the length from the actual sequence lengths
// (prep_kernel; plan_fixed on the host for equal lengths), never below this,
// so cap / min + N segments always fit.
inline int pick_seg_chunks(int cap, int H) {
    const long long nseg = seg_target(H);
    long long per = (cap + nseg - 1) / nseg;
    if (per < 8) per = 8;
    if (per > cap) per = cap > 0 ? cap : 1;
    return (int)per;
}

// Workspace layout (all offsets 256-byte aligned):
// [0, 256)   header: int32 total chunks, int32 total segments, int32 chunks per segment
// chunks     cap x int4 (sequence, first token, length, position in sequence)
// seqs       N x int2 (first chunk id, number of chunks)
// seqsegs    N x int2 (first segment id, number of segments)      [MFMA path]
// segs       seg_cap x int4 (sequence, first chunk id, chunks, index in sequence)
// recs       cap x H chunk records of rec_bytes each, (chunk, head) order
// sstart     seg_cap x H x 128 x 128 fp32: state entering each segment
// rm         seg_cap x H x 128 x 256 fp32: [R | M] of each segment
inline WsLayout ws_layout(int B, int T, int H, int dk, int dv, int N, int C, bool fast,
                          bool dplr = false) {
    WsLayout L{};
    L.cap = chunk_capacity(B, T, N, C);
    if (L.cap < 0) { L.total = 0; return L; }
    const size_t n1 = (size_t)(N > 0 ? N : 1);
    L.off_chunks = 256;
    L.off_seqs = align_up(L.off_chunks + (size_t)L.cap * 16, 256);
    L.off_seqsegs = align_up(L.off_seqs + n1 * 8, 256);
    L.seg_chunks = fast ? pick_seg_chunks(L.cap, H) : 0;
    L.seg_cap = fast ? (L.cap + L.seg_chunks - 1) / L.seg_chunks + (N > 0 ? N : 1) : 0;
    L.off_segs = align_up(L.off_seqsegs + n1 * 8, 256);
    L.off_recs = align_up(L.off_segs + (size_t)L.seg_cap * 16, 256);
    L.rec_bytes = fast ? (size_t)(dplr ? fast_dplr::RD_BYTES : fast::REC_BYTES)
                : (dplr ? dplr_generic_rec_floats(dk, dv, C) : generic_rec_floats(dk, dv, C)) * 4;
    L.off_sstart = align_up(L.off_recs + (size_t)L.cap * H * L.rec_bytes, 256);
    L.off_rm = align_up(L.off_sstart + (size_t)L.seg_cap * H * 128 * 128 * 4, 256);
    L.total = L.off_rm + (size_t)L.seg_cap * H * 128 * 256 * 4;
    return L;
}

// Family modes ([LA-KDA §4] table): KDA; gated linear attention (the erase
// step off: S <- Diag(alpha) S + beta k v^T); DeltaNet (alpha = 1, the gate
// logits unread).
constexpr int kModeKDA = 0, kModeGLA = 1, kModeDeltaNet = 2;

// Chunk bookkeeping of N sequences of T tokens each (no cu_seqlens), planned
// on the host by the rule of the bookkeeping launch (kda_prep.hip): the intra
// launch then derives each workgroup's chunk from its index, and its
// workgroup 0 writes the tables the chain launches read, so that launch is
// not needed.
struct FixedPlan {
    int on;                          // 0: the tables come from the bookkeeping launch
    int N, T, C, cps;                // sequences, tokens each, chunk size, chunks each
    int total, per, nseg;            // chunks; chunks per segment; segments per sequence
    int nseg_total, cap, seg_cap;    // segments (clamped to seg_cap); capacities
    int* hdr; int2* seqs; int2* seqsegs; int4* chunks; int4* segs;   // workspace tables
};

// host: the plan of a batch without cu_seqlens on the MFMA path
FixedPlan plan_fixed(int N, int T, int C, int H, const WsLayout& L, uint8_t* ws);

// The tables of a fixed plan (the same values the bookkeeping launch
// writes), by the nt threads of one workgroup
__device__ inline void write_fixed_tables(const FixedPlan& p, int tid, int nt) {
    if (tid == 0) {
        p.hdr[0] = p.total;
        p.hdr[1] = p.nseg_total;
        p.hdr[2] = p.per;
    }
    for (int s = tid; s < p.N; s += nt) {
        p.seqs[s] = make_int2(s * p.cps, p.cps);
        const int f = min(s * p.nseg, p.seg_cap);
        p.seqsegs[s] = make_int2(f, max(0, min(p.nseg, p.seg_cap - f)));
    }
    for (int c = tid; c < p.cap; c += nt) {
        if (c >= p.total) {
            p.chunks[c] = make_int4(-1, 0, 0, 0);
        } else {
            const int n = c / p.cps, j = c - n * p.cps;
            p.chunks[c] = make_int4(n, n * p.T + j * p.C, min(p.C, p.T - j * p.C), j * p.C);
        }
    }
    for (int g = tid; g < p.seg_cap; g += nt) {
        if (g >= p.nseg_total) {
            p.segs[g] = make_int4(-1, 0, 0, 0);
        } else {
            const int n = g / p.nseg, j = g - n * p.nseg;
            p.segs[g] = make_int4(n, n * p.cps + j * p.per, min(p.per, p.cps - j * p.per), j);
        }
    }
}

struct ChunkArgs {
    const void* q; const void* k; const void* v;
    const float* z; const float* b; const float* A;
    const float* h0; const int* cu;
    int B, T, H, dk, dv, N, C;
    void* o; float* hT;
    uint8_t* ws; WsLayout L;
    float* dbg_intra; float* dbg_state;
    hipEvent_t* ev;            // 4 events recorded around the kernels, or null
    hipEvent_t* ev5;           // 2 more: after the transition and compose phases, or null
    hipStream_t stream;
    // MFMA path only: with a gate, o receives the layer's Sigmoid(gate) * RMSNorm(o);
    // with conv_w, q, k, v are the layer's projections (convolution, Swish and
    // L2Norm applied in the intra kernel)
    const void* gate; const float* norm_w; float rms_eps;
    const float* conv_w; const void* conv_state0; float l2_eps;
    int mode;                  // kModeKDA, kModeGLA or kModeDeltaNet
    const void* la; const void* lb;   // general DPLR only: the low-rank pair a, b [.., DK]
    FixedPlan fx;              // MFMA path without cu_seqlens: tables written by the intra launch
};

// launchers (return hipError_t of the launches)
hipError_t launch_prep(const ChunkArgs& a);
hipError_t launch_fast(const ChunkArgs& a);
hipError_t launch_fast_dplr(const ChunkArgs& a);    // general DPLR on the MFMA path
hipError_t launch_generic(const ChunkArgs& a, int dtype_bf16);
bool generic_supported(int dk, int dv, int C);
hipError_t launch_decode(const void* q, const void* k, const void* v, const float* z,
                         const float* b, const float* A, float* state, void* o,
                         int N, int H, int dk, int dv, int dtype_bf16, hipStream_t s,
                         int mode = kModeKDA);
bool decode_supported(int dk, int dv);
hipError_t launch_layer_pre(const void* q_in, const void* k_in, const void* v_in,
                            const float* conv_w, const void* cs0, const int* cu, int N, int Tfix,
                            int Ttot, int H, int d, float l2_eps, void* q_out, void* k_out,
                            void* v_out, int dtype_bf16, hipStream_t s);
hipError_t launch_layer_convstate(const void* q_in, const void* k_in, const void* v_in,
                                  const void* cs0, const int* cu, int N, int Tfix, int Ttot,
                                  int H, int d, void* cs_out, int dtype_bf16, hipStream_t s);
hipError_t launch_layer_post(const void* o, const void* gate, const float* norm_w, float rms_eps,
                             long long rows, int d, void* y, int dtype_bf16, hipStream_t s);
hipError_t launch_layer_step(const void* q_in, const void* k_in, const void* v_in,
                             const float* conv_w, void* conv_state, const float* z, const float* b,
                             const float* A, float* state, const void* gate, const float* norm_w,
                             float l2_eps, float rms_eps, void* y, int N, int H, int d,
                             int dtype_bf16, hipStream_t s);
hipError_t launch_dplr_generic(const ChunkArgs& a, int dtype_bf16);
hipError_t launch_dplr_intra(const ChunkArgs& a);   // MFMA path: the DPLR intra-chunk launch
hipError_t launch_dplr_decode(const void* q, const void* k, const void* v, const void* la,
                              const void* lb, const float* z, const float* A, float* state,
                              void* o, int N, int H, int d, int dtype_bf16, hipStream_t s);
hipError_t launch_verify(const void* q, const void* k, const void* v, const float* z,
                         const float* b, const float* A, const float* state, void* o, int N,
                         int W, int H, int dk, int dv, int dtype_bf16, hipStream_t s);
hipError_t launch_fold(const void* k, const void* v, const float* z, const float* b,
                       const float* A, const int* n_accept, float* state, int N, int W, int H,
                       int dk, int dv, int dtype_bf16, hipStream_t s);

}  // namespace kda
