// Chunked KDA prefill on MFMA: bf16 inputs, d_k = d_v = 128, chunk C = 64.
//
// Sources:
//   [LA-KDA]  "从线性注意力到 KDA：拆解 Kimi K3 的核心注意力机制", blog-3d3.pages.dev/posts/150
//   [K3-ATTN] "Kimi K3 注意力机制深度解析：KDA、Gated MLA 与 AttnRes 的混合架构"
//
// Per chunk (positions i, j in 0..63, channels c; G = in-chunk inclusive
// cumulative log-decay; Gamma = e^G), the chunked form of [LA-KDA §7] with
// the decay ([LA-KDA §7.2]) and the delta correction ([LA-KDA §7.3]):
//   A_kk[i,j] = beta_i sum_c k_ic k_jc e^{G_ic - G_jc}   (j < i)
//   A_qk[i,j] =        sum_c q_ic k_jc e^{G_ic - G_jc}   (j <= i)
//   T  = (I + A_kk)^{-1} Diag(beta)          (the UT transform)
//   W  = T (K . Gamma),  U = T V             (the WY pair; no S dependence)
//   V~ = U - W S
//   O  = (Q . Gamma) S + A_qk V~
//   S <- Diag(Gamma_C) S + Kbar^T V~,   Kbar = K . e^{G_C - G}
// Only the two C x C matrices A_kk and A_qk are formed: the diagonal and the
// low-rank terms share the same k ([K3-ATTN §2.2]).
//
// Launches:
//   intra       one workgroup per (chunk, head), all chunks in parallel: gate,
//               cumulative decay, A_kk and A_qk on MFMA, the fp32 triangular
//               inverse, W, U, Q . Gamma and Kbar on MFMA.  It writes them as
//               bf16 operand fragments already in the order the chain
//               kernels' lanes load them, with nontemporal stores (the later
//               launches read them back from HBM, never from a cache).
//   transition  per (segment, head): the chain over the segment's chunks on
//               the augmented state [R | M] (see the chain section below);
//   compose     per (sequence, head): segment start states in fp32;
//   output      per (segment, head): the chain from the segment's start
//               state, forming V~, the output rows and the next state.
//
// Exponent range: the lower bound g > -5 ([LA-KDA §5.4]) keeps every
// reciprocal decay factor inside a 16-token sub-tile ([LA-KDA §8]) below
// e^{80} < FLT_MAX.  A_kk/A_qk tiles of row block r use the cumulative decay
// just before block r as reference: the row factor e^{G_i - G_ref} <= 1, the
// column factor e^{G_ref - G_j} <= 1 off the diagonal and < e^{80} on it.
// Gamma, Kbar and gamma_C only ever carry factors <= 1.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_fast_common.hpp"
#include "kda_internal.hpp"

namespace kda {

using namespace fast;
using namespace fastc;

namespace {

// Lane n of each 16-lane row (a 16-token block, lanes n = token) receives the
// row D tokens before its own: lane n - D of the same block when n >= D,
// else lane n - D + 16 of the previous block.  Each source lane sends its
// current row if that row stays inside the block, its previous-block row
// otherwise; a DPP rotate within the 16-lane row moves it (no LDS).
template <int D>
__device__ __forceinline__ unsigned row_ror(unsigned x) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x120 + D, 0xF, 0xF, false);
}

template <int D>
__device__ __forceinline__ uint4 rows_back(uint4 prev, uint4 cur, int n16) {
    const bool own = n16 < 16 - D;
    uint4 r;
    r.x = row_ror<D>(own ? cur.x : prev.x);
    r.y = row_ror<D>(own ? cur.y : prev.y);
    r.z = row_ror<D>(own ? cur.z : prev.z);
    r.w = row_ror<D>(own ? cur.w : prev.w);
    return r;
}

constexpr int kOffRK = 64 * kLdG * 4;                    // CONV: L2Norm partial sums in step 1
constexpr int kOffFac = kOffRK + 64 * kLdK * 2 * 2;
constexpr int kOffBeta = kOffFac + kNFac * 128 * 4;
constexpr int kSmemIntra = kOffBeta + 64 * 4;            // 80128 bytes: two workgroups per CU
// 16 bytes per lane from global memory straight to LDS: lane l's bytes land
// at lds + 16 l (lds is the same for the whole wave)
__device__ __forceinline__ void copy16_to_lds(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// CONV, step 1 (before the factor rows are written): the chunk's gate logits
// [64][128] after the L2Norm partial sums, the head's taps over the factor rows
constexpr int kOffZ = kOffRK + 2 * 64 * 4 * 4;
constexpr int kOffConvW = kOffFac;
static_assert(kOffZ + 64 * 128 * 4 <= kOffFac, "the gate logits leave the factor rows intact");
static_assert(kOffConvW + 3 * 128 * 16 <= kOffBeta, "the taps leave beta intact");
// step 3: partial tiles [20 tiles][3 writers][64 lanes] of f32x4 over L (and
// below the factor rows, which the partial products still read); A_kk after
// them (the factor rows are dead by then); N and the inverse's scratch over
// the partials once they are summed
constexpr int kOffPart = 0;
constexpr int kPartBytes = 20 * 3 * 64 * 16;
constexpr int kOffAkk = kOffPart + kPartBytes;
static_assert(kPartBytes <= kOffFac, "the partial tiles leave the factor rows intact");
static_assert(kOffAkk + 64 * kLdA * 4 <= kOffBeta, "A_kk leaves beta intact");
static_assert(64 * kLdA * 4 + kInvScr * 4 <= kOffAkk, "N and the inverse scratch alias the partial tiles");

// Step 3 splits the ten 16x16 tile pairs (r, s), s <= r, of A_kk and of A_qk
// by channel: wave w contracts only its own 32 channels, and the owner of a
// tile sums the four partial tiles in a fixed order.  Owners (five tiles per
// wave): A_kk pairs 0-2 wave 2, 3-5 wave 3, 6-7 wave 0, 8-9 wave 1; A_qk
// pairs 0-2 wave 0, 3-5 wave 1, 6-7 wave 2, 8-9 wave 3, so that both halves
// of each stored A_qk fragment (tiles (r, 2kb) and (r, 2kb + 1)) meet in one
// wave.  pos: the tile's slot among its owner's five.
__host__ __device__ constexpr int kk_owner(int p) { return p < 3 ? 2 : p < 6 ? 3 : p < 8 ? 0 : 1; }
__host__ __device__ constexpr int kk_pos(int p) { return p < 3 ? p : p < 6 ? p - 3 : p < 8 ? p - 6 : p - 8; }
__host__ __device__ constexpr int qk_owner(int p) { return p < 3 ? 0 : p < 6 ? 1 : p < 8 ? 2 : 3; }
__host__ __device__ constexpr int qk_pos(int p) { return p < 3 ? p + 2 : p < 6 ? p - 1 : p < 8 ? p - 3 : p - 5; }

// Step 3's sums for wave W: the four partial tiles of each tile it owns, in
// the order (own, then writers W + 1, W + 2, W + 3), the causal masks (A_kk
// strictly below the diagonal, A_qk on and below it), beta as A_kk's row
// scale; A_kk to LDS in fp32 for the inverse, A_qk to the record as bf16
// operand fragments (token block tb, k-step kb: tiles (tb, 2kb), (tb, 2kb + 1)).
// A lane holds row 16r + n16, columns 16s + 4g4 .. + 3 of tile (r, s).
template <int W, int MODE, bool DBG>
__device__ __forceinline__ void reduce_tiles(const f32x4 (&own)[5], const float* sPart, float* sAkk,
                                             const float* sBeta, uint8_t* __restrict__ rec,
                                             float* __restrict__ dbase, int lane, int n16, int g4) {
    constexpr int NKK = W < 2 ? 2 : 3;                             // A_kk tiles first, then A_qk
    constexpr int KK0 = W == 0 ? 6 : W == 1 ? 8 : W == 2 ? 0 : 3;  // first A_kk pair owned
    constexpr int QK0 = W == 0 ? 0 : W == 1 ? 3 : W == 2 ? 6 : 8;  // first A_qk pair owned
    f32x4 qt[3];
#pragma unroll
    for (int i = 0; i < 5; i++) {
        const bool kk = i < NKK;
        const int p = kk ? KK0 + i : QK0 + i - NKK;
        const int r = pair_row(p), s = p - r * (r + 1) / 2;
        f32x4 t = zero4();
        if (!kk || MODE != kModeGLA) {
            const int tau = kk ? p : 10 + p;
            t = own[i];
#pragma unroll
            for (int k = 0; k < 3; k++) t += *reinterpret_cast<const f32x4*>(sPart + ((tau * 3 + k) * 64 + lane) * 4);
        }
        if (s == r) {
#pragma unroll
            for (int e = 0; e < 4; e++)
                if (4 * g4 + e > n16 || (kk && 4 * g4 + e == n16)) t[e] = 0.f;
        }
        if (kk) {
            const float b = sBeta[16 * r + n16];
#pragma unroll
            for (int e = 0; e < 4; e++) t[e] *= b;
            *reinterpret_cast<f32x4*>(sAkk + (16 * r + n16) * kLdA + 16 * s + 4 * g4) = t;
        } else {
            qt[i - NKK] = t;
        }
        if (DBG)
#pragma unroll
            for (int e = 0; e < 4; e++) dbase[8192 + (kk ? 0 : 4096) + (16 * r + n16) * 64 + 16 * s + 4 * g4 + e] = t[e];
    }
    auto put = [&](int tb, int kb, const f32x4& lo, const f32x4& hi) {
        __builtin_nontemporal_store(pack_frag(lo, hi), reinterpret_cast<bf16x8*>(rec + REC_A + (rec_a_frag(tb, kb) * 64 + lane) * 16));
    };
    if constexpr (W == 0) {
        put(0, 0, qt[0], zero4());
        put(1, 0, qt[1], qt[2]);
    } else if constexpr (W == 1) {
        put(2, 0, qt[0], qt[1]);
        put(2, 1, qt[2], zero4());
    } else if constexpr (W == 2) {
        put(3, 0, qt[0], qt[1]);
    } else {
        put(3, 1, qt[0], qt[1]);
    }
}

// One workgroup per (chunk, head), 4 waves.  Work on single elements is split
// by channel: wave w owns channels [32w, 32w + 32) of all 64 tokens, lane
// (n, g) token rows 16t + n (t = 0..3) and channels 32w + 8g .. 32w + 8g + 7,
// which is the MFMA operand layout of k-step w.  Decay factors are powers of
// two of L = G log2(e): per element E = 2^(L - L_s(r)) <= 1 (row factor) and
// F = 2^(L_e(r) - L) <= 1 (column factor) for its 16-token block r; every
// other exponent is a per-channel factor of the table above, so
//   A_kk/A_qk tile (r, s):  rows (k|q) . E  with  columns (k . F) . X(r,s)
//   K . Gamma = (k . E) . Y(r),  Q . Gamma = (q . E) . Y(r),  Kbar = (k . F) . Z(r)
// (X(r,s) <= 1 off the diagonal, X(r,r) = 2^(L_s - L_e) < e^80 on it).
// The row operands and k . F stay in the registers of the wave that formed
// them: each wave contracts its own k-step for all ten tile pairs, and the
// four partial tiles of a pair are summed by its owner (step 3).
// With CONV, q, k, v are the layer's projections and step 1 applies the
// layer's steps before the core ([LA-KDA §5.3]): the depthwise causal
// convolution (four taps oldest first, the sequence's first three inputs from
// the carried state cs0 or zeros), Swish, and for q and k the L2Norm over the
// head's 128 channels; the results are rounded to bf16 as the core's inputs.
// MODE selects a row of the family table ([LA-KDA §4]): kModeDeltaNet skips
// the gate (G = 0, every factor 1); kModeGLA drops A_kk (T = Diag(beta)), so
// W = 0: it is not stored, and the GLA chain kernels read none (V~ = U =
// Diag(beta) V).
template <bool DBG, bool CONV, int MODE>
__global__ __launch_bounds__(256, 2)
void fast_intra_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                       const bf16* __restrict__ v, const float* __restrict__ z,
                       const float* __restrict__ bl, const float* __restrict__ A,
                       const int* __restrict__ hdr, const int4* __restrict__ chunks, int H,
                       uint8_t* __restrict__ recs, float* __restrict__ dbg,
                       const float* __restrict__ conv_w, const bf16* __restrict__ cs0,
                       float l2_eps, FixedPlan fx)
{
    // heads fastest (whole input rows), and the H heads of a chunk on one XCD:
    // blocks go to the 8 XCDs round-robin, so block 8 s + x takes chunk
    // 8 (s / H) + x, head s % H, and the heads read the chunk's beta row
    // (H values per token) through one L2.  The grid is a multiple of 8 H.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int cid = (slot / H) * 8 + xcd, h = slot % H;
    // equal-length sequences: the chunk follows from its index, and workgroup
    // 0 writes the bookkeeping tables for the later launches
    int4 cd;
    if (fx.on) {
        if (blockIdx.x == 0) write_fixed_tables(fx, threadIdx.x, 256);
        if (cid >= fx.total) return;
        const int n = cid / fx.cps, j = cid - n * fx.cps;
        cd = make_int4(n, n * fx.T + j * fx.C, min(fx.C, fx.T - j * fx.C), j * fx.C);
    } else {
        if (cid >= hdr[0]) return;
        cd = chunks[cid];
    }
    const int tok0 = cd.y, len = cd.z;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    uint8_t* rec = recs + ((size_t)cid * H + h) * REC_BYTES;
    float* dbase = DBG ? dbg + ((size_t)cid * H + h) * (64 * 128 + 3 * 64 * 64) : nullptr;

    __shared__ __align__(16) uint8_t smem[kSmemIntra];
    float* sG = reinterpret_cast<float*>(smem);                       // [64][kLdG]
    float* sFac = reinterpret_cast<float*>(smem + kOffFac);           // [kNFac][128]
    float* sBeta = reinterpret_cast<float*>(smem + kOffBeta);         // [64]

    // rows past the end of the sequence read the last valid row: they only
    // meet rows and columns that beta = 0 and g = 0 switch off
    const unsigned tstride = (unsigned)H * 128u;
    const size_t base = (size_t)tok0 * tstride + (size_t)h * 128;
    const int lastrow = len - 1;
    auto roff = [&](int row) { return (unsigned)min(row, lastrow) * tstride; };
    const int cw = 32 * w + 8 * g4;

    // ---- 1. loads: q, k, v rows straight to registers (each element used by
    //      one lane); gate [LA-KDA §5.4] and in-chunk cumulative sum in log2 units
    uint4 kr[4], qr[4], vr[4];
    float qkf[2][4][8];              // CONV: q, k after Swish, before the L2Norm
    // the beta logits, issued with the first loads so that their latency hides
    // under the gate scan (wave 0 turns them into beta before the barrier);
    // with CONV after the other loads of step 1, just before its first barrier
    float blx = 0.f;
    auto load_beta_logits = [&]() {
        if (tid < 64) blx = bl[(size_t)(tok0 + min(tid, lastrow)) * H + h];
    };
    if constexpr (!CONV) load_beta_logits();
    // the gate logits (thread = channel c, rows 32 half .. 32 half + 31),
    // likewise issued first (with CONV they go to LDS beside the
    // convolution's loads: its registers leave no room for them)
    const int c = tid & 127, half = tid >> 7;
    float lr[32];
    if constexpr (MODE != kModeDeltaNet && !CONV)
#pragma unroll
        for (int i = 0; i < 32; i++) lr[i] = z[base + roff(32 * half + i) + c];
    float* sL2 = reinterpret_cast<float*>(smem + kOffRK);   // CONV: [2][64 rows][4 waves], free in step 1
    if constexpr (!CONV) {
#pragma unroll
        for (int tt = 0; tt < 4; tt++) {
            const unsigned off = roff(16 * tt + n16) + cw;
            kr[tt] = *reinterpret_cast<const uint4*>(k + base + off);
            qr[tt] = *reinterpret_cast<const uint4*>(q + base + off);
            vr[tt] = *reinterpret_cast<const uint4*>(v + base + off);
        }
    } else {
        // every load of the step is issued before any arithmetic, with no
        // branch between them (the halo rows from in-bounds addresses,
        // zeroed afterwards): the three convolutions then wait once
        const int n = cd.x, p0 = cd.w;       // sequence, position of row 0 within it
        // the head's taps, [3 inputs][128 channels] float4, and the chunk's
        // gate logits are copied straight to LDS (16 bytes per lane, landing
        // at the instruction's LDS base + 16 lane): wave w < 3 copies the taps
        // of input w, every wave 16 rows of logits, two per instruction
        float4* sW = reinterpret_cast<float4*>(smem + kOffConvW);
        if (w < 3)
#pragma unroll
            for (int j = 0; j < 2; j++)
                copy16_to_lds(conv_w + (((size_t)w * H + h) * 128 + 64 * j + lane) * 4, sW + 128 * w + 64 * j);
        if constexpr (MODE != kModeDeltaNet) {
            float* sZ = reinterpret_cast<float*>(smem + kOffZ);
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const int r0 = 16 * w + 2 * i;
                copy16_to_lds(z + base + roff(r0 + (lane >> 5)) + 4 * (lane & 31), sZ + r0 * 128);
            }
        }
        // xr[X][0]: lanes 13..15 hold the three rows before the chunk (block
        // -1), from the sequence or, before its start, from the carried state
        // (zeros without one); xr[X][1 + t]: this lane's row of block t
        uint4 xr[3][5];
        const int src = p0 + n16 - 16;       // position in the sequence of the halo row
        const bool from_seq = src >= 0, from_cs = !from_seq && cs0 != nullptr && src >= -3;
        const bool halo = n16 >= 13 && (from_seq || from_cs);
#pragma unroll
        for (int X = 0; X < 3; X++) {
            const bf16* xin = X == 0 ? q : X == 1 ? k : v;
            const bf16* hp = from_seq ? xin + ((size_t)(tok0 + n16 - 16) * H + h) * 128 + cw
                           : from_cs ? cs0 + ((((size_t)n * 3 + X) * 3 + (3 + src)) * H + h) * 128 + cw
                                     : xin + base + roff(n16) + cw;
            xr[X][0] = *reinterpret_cast<const uint4*>(hp);
#pragma unroll
            for (int tt = 0; tt < 4; tt++)
                xr[X][tt + 1] = *reinterpret_cast<const uint4*>(xin + base + roff(16 * tt + n16) + cw);
        }
        load_beta_logits();
        __syncthreads();
#pragma unroll
        for (int X = 0; X < 3; X++) {
            // one input at a time: the taps of the next are not read early
            __builtin_amdgcn_sched_barrier(0);
            if (!halo) xr[X][0] = make_uint4(0, 0, 0, 0);
            float wt[8][4];
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float4 w4 = sW[X * 128 + cw + e];
                wt[e][0] = w4.x; wt[e][1] = w4.y; wt[e][2] = w4.z; wt[e][3] = w4.w;
            }
#pragma unroll
            for (int tt = 0; tt < 4; tt++) {
                float y[8];
#pragma unroll
                for (int e = 0; e < 8; e++) y[e] = 0.f;
                // tap j (oldest first) reads the row 3 - j before this lane's row
                const uint4 taps[4] = {rows_back<3>(xr[X][tt], xr[X][tt + 1], n16),
                                       rows_back<2>(xr[X][tt], xr[X][tt + 1], n16),
                                       rows_back<1>(xr[X][tt], xr[X][tt + 1], n16), xr[X][tt + 1]};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const bf16x8 xv = __builtin_bit_cast(bf16x8, taps[j]);
#pragma unroll
                    for (int e = 0; e < 8; e++) y[e] = __builtin_fmaf(wt[e][j], (float)xv[e], y[e]);
                }
#pragma unroll
                for (int e = 0; e < 8; e++) y[e] = y[e] * __builtin_amdgcn_rcpf(1.f + ex2(-y[e] * kLog2e));
                if (X == 2) {
                    bf16x8 o8;
#pragma unroll
                    for (int e = 0; e < 8; e++) o8[e] = (bf16)y[e];
                    vr[tt] = __builtin_bit_cast(uint4, o8);
                } else {
                    float ss = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; e++) {
                        qkf[X][tt][e] = y[e];
                        ss = __builtin_fmaf(y[e], y[e], ss);
                    }
                    ss += __shfl_xor(ss, 16, 64);      // the 4 lanes of this row in the wave
                    ss += __shfl_xor(ss, 32, 64);
                    // the four lanes of the row hold the same sum: all store it
                    sL2[(X * 64 + 16 * tt + n16) * 4 + w] = ss;
                }
            }
        }
    }
    {
        float a2 = 0.f;                                 // e^{-e^A z} = 2^(a2 z)
        if constexpr (MODE != kModeDeltaNet) {
            a2 = -expf(A[h]) * kLog2e;
            if constexpr (CONV) {
                const float* sZ = reinterpret_cast<const float*>(smem + kOffZ);
#pragma unroll
                for (int i = 0; i < 32; i++) lr[i] = sZ[(32 * half + i) * 128 + c];
            }
        }
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < 32; i++) {
            const int row = 32 * half + i;
            if constexpr (MODE != kModeDeltaNet) {
                float sg = __builtin_amdgcn_rcpf(1.f + ex2(lr[i] * a2));
                sg = row < len ? sg : 0.f;
                run = fmaf(sg, kGMin * kLog2e, run);
            }
            lr[i] = run;
            sG[row * kLdG + c] = run;
        }
        if (tid < 64) sBeta[tid] = tid < len ? __builtin_amdgcn_rcpf(1.f + ex2(-blx * kLog2e)) : 0.f;
    }
    __syncthreads();
    if constexpr (CONV) {
#pragma unroll
        for (int X = 0; X < 2; X++)
#pragma unroll
            for (int tt = 0; tt < 4; tt++) {
                const float4 p4 = *reinterpret_cast<const float4*>(sL2 + (X * 64 + 16 * tt + n16) * 4);
                const float inv = __builtin_amdgcn_rsqf(((p4.x + p4.y) + (p4.z + p4.w)) + l2_eps);
                bf16x8 o8;
#pragma unroll
                for (int e = 0; e < 8; e++) o8[e] = (bf16)(qkf[X][tt][e] * inv);
                (X == 0 ? qr : kr)[tt] = __builtin_bit_cast(uint4, o8);
            }
    }
    // second half: add L at row 31; per-channel factors
    {
        float* F = sFac + c;
        if (half == 0) {
            const float L15 = lr[15], L31 = lr[31];
            F[(kFX + 0) * 128] = ex2(-L15);
            F[(kFX + 1) * 128] = 1.f;
            F[(kFX + 2) * 128] = ex2(L15 - L31);
            F[(kFX + 3) * 128] = ex2(L31 - L15);
            F[(kFX + 4) * 128] = 1.f;
            F[(kFX + 8) * 128] = 1.f;
            F[(kFY + 0) * 128] = 1.f;
            F[(kFY + 1) * 128] = ex2(L15);
            F[(kFY + 2) * 128] = ex2(L31);
            F[(kFZ + 3) * 128] = 1.f;
            F[(kFL + 0) * 128] = L15;
            F[(kFL + 1) * 128] = L31;
        } else {
            const float L15 = sG[15 * kLdG + c], L31 = sG[31 * kLdG + c];
#pragma unroll
            for (int i = 0; i < 32; i++) {
                lr[i] += L31;
                sG[(32 + i) * kLdG + c] = lr[i];
            }
            const float L47 = lr[15], L63 = lr[31];
            F[(kFX + 5) * 128] = ex2(L31 - L47);
            F[(kFX + 6) * 128] = ex2(L47 - L15);
            F[(kFX + 7) * 128] = ex2(L47 - L31);
            F[(kFX + 9) * 128] = ex2(L47 - L63);
            F[(kFY + 3) * 128] = ex2(L47);
            F[(kFZ + 0) * 128] = ex2(L63 - L15);
            F[(kFZ + 1) * 128] = ex2(L63 - L31);
            F[(kFZ + 2) * 128] = ex2(L63 - L47);
            F[(kFL + 2) * 128] = L47;
            F[(kFL + 3) * 128] = L63;
            __builtin_nontemporal_store(ex2(L63), reinterpret_cast<float*>(rec + REC_G) + c);
        }
    }
    __syncthreads();
    if (DBG) {
        for (int idx = tid; idx < 8192; idx += 256) dbase[idx] = sG[(idx >> 7) * kLdG + (idx & 127)] * kLn2;
        __syncthreads();
    }

    // ---- 2. per element: row and column factors, the row operands and K.F
    //      (kept in registers: lane (n, g) of wave w holds them for token rows
    //      16t + n, channels 32w + 8g .. + 7, the operand layout of k-step w),
    //      and token-contiguous copies via an exact selection product: MFMA(X
    //      rows, one-hot B) returns X in the C layout (4 consecutive tokens of
    //      one channel per lane), MFMA(one-hot A, X rows) returns X^T in it
    bf16x8 sel[2];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        sel[0][e] = (bf16)((8 * g4 + e == n16) ? 1.f : 0.f);
        sel[1][e] = (bf16)((8 * g4 + e == 16 + n16) ? 1.f : 0.f);
    }
    bf16x8 kgf[2][2], vf[2][2];     // (K . Gamma)^T, V^T fragments [token kstep][16-channel half]
    bf16x8 rkr[4], rqr[4];          // rows k . E, q . E of token block t
    float kfr[4][8];                // k . F of token block t
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
        f32x4 tkg[2][2], tkb[2][2], tv[2][2];
#pragma unroll
        for (int t2 = 0; t2 < 2; t2++) {
            const int tt = 2 * kb + t2, row = 16 * tt + n16;
            float L8[8], Ls[8], Le[8], Y8[8], Z8[8];
            load8f(sG + row * kLdG + cw, L8);
            if (tt > 0) load8f(sFac + (kFL + tt - 1) * 128 + cw, Ls);
            else {
#pragma unroll
                for (int e = 0; e < 8; e++) Ls[e] = 0.f;
            }
            load8f(sFac + (kFL + tt) * 128 + cw, Le);
            load8f(sFac + (kFY + tt) * 128 + cw, Y8);
            load8f(sFac + (kFZ + tt) * 128 + cw, Z8);
            const bf16x8 kk = __builtin_bit_cast(bf16x8, kr[tt]);
            const bf16x8 qq = __builtin_bit_cast(bf16x8, qr[tt]);
            bf16x8 rk, rq, akg, akb, aq;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                const float E = ex2(L8[e] - Ls[e]), F = ex2(Le[e] - L8[e]);
                const float kv = (float)kk[e], qv = (float)qq[e];
                const float kE = kv * E, qE = qv * E, kF = kv * F;
                rk[e] = (bf16)kE;
                rq[e] = (bf16)qE;
                akg[e] = (bf16)(kE * Y8[e]);
                aq[e] = (bf16)(qE * Y8[e]);
                akb[e] = (bf16)(kF * Z8[e]);
                kfr[tt][e] = kF;
            }
            rkr[tt] = rk;
            rqr[tt] = rq;
            f32x4 qt[2];
#pragma unroll
            for (int cb = 0; cb < 2; cb++) {
                tkg[t2][cb] = mfma_bf16(akg, sel[cb], zero4());
                tkb[t2][cb] = mfma_bf16(akb, sel[cb], zero4());
                tv[t2][cb] = mfma_bf16(__builtin_bit_cast(bf16x8, vr[tt]), sel[cb], zero4());
                qt[cb] = mfma_bf16(sel[cb], aq, zero4());
            }
            // (Q . Gamma)^T tiles [channel][token] as the chain's A operand (k-step w)
            __builtin_nontemporal_store(pack_frag(qt[0], qt[1]), reinterpret_cast<bf16x8*>(rec + REC_Q + ((tt * 4 + w) * 64 + lane) * 16));
        }
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            kgf[kb][cb] = pack_frag(tkg[0][cb], tkg[1][cb]);
            vf[kb][cb] = pack_frag(tv[0][cb], tv[1][cb]);
            __builtin_nontemporal_store(pack_frag(tkb[0][cb], tkb[1][cb]), reinterpret_cast<bf16x8*>(rec + REC_K + (((w * 2 + cb) * 2 + kb) * 64 + lane) * 16));
        }
    }
    __syncthreads();

    // ---- 3. A_kk and A_qk [LA-KDA §7.2, §7.3], split by channel: every wave
    //      forms the partial tiles of its own 32 channels (k-step w) from its
    //      registers; each tile's owner sums the four partials in a fixed order
    float* sPart = reinterpret_cast<float*>(smem + kOffPart);          // [20][3][64] f32x4
    float* sAkk = reinterpret_cast<float*>(smem + kOffAkk);            // [64][kLdA]
    f32x4 own[5];
#pragma unroll
    for (int i = 0; i < 5; i++) own[i] = zero4();
    auto part_out = [&](int tau, int owner, int pos, const f32x4& t) {
        if (w == owner) own[pos] = t;
        else *reinterpret_cast<f32x4*>(sPart + ((tau * 3 + ((w - owner - 1) & 3)) * 64 + lane) * 4) = t;
    };
#pragma unroll
    for (int p = 0; p < 10; p++) {
        const int r = pair_row(p), s = p - r * (r + 1) / 2;
        float X8[8];
        load8f(sFac + (kFX + p) * 128 + cw, X8);
        bf16x8 col;
#pragma unroll
        for (int e = 0; e < 8; e++) col[e] = (bf16)(kfr[s][e] * X8[e]);
        // columns as the A operand: the lane receives row 16r + n, columns 16s + 4g .. + 3
        if constexpr (MODE != kModeGLA) part_out(p, kk_owner(p), kk_pos(p), mfma_bf16(col, rkr[r], zero4()));
        part_out(10 + p, qk_owner(p), qk_pos(p), mfma_bf16(col, rqr[r], zero4()));
    }
    __syncthreads();
    switch (w) {
        case 0: reduce_tiles<0, MODE, DBG>(own, sPart, sAkk, sBeta, rec, dbase, lane, n16, g4); break;
        case 1: reduce_tiles<1, MODE, DBG>(own, sPart, sAkk, sBeta, rec, dbase, lane, n16, g4); break;
        case 2: reduce_tiles<2, MODE, DBG>(own, sPart, sAkk, sBeta, rec, dbase, lane, n16, g4); break;
        default: reduce_tiles<3, MODE, DBG>(own, sPart, sAkk, sBeta, rec, dbase, lane, n16, g4); break;
    }
    float* sN = reinterpret_cast<float*>(smem);                         // [64][kLdA], over the partials
    float* sP = sN + 64 * kLdA;                                         // inverse scratch
    if (DBG)
        for (int idx = tid; idx < 6 * 256; idx += 256) {  // A_kk and A_qk tiles (r, s), s > r, are zero
            const int t = idx >> 8, e = idx & 255;
            const int r = t < 3 ? 0 : t < 5 ? 1 : 2, s = t < 3 ? t + 1 : t < 5 ? t - 1 : 3;
            const int at = (16 * r + (e >> 4)) * 64 + 16 * s + (e & 15);
            dbase[8192 + at] = 0.f;
            dbase[8192 + 4096 + at] = 0.f;
        }
    __syncthreads();   // the partials are summed: N and its scratch may overwrite them
    for (int idx = tid; idx < 6 * 256; idx += 256) {      // N's blocks (r, s), s > r, are zero
        const int t = idx >> 8, e = idx & 255;
        const int r = t < 3 ? 0 : t < 5 ? 1 : 2, s = t < 3 ? t + 1 : t < 5 ? t - 1 : 3;
        sN[(16 * r + (e >> 4)) * kLdA + 16 * s + (e & 15)] = 0.f;
    }

    // ---- 4. N = (I + A_kk)^{-1} in fp32, 16x16 blocks ----
    unit_lower_inverse(sAkk, sN, sP, w, n16, g4);
    if (DBG)
        for (int idx = tid; idx < 4096; idx += 256)
            dbase[8192 + 8192 + idx] = sN[(idx >> 6) * kLdA + (idx & 63)] * sBeta[idx & 63];

    // ---- 5. products over tokens (wave w: channels [32w, 32w + 32)) ----
    // k-slot order of every token-contracting fragment: lane group g, slot e
    // holds token 32*kb + 4g + e (e < 4) or 32*kb + 16 + 4g + (e - 4) (e >= 4),
    // matching two stacked C tiles.
    bf16x8 tf[4][2];                // T row fragments [row block][kstep]
#pragma unroll
    for (int tb = 0; tb < 4; tb++)
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            const int row = 16 * tb + n16, j0 = 32 * kb + 4 * g4, j1 = j0 + 16;
            const float4 n0 = *reinterpret_cast<const float4*>(sN + row * kLdA + j0);
            const float4 n1 = *reinterpret_cast<const float4*>(sN + row * kLdA + j1);
            const float4 b0 = *reinterpret_cast<const float4*>(sBeta + j0);
            const float4 b1 = *reinterpret_cast<const float4*>(sBeta + j1);
            const f32x4 t0 = {n0.x * b0.x, n0.y * b0.y, n0.z * b0.z, n0.w * b0.w};
            const f32x4 t1 = {n1.x * b1.x, n1.y * b1.y, n1.z * b1.z, n1.w * b1.w};
            tf[tb][kb] = pack_frag(t0, t1);
        }
    // W^T = (K . Gamma)^T T^T: tiles [channel][token], stored negated as the
    // chain's A operand (token block tb, k-step w)
#pragma unroll
    for (int tb = 0; tb < 4; tb++) {
        if constexpr (MODE != kModeGLA) {
            f32x4 wt0 = zero4(), wt1 = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; kb++) {
                wt0 = mfma_bf16(kgf[kb][0], tf[tb][kb], wt0);
                wt1 = mfma_bf16(kgf[kb][1], tf[tb][kb], wt1);
            }
            __builtin_nontemporal_store(pack_frag_neg(wt0, wt1), reinterpret_cast<bf16x8*>(rec + REC_W + ((tb * 4 + w) * 64 + lane) * 16));
        }
    }
    // U = T V: tiles (slice 2w + cb, token block tb)
#pragma unroll
    for (int tb = 0; tb < 4; tb++)
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            f32x4 u = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; kb++) u = mfma_bf16(tf[tb][kb], vf[kb][cb], u);
            __builtin_nontemporal_store(pack4(u), reinterpret_cast<bf16x4*>(rec + REC_U + (((2 * w + cb) * 4 + tb) * 64 + lane) * 8));
        }
}

// ---------------------------------------------------------------------------
// The chain over chunks, split into segments.
//
// A segment's chunks map its incoming state affinely: S_end = M S_start + R,
// with R the state reached from zero and M the product of the per-chunk
// transitions (the context-parallel composition of [LA-KDA §7.5], here
// across the CUs of one GPU).  Three launches:
//   transition  every segment but a sequence's last runs the chain on the
//               augmented state [R | M] (R from 0 with the real U, M from I
//               with U = 0): 256 columns;
//   compose     per (sequence, head, 16 columns): S_start(j+1) = M_j S_start(j) + R_j
//               in fp32, sequentially over the (few) segments;
//   output      every segment re-runs from S_start with outputs; the
//               sequence's last segment writes the final state.
// Per chunk, with S the state entering it:
//   V~ = U - W S,  O = (Q . Gamma) S + A_qk V~,  S <- Diag(gamma_C) S + Kbar^T V~
// (B operands: a bf16 copy of S and V~ gathered in LDS; A operands straight
// from the chunk record).
//
// Output launch: workgroup = (segment, head), 4 waves, all 128 columns, so
// each record byte is read once (a split chain's two halves each read the
// record, through one L2).  Wave w computes V~ and O rows
// [16w, 16w + 16) and owns state rows [32w, 32w + 32) as 8 pairs of fp32 C
// tiles (one pair per 16-column slice).  The bf16 copy of wave w's tiles is
// exactly the B fragment of k-step w.
// Chain kinds: the KDA record; the GLA record, whose W is zero and neither
// stored nor read (V~ = U, and the M columns of a transition only decay); the
// general DPLR record (X~ = Wb S, the folded Uo and Cs terms).
constexpr int kChainKDA = 0, kChainGLA = 1, kChainDPLR = 2;

// With fewer (segment, head) chains than kSplitMaxChains (half the CUs of
// the part) both chain launches split each chain across two workgroups by
// columns, halving the matrix work of every serial step; the grid is sized
// for it whenever the capacity allows it, and each workgroup checks the
// actual segment count (uniform) before it takes its half.
constexpr int kSplitMaxChains = 128;

__device__ __forceinline__ bool chains_split(const int* __restrict__ hdr, int H, int split_grid) {
    return split_grid && (long long)hdr[1] * H <= kSplitMaxChains;
}

// Block b of a split grid: the two halves of a chain are 8 blocks apart, so
// that the round-robin dispatch of blocks to the 8 XCDs puts them on one XCD
// and both read the chain's chunk records through one L2 (the grid is a
// multiple of 16; blocks past the last chain find no segment and return).
__device__ __forceinline__ void split_block(int b, bool split, int& chain, int& half) {
    if (split) {
        half = (b >> 3) & 1;
        chain = ((b >> 4) << 3) | (b & 7);
    } else {
        half = 0;
        chain = b;
    }
}

constexpr int kOutNS = 8;       // 16-column slices
constexpr int kOutDepth = 3;    // record prefetch ring depth (chunks)
constexpr int kLdO = 136;       // bf16 output staging rows [64][kLdO]

// per wave and chunk; KDA uses a (A_qk), DPLR c (Cs), the rest is common.
// NS: the 16-column slices of state and output the workgroup owns (8: all
// 128 columns; 4: one half of a split chain), starting at slice sb.
template <int NS>
struct OutFrags {
    bf16x8 w[4], q[4];          // -W^T (Wb^T), (Q . Gamma)^T (Q'^T) of token block w, k-steps 0..3
    bf16x8 k[4];                // Kbar^T (Abar^T) rows [32w, 32w + 32): [16-row half][token kstep]
    bf16x8 a[2];                // A_qk rows of token block w, token k-steps 0..1
    bf16x4 u[NS];               // U (Uo) tiles of token block w
    bf16x4 c[2][NS];            // Cs tiles of the wave's two row tiles
    float4 g0, g1;              // gamma_C for the wave's two row tiles
};

template <int CK, int NS>
__device__ __forceinline__ void load_out_frags(OutFrags<NS>& f, const uint8_t* __restrict__ rec, int w,
                                               int lane, int g4, int sb) {
    constexpr bool DPLR = CK == kChainDPLR;
    using RL = RecLayout<DPLR>;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        f.w[ks] = CK == kChainGLA ? bf16x8{}
                                  : *reinterpret_cast<const bf16x8*>(rec + RL::W + ((w * 4 + ks) * 64 + lane) * 16);
        f.k[ks] = *reinterpret_cast<const bf16x8*>(rec + RL::K + ((w * 4 + ks) * 64 + lane) * 16);
        f.q[ks] = *reinterpret_cast<const bf16x8*>(rec + RL::Q + ((w * 4 + ks) * 64 + lane) * 16);
    }
    if constexpr (DPLR) {
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int sl = 0; sl < NS; sl++)
                f.c[b][sl] = *reinterpret_cast<const bf16x4*>(rec + RL::C + (((2 * w + b) * 8 + sb + sl) * 64 + lane) * 8);
    } else {
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
            f.a[kb] = rec_a_stored(w, kb)
                          ? *reinterpret_cast<const bf16x8*>(rec + RL::A + (rec_a_frag(w, kb) * 64 + lane) * 16)
                          : bf16x8{};
    }
#pragma unroll
    for (int sl = 0; sl < NS; sl++)
        f.u[sl] = *reinterpret_cast<const bf16x4*>(rec + RL::U + (((sb + sl) * 4 + w) * 64 + lane) * 8);
    const float* gC = reinterpret_cast<const float*>(rec + RL::G);
    f.g0 = *reinterpret_cast<const float4*>(gC + 32 * w + 4 * g4);
    f.g1 = *reinterpret_cast<const float4*>(gC + 32 * w + 16 + 4 * g4);
}

// Output-gate epilogue of the layer entry point ([LA-KDA §5.5]): each stored
// row becomes Sigmoid(gate) * RMSNorm(o) with the row's RMS over its 128
// channels (16 lanes of 8 channels each).
struct OutGate {
    const bf16* gate;         // [tokens, H, 128] logits, or null for the plain output
    float w[8];               // RMSNorm weights of this lane's 8 channels
    float eps;
};

// 64 rows x 256 bytes of O (or, with GATE, of Sigmoid(gate) * RMSNorm(O)),
// 16 bytes per lane, stored nontemporally (written once, read by the caller); with NS = 4 the 128 bytes of the workgroup's column half
// (columns 16 sb ..), staged in sO's first 64 columns.  FULL: every row is
// inside the sequence (a uniform test by the caller), so the stores need no
// per-row test.
template <bool GATE, bool FULL, int NS>
__device__ __forceinline__ void store_rows(const bf16* sO, const bf16x8 (&gpre)[4],
                                           bf16* __restrict__ o, int tok0, int len, int H, int h,
                                           int tid, const OutGate& og, int sb) {
    constexpr int LPR = 2 * NS;                 // 16-byte pieces per row
    static_assert(!GATE || NS == 8, "the gated output needs whole rows");
#pragma unroll
    for (int i = 0; i < LPR / 4; i++) {
        const int idx = i * 256 + tid, row = idx / LPR, c8 = (idx % LPR) * 8;
        const size_t off = ((size_t)(tok0 + row) * H + h) * 128 + 16 * sb + c8;
        if constexpr (GATE) {
            const bf16x8 ob = *reinterpret_cast<const bf16x8*>(sO + row * kLdO + c8);
            float ov[8], ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) {
                ov[e] = (float)ob[e];
                ss = __builtin_fmaf(ov[e], ov[e], ss);
            }
#pragma unroll
            for (int m = 8; m > 0; m >>= 1) ss += __shfl_xor(ss, m, 64);   // the row's 16 lanes
            // hardware reciprocal square root and reciprocal (about 1 ulp;
            // the result is rounded to bf16)
            const float r = __builtin_amdgcn_rsqf(ss * (1.f / 128.f) + og.eps);
            if (FULL || row < len) {
                const bf16x8 gt = gpre[i];
                bf16x8 yv;
#pragma unroll
                for (int e = 0; e < 8; e++) {
                    const float sg = __builtin_amdgcn_rcpf(1.f + ex2(-(float)gt[e] * kLog2e));
                    yv[e] = (bf16)(sg * (ov[e] * r) * og.w[e]);
                }
                __builtin_nontemporal_store(yv, reinterpret_cast<bf16x8*>(o + off));
            }
        } else {
            if (FULL || row < len)
                __builtin_nontemporal_store(*reinterpret_cast<const bf16x8*>(sO + row * kLdO + c8),
                                            reinterpret_cast<bf16x8*>(o + off));
        }
    }
}

// The gate logits of the rows this thread stores for one chunk (rows past
// the end of the sequence read its last row; they are never stored).  The
// caller issues them before the record prefetch of the step: a wave's loads
// complete in order, so loads issued after the prefetch would wait for it.
template <bool GATE>
__device__ __forceinline__ void load_gate_rows(bf16x8 (&gpre)[4], const OutGate& og, int tok0, int len,
                                               int H, int h, int tid) {
    if constexpr (GATE) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int idx = i * 256 + tid, row = min(idx >> 4, len - 1), c8 = (idx & 15) * 8;
            gpre[i] = *reinterpret_cast<const bf16x8*>(og.gate + ((size_t)(tok0 + row) * H + h) * 128 + c8);
        }
    }
}

// One chunk for one wave over all slices.  KDA: V~ = U - W S,
// O = (Q . Gamma) S + A_qk V~, S <- Diag(gamma_C) S + Kbar^T V~.  DPLR:
// X~ = Wb S, O = Q' S + Uo, S <- Diag(gamma_C) S + Abar^T X~ + Cs.
template <bool DBG, bool GATE, int CK, int NS>
__device__ __forceinline__ void out_step(const OutFrags<NS>& f, int cid, int tok0, int len,
                                         f32x4 (&accS)[NS][2], bf16* sS, bf16* sVt, bf16* sO,
                                         bf16* __restrict__ o, float* __restrict__ dbgS, int H,
                                         int h, int w, int lane, int n16, int g4, int tid,
                                         const OutGate& og, int sb, const bf16x8 (&gpre)[4]) {
    constexpr bool DPLR = CK == kChainDPLR;
    if (DBG) {
#pragma unroll
        for (int sl = 0; sl < NS; sl++)
#pragma unroll
            for (int b = 0; b < 2; b++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int row = 32 * w + 16 * b + 4 * g4 + e;
                    dbgS[(((size_t)cid * H + h) * 128 + row) * 128 + 16 * (sb + sl) + n16] = accS[sl][b][e];
                }
    }
    f32x4 accO[NS];
    // V~ and the (Q . Gamma) S part of O, four slices at a time
#pragma unroll
    for (int bb = 0; bb < NS / 4; bb++) {
        bf16x8 sf[4][4];
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++)
#pragma unroll
            for (int ks = 0; ks < 4; ks++)
                sf[s4][ks] = *reinterpret_cast<const bf16x8*>(sS + (((4 * bb + s4) * 4 + ks) * 64 + lane) * 8);
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++) {
            const int sl = 4 * bb + s4;
            f32x4 accV = DPLR ? zero4() : unpack4(f.u[sl]);
            f32x4 acc = DPLR ? unpack4(f.u[sl]) : zero4();
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                if constexpr (CK != kChainGLA) accV = mfma_bf16(f.w[ks], sf[s4][ks], accV);
                acc = mfma_bf16(f.q[ks], sf[s4][ks], acc);
            }
            *reinterpret_cast<bf16x4*>(sVt + ((sl * 4 + w) * 64 + lane) * 4) = pack4(accV);
            accO[sl] = acc;
        }
    }
    __syncthreads();
#pragma unroll
    for (int sl = 0; sl < NS; sl++) {
        bf16x8 vfr[2];
#pragma unroll
        for (int kb = 0; kb < 2; kb++)
            vfr[kb] = concat44(*reinterpret_cast<const bf16x4*>(sVt + ((sl * 4 + 2 * kb) * 64 + lane) * 4),
                               *reinterpret_cast<const bf16x4*>(sVt + ((sl * 4 + 2 * kb + 1) * 64 + lane) * 4));
        f32x4& s0 = accS[sl][0];
        f32x4& s1 = accS[sl][1];
        s0[0] *= f.g0.x; s0[1] *= f.g0.y; s0[2] *= f.g0.z; s0[3] *= f.g0.w;
        s1[0] *= f.g1.x; s1[1] *= f.g1.y; s1[2] *= f.g1.z; s1[3] *= f.g1.w;
        if constexpr (DPLR) {
            s0 += unpack4(f.c[0][sl]);
            s1 += unpack4(f.c[1][sl]);
        }
        f32x4 acc = accO[sl];
#pragma unroll
        for (int kb = 0; kb < 2; kb++) {
            s0 = mfma_bf16(f.k[kb], vfr[kb], s0);
            s1 = mfma_bf16(f.k[2 + kb], vfr[kb], s1);
            if (!DPLR && rec_a_stored(w, kb)) acc = mfma_bf16(f.a[kb], vfr[kb], acc);
        }
        *reinterpret_cast<bf16x8*>(sS + ((sl * 4 + w) * 64 + lane) * 8) = pack_frag(s0, s1);
#pragma unroll
        for (int e = 0; e < 4; e++) sO[(16 * w + 4 * g4 + e) * kLdO + 16 * sl + n16] = (bf16)acc[e];
    }
    __syncthreads();
    if (len >= C) store_rows<GATE, true, NS>(sO, gpre, o, tok0, len, H, h, tid, og, sb);
    else store_rows<GATE, false, NS>(sO, gpre, o, tok0, len, H, h, tid, og, sb);
}

// The output chain of one (segment, head) over NS slices starting at sb.
template <bool DBG, bool GATE, int CK, int NS>
__device__ __forceinline__ void out_body(const uint8_t* __restrict__ recs, const int4* __restrict__ chunks,
                                         int seg_id, int h, int n, int c0, int nch, bool last, int H,
                                         int sb, const float* __restrict__ sstart, bf16* __restrict__ o,
                                         float* __restrict__ hT, float* __restrict__ dbgS,
                                         const bf16* __restrict__ gate, const float* __restrict__ norm_w,
                                         float rms_eps, bf16* sS, bf16* sVt, bf16* sO) {
    constexpr bool DPLR = CK == kChainDPLR;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;

    f32x4 accS[NS][2];
    const float* st = sstart + ((size_t)seg_id * H + h) * 128 * 128;
#pragma unroll
    for (int sl = 0; sl < NS; sl++) {
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                accS[sl][b][e] = st[(32 * w + 16 * b + 4 * g4 + e) * 128 + 16 * (sb + sl) + n16];
        *reinterpret_cast<bf16x8*>(sS + ((sl * 4 + w) * 64 + lane) * 8) = pack_frag(accS[sl][0], accS[sl][1]);
    }
    int seg_tok0 = 0, seg_len = 0;
    if (nch > 0) {
        const int4 first = chunks[c0], lastc = chunks[c0 + nch - 1];
        seg_tok0 = first.y;
        seg_len = lastc.y + lastc.z - first.y;
    }

    OutGate og;
    og.gate = gate;
    og.eps = rms_eps;
#pragma unroll
    for (int e = 0; e < 8; e++) og.w[e] = GATE ? norm_w[(tid & 15) * 8 + e] : 0.f;

    constexpr int D = kOutDepth;
    auto rec = [&](int c) { return recs + ((size_t)(c0 + c) * H + h) * RecLayout<DPLR>::BYTES; };
    OutFrags<NS> F[D];
    if (nch > 0) {
#pragma unroll
        for (int u = 0; u < D - 1; u++) load_out_frags<CK, NS>(F[u], rec(min(u, nch - 1)), w, lane, g4, sb);
    }
    __syncthreads();
    const int nfull = nch / D * D;
    for (int ci = 0; ci < nfull; ci += D) {
#pragma unroll
        for (int u = 0; u < D; u++) {
            const int t0 = (ci + u) * C;
            bf16x8 gpre[4];
            load_gate_rows<GATE>(gpre, og, seg_tok0 + t0, seg_len - t0, H, h, tid);
            // unconditional prefetch (index clamped) keeps the wait counts exact
            load_out_frags<CK, NS>(F[(u + D - 1) % D], rec(min(ci + u + D - 1, nch - 1)), w, lane, g4, sb);
            out_step<DBG, GATE, CK, NS>(F[u], c0 + ci + u, seg_tok0 + t0, seg_len - t0, accS, sS, sVt, sO, o,
                                        dbgS, H, h, w, lane, n16, g4, tid, og, sb, gpre);
        }
    }
#pragma unroll
    for (int u = 0; u < D - 1; u++)
        if (nfull + u < nch) {
            const int t0 = (nfull + u) * C;
            bf16x8 gpre[4];
            load_gate_rows<GATE>(gpre, og, seg_tok0 + t0, seg_len - t0, H, h, tid);
            out_step<DBG, GATE, CK, NS>(F[u], c0 + nfull + u, seg_tok0 + t0, seg_len - t0, accS, sS, sVt,
                                        sO, o, dbgS, H, h, w, lane, n16, g4, tid, og, sb, gpre);
        }

    if (last && hT) {
#pragma unroll
        for (int sl = 0; sl < NS; sl++)
#pragma unroll
            for (int b = 0; b < 2; b++)
#pragma unroll
                for (int e = 0; e < 4; e++)
                    hT[(((size_t)n * H + h) * 128 + 32 * w + 16 * b + 4 * g4 + e) * 128 + 16 * (sb + sl) + n16] =
                        accS[sl][b][e];
    }
}

// grid: seg_cap * H blocks, block = (segment, head), times 2 (the column
// halves, placed by split_block, the grid rounded up to a multiple of 16)
// when split_grid.  With GATE the rows stored are the layer's gated
// RMSNorm of O instead of O; the gated, debug and DPLR outputs never split.
template <bool DBG, bool GATE, int CK>
__global__ __launch_bounds__(256, 1)
void seg_out_kernel(const uint8_t* __restrict__ recs, const int4* __restrict__ chunks,
                    const int4* __restrict__ segs, const int2* __restrict__ seqsegs,
                    const int* __restrict__ hdr, int H, const float* __restrict__ sstart,
                    bf16* __restrict__ o, float* __restrict__ hT, float* __restrict__ dbgS,
                    const bf16* __restrict__ gate, const float* __restrict__ norm_w, float rms_eps,
                    int split_grid)
{
    constexpr bool CAN_SPLIT = !DBG && !GATE && CK != kChainDPLR;
    int chain, half;
    split_block(blockIdx.x, CAN_SPLIT && split_grid, chain, half);
    const int seg_id = chain / H, h = chain % H;
    if (seg_id >= hdr[1]) return;
    const int4 sg = segs[seg_id];          // (sequence, first chunk, chunks, index in sequence)
    const int n = sg.x;
    const bool last = sg.w == seqsegs[n].y - 1;

    __shared__ __align__(16) bf16 sS[kOutNS * 4 * 64 * 8];
    __shared__ __align__(16) bf16 sVt[kOutNS * 4 * 64 * 4];
    __shared__ __align__(16) bf16 sO[64 * kLdO];
    if constexpr (CAN_SPLIT) {
        if (chains_split(hdr, H, split_grid)) {
            out_body<DBG, GATE, CK, kOutNS / 2>(recs, chunks, seg_id, h, n, sg.y, sg.z, last, H,
                                                half * kOutNS / 2, sstart, o, hT, dbgS, gate, norm_w,
                                                rms_eps, sS, sVt, sO);
            return;
        }
        if (half != 0) return;
    }
    out_body<DBG, GATE, CK, kOutNS>(recs, chunks, seg_id, h, n, sg.y, sg.z, last, H, 0, sstart, o, hT,
                                    dbgS, gate, norm_w, rms_eps, sS, sVt, sO);
}

// Transition launch: one workgroup of 8 waves per (segment, head) carries the
// whole augmented state [R | M], 256 columns = 16 slices (R in slices 0..7,
// M in 8..15).  Columns evolve independently, so wave w owns the 32 columns of
// slices 2w and 2w + 1 for all 128 rows (8 row tiles x 2 slices of fp32 C
// tiles): its S fragments for V~ = U - W S and its V~ fragments for the state
// update come from its own registers (two stacked C tiles are exactly one
// operand fragment).  Only the chunk's W, Kbar, U and gamma_C are shared: the
// workgroup copies them into LDS two chunks ahead with one barrier per chunk
// (KDA and GLA: direct global-to-LDS loads into a ring of three stages;
// DPLR, whose stage is larger: through registers into two stages).
// stage of one chunk: W, Kbar, U (KDA) or Cs (DPLR) and gamma_C
template <bool DPLR> struct TransStage {
    static constexpr int W = 0, K = 16384, U = 32768, C = 32768;
    static constexpr int G = DPLR ? 65536 : 49152;
    static constexpr int BYTES = G + 512;
};

// the 16-byte pieces of a record's stage that thread t copies
typedef unsigned u32x4 __attribute__((__vector_size__(4 * sizeof(unsigned))));
struct StageRegs {
    u32x4 w0, w1, k0, k1, x0, x1, x2, x3, g;      // x: U (two pieces) or Cs (four)
};

template <int CK>
__device__ __forceinline__ StageRegs stage_load(const uint8_t* __restrict__ rec, int t) {
    constexpr bool DPLR = CK == kChainDPLR;
    using RL = RecLayout<DPLR>;
    auto ld = [&](int off) { return *reinterpret_cast<const u32x4*>(rec + off + t * 16); };
    StageRegs r;
    if constexpr (CK != kChainGLA) {
        r.w0 = ld(RL::W); r.w1 = ld(RL::W + 8192);
    }
    r.k0 = ld(RL::K); r.k1 = ld(RL::K + 8192);
    if constexpr (DPLR) {
        r.x0 = ld(RL::C); r.x1 = ld(RL::C + 8192); r.x2 = ld(RL::C + 16384); r.x3 = ld(RL::C + 24576);
    } else {
        r.x0 = ld(RL::U); r.x1 = ld(RL::U + 8192);
    }
    r.g = *reinterpret_cast<const u32x4*>(rec + RL::G + (t & 31) * 16);
    return r;
}

template <int CK>
__device__ __forceinline__ void stage_store(const StageRegs& r, uint8_t* st, int t) {
    constexpr bool DPLR = CK == kChainDPLR;
    using TS = TransStage<DPLR>;
    auto stv = [&](int off, u32x4 x) { *reinterpret_cast<u32x4*>(st + off + t * 16) = x; };
    if constexpr (CK != kChainGLA) {
        stv(TS::W, r.w0); stv(TS::W + 8192, r.w1);
    }
    stv(TS::K, r.k0); stv(TS::K + 8192, r.k1);
    if constexpr (DPLR) {
        stv(TS::C, r.x0); stv(TS::C + 8192, r.x1); stv(TS::C + 16384, r.x2); stv(TS::C + 24576, r.x3);
    } else {
        stv(TS::U, r.x0); stv(TS::U + 8192, r.x1);
    }
    if (t < 32) *reinterpret_cast<u32x4*>(st + TS::G + t * 16) = r.g;
}

// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8): vm_wait(n) waits for vector memory operations only, down to n
// outstanding; kWaitLgkm0 for LDS and scalar memory operations only
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitVm4 = vm_wait(4), kWaitVm6 = vm_wait(6);
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);   // LDS and scalar memory only

// KDA and GLA stages are copied straight from global memory to LDS (16 bytes
// per lane; a lane's bytes land at the instruction's LDS base + 16 lane): wave
// w copies the 1 KiB run [1024 w, 1024 w + 1024) of each 8 KiB half of W,
// Kbar and U, and lanes 0-31 of wave 0 the 512 bytes of gamma_C.  Six loads
// per wave and chunk (four for GLA, which has no W), one more on wave 0.
template <int CK>
__device__ __forceinline__ void stage_dma(const uint8_t* __restrict__ rec, uint8_t* st, int w, int lane) {
    static_assert(CK != kChainDPLR, "the DPLR stage is copied through registers");
    using RL = RecLayout<false>;
    using TS = TransStage<false>;
    auto cp = [&](int roff, int soff) {
        __builtin_amdgcn_global_load_lds(rec + roff + (w * 64 + lane) * 16, st + soff + w * 1024, 16, 0, 0);
    };
    if constexpr (CK != kChainGLA) {
        cp(RL::W, TS::W);
        cp(RL::W + 8192, TS::W + 8192);
    }
    cp(RL::K, TS::K);
    cp(RL::K + 8192, TS::K + 8192);
    cp(RL::U, TS::U);
    cp(RL::U + 8192, TS::U + 8192);
    if (w == 0 && lane < 32) __builtin_amdgcn_global_load_lds(rec + RL::G + lane * 16, st + TS::G, 16, 0, 0);
}

// gamma_C of the rows 16 RT + 4 g4 + e (e = 0..3) that lane (n16, g4) holds in
// row tile RT.  Lane (n16, g4) has read gv0 = gamma_C[16 (n16 >> 2) + 4 g4 +
// (n16 & 3)] and gv1 the same 64 rows on; the value of element e of tile RT
// sits in lane 4 (RT & 3) + e of the lane's own 16-lane row, and a DPP row
// broadcast hands it to the whole row (two 4-byte LDS reads per lane and
// chunk instead of a 16-byte read per row tile).
template <int L>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + L,
                                                              0xF, 0xF, false));
}

template <int RT>
__device__ __forceinline__ float4 gamma_rows(float gv0, float gv1) {
    const float x = RT < 4 ? gv0 : gv1;
    constexpr int L0 = 4 * (RT & 3);
    return make_float4(row_bcast<L0>(x), row_bcast<L0 + 1>(x), row_bcast<L0 + 2>(x), row_bcast<L0 + 3>(x));
}

__device__ __forceinline__ float4 gamma_tile(int rt, float gv0, float gv1) {
    switch (rt) {      // rt is a constant wherever the callers' loops are unrolled
        case 0: return gamma_rows<0>(gv0, gv1);
        case 1: return gamma_rows<1>(gv0, gv1);
        case 2: return gamma_rows<2>(gv0, gv1);
        case 3: return gamma_rows<3>(gv0, gv1);
        case 4: return gamma_rows<4>(gv0, gv1);
        case 5: return gamma_rows<5>(gv0, gv1);
        case 6: return gamma_rows<6>(gv0, gv1);
        default: return gamma_rows<7>(gv0, gv1);
    }
}

// One chunk for one wave from the staged record: NJ slices of 16 columns of
// [R | M], the first at slice index s0 (slices 0..7 are R, 8..15 M; is_m: the
// wave's slices are M columns).  KDA: V~ = U - W S (U = 0 for M),
// S <- Diag(gamma_C) S + Kbar^T V~.  GLA: V~ = U, so the M columns (V~ = 0)
// only decay.  DPLR: X~ = Wb S, S <- Diag(gamma_C) S + Abar^T X~ + Cs (Cs for
// R only).
template <int CK, int NJ>
__device__ __forceinline__ void trans_chunk(const uint8_t* st, f32x4 (&acc)[8][NJ], int s0, bool is_m,
                                            int lane, int g4) {
    constexpr bool DPLR = CK == kChainDPLR;
    using TS = TransStage<DPLR>;
    const float* gC = reinterpret_cast<const float*>(st + TS::G);
    const int n16 = lane & 15;
    const float gv0 = gC[16 * (n16 >> 2) + 4 * g4 + (n16 & 3)];
    const float gv1 = gC[64 + 16 * (n16 >> 2) + 4 * g4 + (n16 & 3)];
    if (CK == kChainGLA && is_m) {
#pragma unroll
        for (int rt = 0; rt < 8; rt++) {
            const float4 g = gamma_tile(rt, gv0, gv1);
#pragma unroll
            for (int j = 0; j < NJ; j++) {
                f32x4& a = acc[rt][j];
                a[0] *= g.x; a[1] *= g.y; a[2] *= g.z; a[3] *= g.w;
            }
        }
        return;
    }
    // S fragments of k-step ks: row tiles 2ks, 2ks + 1 of each owned slice
    bf16x8 sf[4][NJ];
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
#pragma unroll
        for (int j = 0; j < NJ; j++) sf[ks][j] = pack_frag(acc[2 * ks][j], acc[2 * ks + 1][j]);
    // V~ = U - W S for the 4 token blocks of the owned slices (U = 0 for M)
    f32x4 vt[4][NJ];
#pragma unroll
    for (int tb = 0; tb < 4; tb++) {
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            vt[tb][j] = zero4();
            if (!DPLR && !is_m)
                vt[tb][j] = unpack4(*reinterpret_cast<const bf16x4*>(
                    st + TS::U + (((s0 + j) * 4 + tb) * 64 + lane) * 8));
        }
        if constexpr (CK != kChainGLA) {
#pragma unroll
            for (int ks = 0; ks < 4; ks++) {
                const bf16x8 wf = *reinterpret_cast<const bf16x8*>(st + TS::W + ((tb * 4 + ks) * 64 + lane) * 16);
#pragma unroll
                for (int j = 0; j < NJ; j++) vt[tb][j] = mfma_bf16(wf, sf[ks][j], vt[tb][j]);
            }
        }
    }
    // V~ fragments over tokens, then S <- Diag(gamma_C) S + Kbar^T V~
    bf16x8 vf[2][NJ];
#pragma unroll
    for (int kb = 0; kb < 2; kb++)
#pragma unroll
        for (int j = 0; j < NJ; j++) vf[kb][j] = pack_frag(vt[2 * kb][j], vt[2 * kb + 1][j]);
#pragma unroll
    for (int rt = 0; rt < 8; rt++) {
        const float4 g = gamma_tile(rt, gv0, gv1);
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(st + TS::K + ((rt * 2 + 0) * 64 + lane) * 16);
        const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(st + TS::K + ((rt * 2 + 1) * 64 + lane) * 16);
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            f32x4& a = acc[rt][j];
            a[0] *= g.x; a[1] *= g.y; a[2] *= g.z; a[3] *= g.w;
            if (DPLR && !is_m)
                a += unpack4(*reinterpret_cast<const bf16x4*>(
                    st + TS::C + ((rt * 8 + s0 + j) * 64 + lane) * 8));
            a = mfma_bf16(k0, vf[0][j], a);
            a = mfma_bf16(k1, vf[1][j], a);
        }
    }
}

// The transition of one (segment, head): NJ = 2, wave w owns slices 2w and
// 2w + 1 (all 256 columns in one workgroup); NJ = 1, wave w of half `half`
// owns slice 8 half + w (R in half 0, M in half 1).
template <int CK, int NJ>
__device__ __forceinline__ void trans_body(const uint8_t* __restrict__ recs, int c0, int nch, int H,
                                           int h, int seg_id, int half, float* __restrict__ rm,
                                           uint8_t (*stage)[TransStage<CK == kChainDPLR>::BYTES]) {
    constexpr bool DPLR = CK == kChainDPLR;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int s0 = NJ == 2 ? 2 * w : 8 * half + w;
    const bool is_m = s0 >= 8;

    f32x4 acc[8][NJ];       // R from 0, M from the identity
#pragma unroll
    for (int rt = 0; rt < 8; rt++)
#pragma unroll
        for (int j = 0; j < NJ; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int row = 16 * rt + 4 * g4 + e, col = 16 * (s0 + j) + n16;
                acc[rt][j][e] = (row == col - 128) ? 1.f : 0.f;
            }
    auto rec = [&](int c) {
        return recs + ((size_t)(c0 + min(c, nch - 1)) * H + h) * RecLayout<DPLR>::BYTES;
    };
    if constexpr (!DPLR) {
        // chunk c sits in stage c % 3, copied there by DMA two chunks ahead;
        // the loads are unconditional (index clamped), so that a wave's own
        // copy of chunk c is complete once at most one chunk's loads remain
        // (the loop issues no other vector memory operation, which the
        // explicit wait below relies on)
        // one copy of the loop per column kind (R or M, uniform per wave), so
        // that the step is compiled with its kind fixed
        auto run = [&](auto m_cols) {
            constexpr bool IM = decltype(m_cols)::value;
            stage_dma<CK>(rec(0), stage[0], w, lane);
            stage_dma<CK>(rec(1), stage[1], w, lane);
            for (int c = 0; c < nch; c++) {
                if constexpr (CK == kChainGLA) __builtin_amdgcn_s_waitcnt(kWaitVm4);
                else __builtin_amdgcn_s_waitcnt(kWaitVm6);
                // every wave's copy of chunk c has landed, and every wave is
                // done with chunk c - 1, whose stage the next copy overwrites.
                // A plain barrier: the LDS is the CU's own, the wait above
                // covers this wave's copies, and a fenced barrier would also
                // wait for the next chunk's copy still in flight
                __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
                asm volatile("" ::: "memory");   // no LDS access moves across the barrier
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                stage_dma<CK>(rec(c + 2), stage[(c + 2) % 3], w, lane);
                trans_chunk<CK, NJ>(stage[c % 3], acc, s0, IM, lane, g4);
            }
            __builtin_amdgcn_s_waitcnt(0);   // no copy outlives the workgroup's LDS
        };
        if (nch > 0) {
            if (is_m) run(std::true_type{});
            else run(std::false_type{});
        }
    } else if (nch > 0) {
        // chunk c sits in stage c & 1; its copy passes through register set c & 1
        StageRegs R0 = stage_load<CK>(rec(0), tid);
        StageRegs R1 = stage_load<CK>(rec(1), tid);
        stage_store<CK>(R0, stage[0], tid);
        R0 = stage_load<CK>(rec(2), tid);
        __syncthreads();
        int c = 0;
        for (; c + 2 <= nch; c += 2) {
            trans_chunk<CK, NJ>(stage[0], acc, s0, is_m, lane, g4);
            stage_store<CK>(R1, stage[1], tid);    // chunk c + 1
            R1 = stage_load<CK>(rec(c + 3), tid);
            __syncthreads();
            trans_chunk<CK, NJ>(stage[1], acc, s0, is_m, lane, g4);
            stage_store<CK>(R0, stage[0], tid);    // chunk c + 2
            R0 = stage_load<CK>(rec(c + 4), tid);
            __syncthreads();
        }
        if (c < nch) trans_chunk<CK, NJ>(stage[0], acc, s0, is_m, lane, g4);
    }
#pragma unroll
    for (int rt = 0; rt < 8; rt++)
#pragma unroll
        for (int j = 0; j < NJ; j++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int row = 16 * rt + 4 * g4 + e, col = 16 * (s0 + j) + n16;
                rm[(((size_t)seg_id * H + h) * 128 + row) * 256 + col] = acc[rt][j][e];
            }
}

// grid: seg_cap * H blocks, block = (segment, head), times 2 (the halves,
// placed by split_block, the grid rounded up to a multiple of 16) when
// split_grid
template <int CK>
__global__ __launch_bounds__(512, 1)
void seg_trans_kernel(const uint8_t* __restrict__ recs, const int4* __restrict__ segs,
                      const int2* __restrict__ seqsegs, const int* __restrict__ hdr, int H,
                      float* __restrict__ rm, int split_grid)
{
    constexpr bool DPLR = CK == kChainDPLR;
    int chain, half;
    split_block(blockIdx.x, split_grid != 0, chain, half);
    const int seg_id = chain / H, h = chain % H;
    if (seg_id >= hdr[1]) return;
    const int4 sg = segs[seg_id];          // (sequence, first chunk, chunks, index in sequence)
    const int2 ss = seqsegs[sg.x];
    if (sg.w == ss.y - 1) return;          // the last segment's transition is never needed
    __shared__ __align__(16) uint8_t stage[DPLR ? 2 : 3][TransStage<DPLR>::BYTES];
    if (chains_split(hdr, H, split_grid))
        trans_body<CK, 1>(recs, sg.y, sg.z, H, h, seg_id, half, rm, stage);
    else if (half == 0)
        trans_body<CK, 2>(recs, sg.y, sg.z, H, h, seg_id, 0, rm, stage);
}

// Segment starts, fp32: per (sequence, head, 16 columns), S_start(0) = h0 and
// S_start(j+1) = M_j S_start(j) + R_j, sequentially over the segments.  A
// sequence without chunks gets hT = h0 here.  M_j is staged in LDS; wave w
// (of 8) computes state rows [16w, 16w + 16) with fp32 MFMA, each lane
// holding the C-tile elements (rows 16w + 4g4 + e, column 16*slice + n16).
// grid: ceil(N*H / 8) * 64 blocks; the 8 slices of one (sequence, head) are
// 8 blocks apart (same XCD), so they read M_j and R_j through one L2.
__global__ __launch_bounds__(512)
void compose_kernel(const int2* __restrict__ seqsegs, const float* __restrict__ h0,
                    const float* __restrict__ rm, float* __restrict__ sstart,
                    float* __restrict__ hT, int N, int H)
{
    const int id = blockIdx.x;
    const int p = (id >> 6) * 8 + (id & 7);
    const int sl = (id >> 3) & 7;
    if (p >= N * H) return;
    const int n = p / H, h = p % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n16 = lane & 15, g4 = lane >> 4;
    const int col = 16 * sl + n16;
    const int row0 = 16 * w + 4 * g4;          // this lane's rows: row0 + e
    __shared__ __align__(16) float sM[128 * 132];
    __shared__ float sSt[128 * 17];

    f32x4 x;
#pragma unroll
    for (int e = 0; e < 4; e++) x[e] = h0 ? h0[((size_t)p * 128 + row0 + e) * 128 + col] : 0.f;
    const int2 ss = seqsegs[n];
    if (ss.y == 0) {
        if (hT)
#pragma unroll
            for (int e = 0; e < 4; e++) hT[((size_t)p * 128 + row0 + e) * 128 + col] = x[e];
        return;
    }
    for (int j = 0; j < ss.y; j++) {
        const size_t seg = (size_t)(ss.x + j);
#pragma unroll
        for (int e = 0; e < 4; e++) sstart[((seg * H + h) * 128 + row0 + e) * 128 + col] = x[e];
        if (j == ss.y - 1) break;
        const float* RM = rm + (seg * H + h) * 128 * 256;
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; e++) r[e] = RM[(size_t)(row0 + e) * 256 + col];
        __syncthreads();                       // previous step done with sM, sSt
#pragma unroll
        for (int i = 0; i < 8; i++) {          // M = columns 128..255 of [R | M]
            const int idx = i * 512 + tid;     // float4 index over 128 rows x 32 float4
            const int row = idx >> 5, c4 = idx & 31;
            *reinterpret_cast<float4*>(sM + row * 132 + 4 * c4) =
                *reinterpret_cast<const float4*>(RM + (size_t)row * 256 + 128 + 4 * c4);
        }
#pragma unroll
        for (int e = 0; e < 4; e++) sSt[(row0 + e) * 17 + n16] = x[e];
        __syncthreads();
        // the contraction over 128 rows in four independent quarters (four
        // short accumulation chains instead of one of 32), summed in a fixed
        // order
        const float* Ab = sM + (16 * w + n16) * 132;
        f32x4 part[4];
#pragma unroll
        for (int qk = 0; qk < 4; qk++) {
            f32x4 acc = zero4();
#pragma unroll
            for (int ks = 8 * qk; ks < 8 * qk + 8; ks++)
                acc = mfma_f32(Ab[4 * ks + g4], sSt[(4 * ks + g4) * 17 + n16], acc);
            part[qk] = acc;
        }
        x = r + ((part[0] + part[1]) + (part[2] + part[3]));
    }
}

}  // namespace

template <int CK>
hipError_t launch_chain(const ChunkArgs& a) {
    const int* hdr = reinterpret_cast<const int*>(a.ws);
    const int4* chunks = reinterpret_cast<const int4*>(a.ws + a.L.off_chunks);
    const int2* seqsegs = reinterpret_cast<const int2*>(a.ws + a.L.off_seqsegs);
    const int4* segs = reinterpret_cast<const int4*>(a.ws + a.L.off_segs);
    uint8_t* recs = a.ws + a.L.off_recs;
    float* sstart = reinterpret_cast<float*>(a.ws + a.L.off_sstart);
    float* rm = reinterpret_cast<float*>(a.ws + a.L.off_rm);
    hipError_t e;
    // the split of each chain across two workgroups can only apply when the
    // segment capacity is small; otherwise the grids keep one per chain
    const long long chains = (long long)a.L.seg_cap * a.H;
    const int split_grid = chains <= 2 * kSplitMaxChains ? 1 : 0;
    const dim3 gc((unsigned)chains), gc2((unsigned)(split_grid ? (2 * chains + 15) / 16 * 16 : chains));
    hipLaunchKernelGGL((seg_trans_kernel<CK>), gc2, dim3(512), 0, a.stream, (const uint8_t*)recs,
                       segs, seqsegs, hdr, a.H, rm, split_grid);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.ev5 && (e = hipEventRecord(a.ev5[0], a.stream)) != hipSuccess) return e;
    const unsigned cblk = (unsigned)(((long long)a.N * a.H + 7) / 8 * 64);
    hipLaunchKernelGGL(compose_kernel, dim3(cblk), dim3(512), 0, a.stream,
                       seqsegs, a.h0, (const float*)rm, sstart, a.hT, a.N, a.H);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.ev5 && (e = hipEventRecord(a.ev5[1], a.stream)) != hipSuccess) return e;
    const bf16* gate = static_cast<const bf16*>(a.gate);
#define KDA_OUT(DBG, GATE)                                                                       \
    do {                                                                                         \
        constexpr bool can_split = !DBG && !GATE && CK != kChainDPLR;                             \
        hipLaunchKernelGGL((seg_out_kernel<DBG, GATE, CK>), can_split ? gc2 : gc, dim3(256), 0,    \
                           a.stream, (const uint8_t*)recs, chunks, segs, seqsegs, hdr, a.H,       \
                           (const float*)sstart, (bf16*)a.o, a.hT,                                 \
                           DBG ? a.dbg_state : (float*)nullptr, gate, a.norm_w, a.rms_eps,         \
                           can_split ? split_grid : 0);                                            \
    } while (0)
    // the debug and gated variants exist for KDA only (the API enforces it)
    if constexpr (CK != kChainKDA) {
        KDA_OUT(false, false);
    } else {
        if (a.dbg_state) KDA_OUT(true, false);
        else if (gate) KDA_OUT(false, true);
        else KDA_OUT(false, false);
    }
#undef KDA_OUT
    return hipGetLastError();
}

hipError_t launch_fast(const ChunkArgs& a) {
    const int* hdr = reinterpret_cast<const int*>(a.ws);
    const int4* chunks = reinterpret_cast<const int4*>(a.ws + a.L.off_chunks);
    uint8_t* recs = a.ws + a.L.off_recs;
    const dim3 gi((unsigned)(((long long)a.L.cap + 7) / 8 * 8 * a.H));
    const bf16* cs0 = static_cast<const bf16*>(a.conv_state0);
#define KDA_INTRA(DBG, CONV, MODE, DBGP)                                                      \
    hipLaunchKernelGGL((fast_intra_kernel<DBG, CONV, MODE>), gi, dim3(256), 0, a.stream,         \
                       (const bf16*)a.q, (const bf16*)a.k, (const bf16*)a.v, a.z, a.b, a.A, hdr, \
                       chunks, a.H, recs, DBGP, a.conv_w, cs0, a.l2_eps, a.fx)
    // the debug and layer variants exist for KDA only (the API enforces it)
    if (a.dbg_intra) KDA_INTRA(true, false, kModeKDA, a.dbg_intra);
    else if (a.conv_w) KDA_INTRA(false, true, kModeKDA, (float*)nullptr);
    else if (a.mode == kModeGLA) KDA_INTRA(false, false, kModeGLA, (float*)nullptr);
    else if (a.mode == kModeDeltaNet) KDA_INTRA(false, false, kModeDeltaNet, (float*)nullptr);
    else KDA_INTRA(false, false, kModeKDA, (float*)nullptr);
#undef KDA_INTRA
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.ev && (e = hipEventRecord(a.ev[2], a.stream)) != hipSuccess) return e;
    return a.mode == kModeGLA ? launch_chain<kChainGLA>(a) : launch_chain<kChainKDA>(a);
}

hipError_t launch_fast_dplr(const ChunkArgs& a) {
    hipError_t e = launch_dplr_intra(a);
    if (e != hipSuccess) return e;
    if (a.ev && (e = hipEventRecord(a.ev[2], a.stream)) != hipSuccess) return e;
    return launch_chain<kChainDPLR>(a);
}

}  // namespace kda
