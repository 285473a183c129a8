// Chunk bookkeeping for kda_chunk_fwd, done on the device so the host never
// reads cu_seqlens.  Chunks restart at every sequence start and are numbered
// sequence by sequence in token order; a sequence shorter than a multiple of
// the chunk size ends in a short chunk.  A batch without cu_seqlens on the
// MFMA path is planned on the host instead (plan_fixed), and the intra launch
// writes its tables.
#include <algorithm>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

__device__ __forceinline__ void seq_extent(const int* cu, int s, int Tfix, int Ttot,
                                           int& start, int& len) {
    if (cu) {
        int a = cu[s], e = cu[s + 1];
        a = min(max(a, 0), Ttot);
        e = min(max(e, a), Ttot);
        start = a;
        len = e - a;
    } else {
        start = s * Tfix;
        len = Tfix;
    }
}

// Block-wide inclusive scan of one int per thread (1024 threads): a scan
// inside each wave, then the wave totals.  Every thread also finds the block
// total in s_scan[1023] until the next call.
__device__ __forceinline__ int block_scan_1024(int x, int* s_scan) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_scan[w] = x;
    __syncthreads();
    int before = 0, total = 0;
    for (int i = 0; i < 16; i++) {
        const int v = s_scan[i];
        if (i < w) before += v;
        total += v;
    }
    __syncthreads();                            // every wave has read the totals
    if (t == 1023) s_scan[1023] = total;
    __syncthreads();
    return before + x;
}

// Block-wide sum (or maximum) of one int per thread (1024 threads), returned
// to every thread; s_red holds 16 ints.
template <bool MAX>
__device__ __forceinline__ int block_reduce_1024(int x, int* s_red) {
    for (int m = 32; m > 0; m >>= 1) {
        const int y = __shfl_xor(x, m, 64);
        x = MAX ? max(x, y) : x + y;
    }
    if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = x;
    __syncthreads();
    int r = s_red[0];
    for (int i = 1; i < 16; i++) r = MAX ? max(r, s_red[i]) : r + s_red[i];
    __syncthreads();                            // s_red may be written again
    return r;
}

// Sum over the N sequences of ceil(chunks / per): the segments that `per`
// chunks per segment give (seqs[].y are the clamped chunk counts).
__device__ long long count_segments(const int2* __restrict__ seqs, int N, int per, int* s_red) {
    long long total = 0;
    for (int base = 0; base < N; base += 1024) {
        const int s = base + threadIdx.x;
        const int nc = s < N ? seqs[s].y : 0;
        total += block_reduce_1024<false>((nc + per - 1) / per, s_red);
    }
    return total;
}

// Segment slot g: owning sequence (binary search over the first-segment ids)
// and (sequence, first chunk, chunks, index in sequence); -1 past the total.
__device__ __forceinline__ void fill_seg(int g, int N, int nseg_total, int per,
                                         const int2* __restrict__ seqs,
                                         const int2* __restrict__ seqsegs, int4* __restrict__ segs) {
    if (g >= nseg_total) { segs[g] = make_int4(-1, 0, 0, 0); return; }
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seqsegs[mid].x <= g) lo = mid; else hi = mid - 1;
    }
    const int j = g - seqsegs[lo].x;
    const int2 sq = seqs[lo];
    segs[g] = make_int4(lo, sq.x + j * per, min(per, sq.y - j * per), j);
}

// Chunk slot c: the owning sequence by binary search over the first-chunk
// ids (empty sequences share the next one's id, so the largest s with
// seqs[s].x <= c is the non-empty owner) and (sequence, first token, length,
// position of the first token within the sequence); -1 past the total.
__device__ __forceinline__ void fill_chunk(int c, const int* __restrict__ cu, int N, int Tfix,
                                           int Ttot, int C, int total,
                                           const int2* __restrict__ seqs, int4* __restrict__ chunks) {
    if (c >= total) { chunks[c] = make_int4(-1, 0, 0, 0); return; }
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seqs[mid].x <= c) lo = mid; else hi = mid - 1;
    }
    int start, len;
    seq_extent(cu, lo, Tfix, Ttot, start, len);
    const int j = c - seqs[lo].x;
    chunks[c] = make_int4(lo, start + j * C, min(C, len - j * C), j * C);
}

// The chunk bookkeeping in one workgroup (one launch): per-sequence chunk
// counts and their exclusive prefix sum (clamped to the capacity), the
// total, the chunk table; with min_seg > 0 also the segments of the MFMA
// chain and the segment table.  Both chain launches run one workgroup per (segment, head),
// so the segment length `per` is the smallest value >= min_seg whose segments
// (each sequence cut into ceil(chunks / per)) number at most seg_target (or
// one per non-empty sequence when there are more of those): one round of
// workgroups whose longest chain is as short as that round allows.  Any such
// per gives at most cap / min_seg + N segments, the capacity the host sized.
// hdr: [0] chunks, [1] segments, [2] per.
__global__ __launch_bounds__(1024)
void prep_kernel(const int* __restrict__ cu, int N, int Tfix, int Ttot, int C, int cap,
                 int min_seg, int seg_target, int seg_cap, int* __restrict__ hdr,
                 int2* __restrict__ seqs, int2* __restrict__ seqsegs, int4* __restrict__ chunks,
                 int4* __restrict__ segs)
{
    __shared__ int s_scan[1024];
    const int t = threadIdx.x;
    long long carry = 0;
    for (int base = 0; base < N; base += 1024) {
        const int s = base + t;
        int start = 0, len = 0;
        if (s < N) seq_extent(cu, s, Tfix, Ttot, start, len);
        const int nch = (len + C - 1) / C;
        const int incl = block_scan_1024(nch, s_scan);
        const int tile_total = s_scan[1023];
        if (s < N) {
            const long long first = carry + incl - nch;
            const int f = (int)min(first, (long long)cap);
            const int nc = (int)max(0LL, min((long long)nch, (long long)cap - f));
            seqs[s] = make_int2(f, nc);
        }
        __syncthreads();
        carry += tile_total;
    }
    int per = 0;
    long long carry_seg = 0;
    if (min_seg > 0) {
        __syncthreads();                        // seqs[] complete for the whole workgroup
        int max_nc = 0;
        for (int base = 0; base < N; base += 1024) {
            const int s = base + t;
            max_nc = max(max_nc, block_reduce_1024<true>(s < N ? seqs[s].y : 0, s_scan));
        }
        const long long total = min(carry, (long long)cap);
        const long long nonempty = count_segments(seqs, N, max(max_nc, 1), s_scan);
        const long long target = max((long long)seg_target, nonempty);
        // count_segments(per) is non-increasing in per, at least total / per and
        // at most total / per + nonempty: the answer lies in [lo, hi]
        long long lo = max((long long)min_seg, (total + target - 1) / target);
        long long hi = target > nonempty ? (total + (target - nonempty) - 1) / (target - nonempty)
                                         : (long long)max_nc;
        hi = max(hi, lo);
        if (count_segments(seqs, N, (int)lo, s_scan) <= target) hi = lo;   // one sequence: always
        while (lo < hi) {
            const long long mid = lo + (hi - lo) / 2;
            if (count_segments(seqs, N, (int)mid, s_scan) <= target) hi = mid; else lo = mid + 1;
        }
        per = (int)lo;
        for (int base = 0; base < N; base += 1024) {
            const int s = base + t;
            const int nc = s < N ? seqs[s].y : 0;
            const int nseg = (nc + per - 1) / per;
            const int sincl = block_scan_1024(nseg, s_scan);
            if (s < N) {
                const long long first = carry_seg + sincl - nseg;
                const int f = (int)min(first, (long long)seg_cap);
                const int ns = (int)max(0LL, min((long long)nseg, (long long)seg_cap - f));
                seqsegs[s] = make_int2(f, ns);
            }
            carry_seg += s_scan[1023];
            __syncthreads();
        }
    }
    const int total = (int)min(carry, (long long)cap);
    const int nseg_total = (int)min(carry_seg, (long long)seg_cap);
    if (t == 0) {
        hdr[0] = total;
        hdr[1] = nseg_total;
        hdr[2] = per;
    }
    __syncthreads();                            // seqs[] and seqsegs[] complete
    for (int c = t; c < cap; c += 1024) fill_chunk(c, cu, N, Tfix, Ttot, C, total, seqs, chunks);
    if (min_seg > 0)
        for (int g = t; g < seg_cap; g += 1024) fill_seg(g, N, nseg_total, per, seqs, seqsegs, segs);
}

// Sum and maximum over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ long long wave_sum64(long long x) {
    for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}
__device__ __forceinline__ int wave_max(int x) {
    for (int m = 32; m > 0; m >>= 1) x = max(x, __shfl_xor(x, m, 64));
    return x;
}

// The same bookkeeping for batches of at most 64 sequences: wave 0 (lane s =
// sequence s) does every scan, reduction and the search for the segment
// length with cross-lane operations, and leaves the per-sequence tables in
// LDS; after one barrier the whole workgroup fills the chunk and segment
// tables.  Same results as prep_kernel.
__global__ __launch_bounds__(1024)
void prep_small_kernel(const int* __restrict__ cu, int N, int Tfix, int Ttot, int C, int cap,
                       int min_seg, int seg_target, int seg_cap, int* __restrict__ hdr,
                       int2* __restrict__ seqs, int2* __restrict__ seqsegs,
                       int4* __restrict__ chunks, int4* __restrict__ segs)
{
    __shared__ int2 s_seqs[64], s_seqsegs[64];
    __shared__ int s_hdr[3];
    const int t = threadIdx.x;
    if (t < 64) {
        const int s = t;
        int start = 0, len = 0;
        if (s < N) seq_extent(cu, s, Tfix, Ttot, start, len);
        const long long nch = (len + C - 1) / C;
        long long incl = nch;
        for (int d = 1; d < 64; d <<= 1) {
            const long long y = __shfl_up(incl, d, 64);
            if (s >= d) incl += y;
        }
        const long long carry = __shfl(incl, 63, 64);
        const int f = (int)min(incl - nch, (long long)cap);
        const int nc = (int)max(0LL, min(nch, (long long)cap - f));
        if (s < N) {
            s_seqs[s] = make_int2(f, nc);
            seqs[s] = make_int2(f, nc);
        }
        auto count = [&](long long per) { return wave_sum64(s < N ? (nc + per - 1) / per : 0); };
        int per = 0;
        long long carry_seg = 0;
        if (min_seg > 0) {
            const int max_nc = wave_max(s < N ? nc : 0);
            const long long total = min(carry, (long long)cap);
            const long long nonempty = count(max(max_nc, 1));
            const long long target = max((long long)seg_target, nonempty);
            long long lo = max((long long)min_seg, (total + target - 1) / target);
            long long hi = target > nonempty ? (total + (target - nonempty) - 1) / (target - nonempty)
                                             : (long long)max_nc;
            hi = max(hi, lo);
            if (count(lo) <= target) hi = lo;
            while (lo < hi) {
                const long long mid = lo + (hi - lo) / 2;
                if (count(mid) <= target) hi = mid; else lo = mid + 1;
            }
            per = (int)lo;
            const long long nseg = s < N ? (nc + per - 1) / per : 0;
            long long sincl = nseg;
            for (int d = 1; d < 64; d <<= 1) {
                const long long y = __shfl_up(sincl, d, 64);
                if (s >= d) sincl += y;
            }
            carry_seg = __shfl(sincl, 63, 64);
            const int fs = (int)min(sincl - nseg, (long long)seg_cap);
            const int ns = (int)max(0LL, min(nseg, (long long)seg_cap - fs));
            if (s < N) {
                s_seqsegs[s] = make_int2(fs, ns);
                seqsegs[s] = make_int2(fs, ns);
            }
        }
        if (s == 0) {
            s_hdr[0] = (int)min(carry, (long long)cap);
            s_hdr[1] = (int)min(carry_seg, (long long)seg_cap);
            s_hdr[2] = per;
            hdr[0] = s_hdr[0];
            hdr[1] = s_hdr[1];
            hdr[2] = per;
        }
    }
    __syncthreads();
    const int total = s_hdr[0], nseg_total = s_hdr[1], per = s_hdr[2];
    for (int c = t; c < cap; c += 1024) fill_chunk(c, cu, N, Tfix, Ttot, C, total, s_seqs, chunks);
    if (min_seg > 0)
        for (int g = t; g < seg_cap; g += 1024) fill_seg(g, N, nseg_total, per, s_seqs, s_seqsegs, segs);
}

// The bookkeeping of N sequences of T tokens each, on the host: every
// sequence has the same chunk count, so the per-sequence scans are products
// and the segment length is found by the search of the kernels above on the
// same integers.
FixedPlan plan_fixed(int N, int T, int C, int H, const WsLayout& L, uint8_t* ws) {
    FixedPlan p{};
    p.on = 1;
    p.N = N; p.T = T; p.C = C;
    p.cps = (T + C - 1) / C;
    p.cap = L.cap; p.seg_cap = L.seg_cap;
    const long long total = std::min((long long)N * p.cps, (long long)L.cap);
    p.total = (int)total;
    auto count = [&](long long per) { return (long long)N * ((p.cps + per - 1) / per); };
    const int max_nc = p.cps;
    const long long nonempty = count(std::max(max_nc, 1));
    const long long target = std::max((long long)seg_target(H), nonempty);
    long long lo = std::max((long long)L.seg_chunks, (total + target - 1) / target);
    long long hi = target > nonempty ? (total + (target - nonempty) - 1) / (target - nonempty)
                                     : (long long)max_nc;
    hi = std::max(hi, lo);
    if (count(lo) <= target) hi = lo;
    while (lo < hi) {
        const long long mid = lo + (hi - lo) / 2;
        if (count(mid) <= target) hi = mid; else lo = mid + 1;
    }
    p.per = (int)lo;
    p.nseg = (p.cps + p.per - 1) / p.per;
    p.nseg_total = (int)std::min((long long)N * p.nseg, (long long)L.seg_cap);
    p.hdr = reinterpret_cast<int*>(ws);
    p.seqs = reinterpret_cast<int2*>(ws + L.off_seqs);
    p.seqsegs = reinterpret_cast<int2*>(ws + L.off_seqsegs);
    p.chunks = reinterpret_cast<int4*>(ws + L.off_chunks);
    p.segs = reinterpret_cast<int4*>(ws + L.off_segs);
    return p;
}

hipError_t launch_prep(const ChunkArgs& a) {
    int* hdr = reinterpret_cast<int*>(a.ws);
    int4* chunks = reinterpret_cast<int4*>(a.ws + a.L.off_chunks);
    int2* seqs = reinterpret_cast<int2*>(a.ws + a.L.off_seqs);
    int2* seqsegs = reinterpret_cast<int2*>(a.ws + a.L.off_seqsegs);
    int4* segs = reinterpret_cast<int4*>(a.ws + a.L.off_segs);
    const int Ttot = a.cu ? a.T : a.B * a.T;
    if (a.N <= 64)
        hipLaunchKernelGGL(prep_small_kernel, dim3(1), dim3(1024), 0, a.stream,
                           a.cu, a.N, a.T, Ttot, a.C, a.L.cap, a.L.seg_chunks, seg_target(a.H),
                           a.L.seg_cap, hdr, seqs, seqsegs, chunks, segs);
    else
        hipLaunchKernelGGL(prep_kernel, dim3(1), dim3(1024), 0, a.stream,
                           a.cu, a.N, a.T, Ttot, a.C, a.L.cap, a.L.seg_chunks, seg_target(a.H),
                           a.L.seg_cap, hdr, seqs, seqsegs, chunks, segs);
    return hipGetLastError();
}

}  // namespace kda
