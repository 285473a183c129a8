// Chunk bookkeeping for kda_chunk_fwd, done on the device so the host never
// reads cu_seqlens.  Chunks restart at every sequence start and are numbered
// sequence by sequence in token order; a sequence shorter than a multiple of
// the chunk size ends in a short chunk.
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

// Block-wide inclusive scan of one int per thread (1024 threads).
__device__ __forceinline__ int block_scan_1024(int x, int* s_scan) {
    const int t = threadIdx.x;
    s_scan[t] = x;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int y = t >= off ? s_scan[t - off] : 0;
        __syncthreads();
        s_scan[t] += y;
        __syncthreads();
    }
    return s_scan[t];
}

// One workgroup: per-sequence chunk counts and their exclusive prefix sum
// (clamped to the capacity), the total; with seg_chunks > 0 also the
// per-sequence segment counts (seg_chunks chunks per segment) and their prefix.
__global__ __launch_bounds__(1024)
void prep_seq_kernel(const int* __restrict__ cu, int N, int Tfix, int Ttot, int C, int cap,
                     int seg_chunks, int seg_cap, int* __restrict__ hdr,
                     int2* __restrict__ seqs, int2* __restrict__ seqsegs)
{
    __shared__ int s_scan[1024];
    const int t = threadIdx.x;
    long long carry = 0, carry_seg = 0;
    for (int base = 0; base < N; base += 1024) {
        const int s = base + t;
        int start = 0, len = 0;
        if (s < N) seq_extent(cu, s, Tfix, Ttot, start, len);
        const int nch = (len + C - 1) / C;
        const int incl = block_scan_1024(nch, s_scan);
        const int tile_total = s_scan[1023];
        int nc = 0;
        if (s < N) {
            const long long first = carry + incl - nch;
            const int f = (int)min(first, (long long)cap);
            nc = (int)max(0LL, min((long long)nch, (long long)cap - f));
            seqs[s] = make_int2(f, nc);
        }
        __syncthreads();
        if (seg_chunks > 0) {
            const int nseg = (nc + seg_chunks - 1) / seg_chunks;
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
        carry += tile_total;
    }
    if (t == 0) {
        hdr[0] = (int)min(carry, (long long)cap);
        hdr[1] = (int)min(carry_seg, (long long)seg_cap);
    }
}

// One thread per segment slot: owning sequence (binary search over the
// first-segment ids) and (sequence, first chunk, chunks, index in sequence).
__global__ __launch_bounds__(256)
void prep_seg_kernel(int N, int seg_chunks, int seg_cap, const int* __restrict__ hdr,
                     const int2* __restrict__ seqs, const int2* __restrict__ seqsegs,
                     int4* __restrict__ segs)
{
    const int g = blockIdx.x * 256 + threadIdx.x;
    if (g >= seg_cap) return;
    if (g >= hdr[1]) { segs[g] = make_int4(-1, 0, 0, 0); return; }
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seqsegs[mid].x <= g) lo = mid; else hi = mid - 1;
    }
    const int j = g - seqsegs[lo].x;
    const int2 sq = seqs[lo];
    const int first = sq.x + j * seg_chunks;
    segs[g] = make_int4(lo, first, min(seg_chunks, sq.y - j * seg_chunks), j);
}

// One thread per chunk slot: locate the owning sequence by binary search
// over the first-chunk ids and record (sequence, first token, length,
// position of the first token within the sequence).
__global__ __launch_bounds__(256)
void prep_chunk_kernel(const int* __restrict__ cu, int N, int Tfix, int Ttot, int C, int cap,
                       const int* __restrict__ hdr, const int2* __restrict__ seqs,
                       int4* __restrict__ chunks)
{
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= cap) return;
    const int total = hdr[0];
    if (c >= total) { chunks[c] = make_int4(-1, 0, 0, 0); return; }
    // largest s with seqs[s].x <= c; empty sequences share the next one's id,
    // so the largest such s is the non-empty owner
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

hipError_t launch_prep(const ChunkArgs& a) {
    int* hdr = reinterpret_cast<int*>(a.ws);
    int4* chunks = reinterpret_cast<int4*>(a.ws + a.L.off_chunks);
    int2* seqs = reinterpret_cast<int2*>(a.ws + a.L.off_seqs);
    int2* seqsegs = reinterpret_cast<int2*>(a.ws + a.L.off_seqsegs);
    int4* segs = reinterpret_cast<int4*>(a.ws + a.L.off_segs);
    const int Ttot = a.cu ? a.T : a.B * a.T;
    hipLaunchKernelGGL(prep_seq_kernel, dim3(1), dim3(1024), 0, a.stream,
                       a.cu, a.N, a.T, Ttot, a.C, a.L.cap, a.L.seg_chunks, a.L.seg_cap, hdr, seqs,
                       seqsegs);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned nb = (unsigned)((a.L.cap + 255) / 256);
    hipLaunchKernelGGL(prep_chunk_kernel, dim3(nb), dim3(256), 0, a.stream,
                       a.cu, a.N, a.T, Ttot, a.C, a.L.cap, (const int*)hdr, (const int2*)seqs, chunks);
    e = hipGetLastError();
    if (e != hipSuccess || a.L.seg_chunks == 0) return e;
    const unsigned ns = (unsigned)((a.L.seg_cap + 255) / 256);
    hipLaunchKernelGGL(prep_seg_kernel, dim3(ns), dim3(256), 0, a.stream, a.N, a.L.seg_chunks,
                       a.L.seg_cap, (const int*)hdr, (const int2*)seqs, (const int2*)seqsegs, segs);
    return hipGetLastError();
}

}  // namespace kda
