// Grouping of the (token, k) pairs by expert, on the GPU.
//
// Strata compare v0.1.35...v0.1.37 page, include/strata/prefill/moe_fused.hpp,
// group: the fused path sorts the routed pairs by expert on the device,
// straight from the router's output, so the host does not have to wait for
// the routing.  Its tables: where each expert's rows start, which row each
// pair lands in (slot) and which token each row reads (src); work lists of
// row chunks (here at most kChunkRows rows each).  The pages leave the order
// of one expert's rows open; these kernels keep pairs in ascending pair index,
// the order the MMQ path's host counting sort gives (Winery-Strata prefill.cpp
// page, Prefill::run, MoE half), which makes the tables unique and exactly
// comparable.
//
// Three launches, none of which waits on the host (one, group_small_kernel,
// where the pairs fill at most kGroupSmallChunks chunks):
//   hist    one workgroup per chunk of 2048 pairs: LDS histogram of its ids;
//   scan    one workgroup: per expert the exclusive prefix over chunks, the
//           counts' exclusive scan over experts (offsets), and the two lists
//           of row chunks (at most kChunkRows rows of one expert each) the
//           GEMMs walk: chunks of more than kSmallRows rows and the others;
//   scatter one workgroup of 8 waves per chunk, 256 pairs per wave: each
//           lane's rank among the lanes of the same expert comes from ballots
//           over the id bits (multi-split); a first pass counts per wave and
//           expert, a scan over the waves gives each wave's first rows, and a
//           second pass assigns the rows in pair order.
// group_small_kernel does the three in one workgroup for short prompts, which
// otherwise pay three launches' latency for little work: the histogram in
// LDS, the same scan, then the chunks' scatter one after the other with a
// running first row per expert.
#include "internal.h"

namespace strata_moe {

namespace {

__global__ void __launch_bounds__(256) group_hist_kernel(const int32_t* __restrict__ ids, int64_t n, int32_t E,
                                                         int32_t* __restrict__ hist, int32_t* __restrict__ err) {
    __shared__ int32_t h[kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int64_t i0 = (int64_t)blockIdx.x * kGroupChunk;
    const int64_t i1 = i0 + kGroupChunk < n ? i0 + kGroupChunk : n;
    // the thread's kGroupChunk / 256 ids, all loads in flight at once
    constexpr int kPer = kGroupChunk / 256;
    int32_t ev[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int64_t i = i0 + threadIdx.x + 256 * j;
        ev[j] = i < i1 ? ids[i] : 0;
    }
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        if (i0 + threadIdx.x + 256 * j >= i1) continue;
        const int32_t e = ev[j];
        if (e < 0 || e >= E)
            bad = true;
        else
            atomicAdd(&h[e], 1);
    }
    if (bad) atomicOr(err, 1);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

// An expert's rows in chunks of at most kChunkRows, of equal size rounded up to
// whole 16-row tiles (so no chunk is much smaller than the others); returns
// the chunk count and the rows per chunk (the last may have fewer).
__device__ int chunk_split(int cnt, int* per) {
    if (cnt <= 0) {
        *per = 0;
        return 0;
    }
    const int n0 = (cnt + kChunkRows - 1) / kChunkRows;
    const int p = ((cnt + n0 - 1) / n0 + 15) / 16 * 16;
    *per = p;
    return (cnt + p - 1) / p;
}

// Exclusive scans of four values per thread over a workgroup of 1024
// threads, side by side (one pass of barriers for the four): returns the
// four exclusive prefixes, and the four totals in *total.
__device__ int4 block_exclusive_scan4(int4 v, int4* total) {
    __shared__ int4 wsum4[16];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int4 incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int4 o = make_int4(__shfl_up(incl.x, off), __shfl_up(incl.y, off), __shfl_up(incl.z, off),
                                 __shfl_up(incl.w, off));
        if (lane >= off) incl.x += o.x, incl.y += o.y, incl.z += o.z, incl.w += o.w;
    }
    if (lane == 63) wsum4[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        const int4 w = lane < 16 ? wsum4[lane] : make_int4(0, 0, 0, 0);
        int4 wi = w;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int4 o = make_int4(__shfl_up(wi.x, off), __shfl_up(wi.y, off), __shfl_up(wi.z, off),
                                     __shfl_up(wi.w, off));
            if (lane >= off) wi.x += o.x, wi.y += o.y, wi.z += o.z, wi.w += o.w;
        }
        if (lane < 16) wsum4[lane] = make_int4(wi.x - w.x, wi.y - w.y, wi.z - w.z, wi.w - w.w);  // exclusive over waves
        if (lane == 15) *total = wi;
    }
    __syncthreads();
    const int4 b = wsum4[wave];
    const int4 r = make_int4(b.x + incl.x - v.x, b.y + incl.y - v.y, b.z + incl.z - v.z, b.w + incl.w - v.w);
    __syncthreads();
    return r;
}

// Expert e's nt chunks (rows off.. off+cnt, `per` rows each, the last one
// shorter) into the two lists at the expert's offsets in each; toff: the
// expert's first row in the tiled row space (a multiple of 16), where its
// rows follow in order (per is a multiple of 16, so every chunk starts a tile).
__device__ void emit_chunks(const ChunkLists& cl, int e, int off, int cnt, int nt, int per, int bpos, int spos,
                            int toff) {
    for (int i = 0; i < nt; ++i) {
        Tile tl;
        tl.e = e;
        tl.row0 = off + i * per;
        tl.nrows = cnt - i * per < per ? cnt - i * per : per;
        tl.tile0 = (toff + i * per) / 16;
        if (tl.nrows > kSmallRows)
            cl.tiles[bpos++] = tl;
        else
            cl.tiles[cl.cap + spos++] = tl;
        for (int r = 0; r < tl.nrows; r += 16)
            cl.trows[tl.tile0 + r / 16] =
                TileRows{tl.row0 + r, tl.nrows - r < 16 ? tl.nrows - r : 16, tl.nrows > kSmallRows ? 1 : 0};
    }
}

// Chunks of expert e with at most kSmallRows rows (the others are big).
__device__ int small_chunks(int cnt, int nt, int per) {
    int ns = 0;
    for (int i = 0; i < nt; ++i) ns += (cnt - i * per < per ? cnt - i * per : per) <= kSmallRows;
    return ns;
}

// Expert e's entries of the first table (the totals for e = E).
__device__ void write_first(const ChunkLists& cl, int32_t E, int e, int bpos, int spos, int tile) {
    if (!cl.first) return;
    cl.first[e] = bpos;
    cl.first[E + 1 + e] = spos;
    cl.first[2 * (E + 1) + e] = tile;
}

// The list counts and the tile count (one thread).
__device__ void finish_lists(const ChunkLists& cl, int32_t E, int nbig, int nsmall, int tiled_rows) {
    if (threadIdx.x == 0) {
        cl.sched[0] = nbig;
        cl.sched[1] = nsmall;
        cl.sched[2] = tiled_rows / 16;
        write_first(cl, E, E, nbig, nsmall, tiled_rows / 16);
    }
}

__global__ void __launch_bounds__(1024) group_scan_kernel(const int32_t* __restrict__ hist, int64_t nchunks, int64_t n,
                                                          int32_t E, int32_t* __restrict__ base,
                                                          int32_t* __restrict__ offsets, ChunkLists cl) {
    const int e = threadIdx.x;
    int cnt = 0;
    if (e < E) {
        // exclusive prefix over chunks, 8 loads in flight per thread
        int64_t c = 0;
        for (; c + 8 <= nchunks; c += 8) {
            int h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) h[j] = hist[(c + j) * E + e];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                base[(c + j) * E + e] = cnt;
                cnt += h[j];
            }
        }
        for (; c < nchunks; ++c) {
            const int h = hist[c * E + e];
            base[c * E + e] = cnt;
            cnt += h;
        }
    }
    int per = 0;
    const int nt = e < E ? chunk_split(cnt, &per) : 0;
    const int ns = small_chunks(cnt, nt, per);
    __shared__ int4 tot4;
    const int4 pre = block_exclusive_scan4(make_int4(e < E ? cnt : 0, e < E ? (cnt + 15) / 16 * 16 : 0, nt - ns, ns),
                                           &tot4);
    const int off = pre.x, toff = pre.y, bpos = pre.z, spos = pre.w;
    const int total_big = tot4.z, total_small = tot4.w, total_tiled = tot4.y;
    if (e < E) {
        offsets[e] = off;
        emit_chunks(cl, e, off, cnt, nt, per, bpos, spos, toff);
        write_first(cl, E, e, bpos, spos, toff / 16);
    }
    if (e == 0) offsets[E] = (int32_t)n;
    finish_lists(cl, E, total_big, total_small, total_tiled);
}

constexpr int kScatterWaves = kGroupChunk / 256;  // 8 waves of 256 pairs per chunk
// group_small_kernel up to this many chunks: one.  Its chunks' scatter runs
// one after another on one CU; at 5 chunks (1024 tokens, K = 10) it measured
// 55 us against 19 us for the three kernels, at one chunk 13 us against 21
// plus two launch gaps.
constexpr int kGroupSmallChunks = 1;

// The lanes of this wave whose id equals this lane's (all lanes with a valid
// id take part in the ballots); 0 for an invalid id.
__device__ __forceinline__ uint64_t same_expert_lanes(int32_t e, bool ok, int nbits) {
    uint64_t same = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = ok && ((e >> b) & 1);
        const uint64_t m = __ballot(bit);
        same &= bit ? m : ~m;
    }
    return ok ? same : 0ull;
}

// The multi-split scatter of the pairs [i0, i0 + 256) by one wave, as
// group_scatter_kernel's two passes: count[e] gets the wave's count per
// expert (pass 1), then (pass 2, with count[e] set to the wave's first row per
// expert) the rows in pair order.  The wave's ids and weights are loaded once,
// all in flight together (pair i0 + 64 step + lane in entry step of the
// lane), and both passes work from the registers.
struct WavePairs {
    int32_t e[4];  // expert id, -1 past n
    float p[4];    // routing weight (when the rows' weights are wanted)
};
__device__ __forceinline__ WavePairs load_pairs(const int32_t* __restrict__ ids, const float* __restrict__ p,
                                                int64_t n, int64_t i0, int lane) {
    WavePairs v;
#pragma unroll
    for (int step = 0; step < 4; ++step) {
        const int64_t i = i0 + step * 64 + lane;
        v.e[step] = i < n ? ids[i] : -1;
        v.p[step] = p && i < n ? p[i] : 0.0f;
    }
    return v;
}
__device__ __forceinline__ void scatter_count(const WavePairs& v, int32_t E, int nbits, int lane, int32_t* count) {
#pragma unroll
    for (int step = 0; step < 4; ++step) {
        const int32_t e = v.e[step];
        const bool ok = e >= 0 && e < E;
        const uint64_t same = same_expert_lanes(e, ok, nbits);
        if (ok && (same >> lane) == 1ull) count[e] += __popcll(same);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}
__device__ __forceinline__ void scatter_rows(const WavePairs& v, int32_t K, int32_t E, int nbits, int64_t i0,
                                             int lane, int32_t* next, int32_t* __restrict__ src,
                                             int32_t* __restrict__ slot, float* __restrict__ prow) {
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int step = 0; step < 4; ++step) {
        const int64_t i = i0 + step * 64 + lane;
        const int32_t e = v.e[step];
        const bool ok = e >= 0 && e < E;
        const uint64_t same = same_expert_lanes(e, ok, nbits);
        const int rank = __popcll(same & below);
        const int first = ok ? next[e] : 0;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (ok) {
            const int row = first + rank;
            slot[i] = row;
            src[row] = (int32_t)(i / K);
            if (prow) prow[row] = v.p[step];
            if ((same >> lane) == 1ull) next[e] = first + __popcll(same);  // the highest lane of this expert
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    }
}

__global__ void __launch_bounds__(64 * kScatterWaves) group_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ p, int64_t n, int32_t K, int32_t E,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offsets, int32_t* __restrict__ src,
    int32_t* __restrict__ slot, float* __restrict__ prow) {
    __shared__ int32_t next[kScatterWaves][kMaxExperts];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int i = threadIdx.x; i < kScatterWaves * E; i += blockDim.x) next[i / E][i % E] = 0;
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const int64_t i0 = (int64_t)blockIdx.x * kGroupChunk + 256 * w;
    const WavePairs v = load_pairs(ids, prow ? p : nullptr, n, i0, lane);
    scatter_count(v, E, nbits, lane, next[w]);
    __syncthreads();
    // each wave's first row per expert: the chunk's first row, then the waves before it
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int run = offsets[e] + base[(int64_t)blockIdx.x * E + e];
        for (int ww = 0; ww < kScatterWaves; ++ww) {
            const int t = next[ww][e];
            next[ww][e] = run;
            run += t;
        }
    }
    __syncthreads();
    scatter_rows(v, K, E, nbits, i0, lane, next[w], src, slot, prow);
}

// All of the grouping in one workgroup of 1024 threads, for n pairs in at
// most kGroupSmallChunks chunks of kGroupChunk: the same tables as the three
// kernels (the same scan; the scatter's order is pair order either way).
__global__ void __launch_bounds__(1024) group_small_kernel(const int32_t* __restrict__ ids,
                                                           const float* __restrict__ p, int64_t n, int32_t K,
                                                           int32_t E, int32_t* __restrict__ offsets, ChunkLists cl,
                                                           int32_t* __restrict__ src, int32_t* __restrict__ slot,
                                                           float* __restrict__ prow, int32_t* __restrict__ err) {
    __shared__ int32_t cur[kMaxExperts];  // counts, then each expert's next free row
    __shared__ int32_t next[kScatterWaves][kMaxExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cur[e] = 0;
    __syncthreads();
    bool bad = false;
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
        const int32_t e = ids[i];
        if (e < 0 || e >= E)
            bad = true;
        else
            atomicAdd(&cur[e], 1);
    }
    if (bad) atomicOr(err, 1);
    __syncthreads();
    const int e = threadIdx.x;
    const int cnt = e < E ? cur[e] : 0;
    int per = 0;
    const int nt = e < E ? chunk_split(cnt, &per) : 0;
    const int ns = small_chunks(cnt, nt, per);
    __shared__ int4 tot4;
    const int4 pre = block_exclusive_scan4(make_int4(cnt, (cnt + 15) / 16 * 16, nt - ns, ns), &tot4);
    const int off = pre.x, toff = pre.y, bpos = pre.z, spos = pre.w;
    const int total_big = tot4.z, total_small = tot4.w, total_tiled = tot4.y;
    if (e < E) {
        offsets[e] = off;
        emit_chunks(cl, e, off, cnt, nt, per, bpos, spos, toff);
        write_first(cl, E, e, bpos, spos, toff / 16);
        cur[e] = off;
    }
    if (e == 0) offsets[E] = (int32_t)n;
    finish_lists(cl, E, total_big, total_small, total_tiled);
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int64_t c0 = 0; c0 < n; c0 += kGroupChunk) {
        for (int i = threadIdx.x; i < kScatterWaves * E; i += blockDim.x) next[i / E][i % E] = 0;
        __syncthreads();  // also orders the cur[] writes above and the last chunk's rows
        WavePairs v{};
        if (w < kScatterWaves) {
            v = load_pairs(ids, prow ? p : nullptr, n, c0 + 256 * w, lane);
            scatter_count(v, E, nbits, lane, next[w]);
        }
        __syncthreads();
        for (int ee = threadIdx.x; ee < E; ee += blockDim.x) {
            int run = cur[ee];
            for (int ww = 0; ww < kScatterWaves; ++ww) {
                const int t = next[ww][ee];
                next[ww][ee] = run;
                run += t;
            }
            cur[ee] = run;
        }
        __syncthreads();
        if (w < kScatterWaves) scatter_rows(v, K, E, nbits, c0 + 256 * w, lane, next[w], src, slot, prow);
        __syncthreads();
    }
}

// The chunk lists of a given grouping (offsets from the caller).  An expert
// whose rows are not inside [0, n) gets none: the lists and tiled rows never
// index past their buffers, whatever the offsets hold.
__global__ void __launch_bounds__(1024) chunks_from_offsets_kernel(const int32_t* __restrict__ offsets, int32_t E,
                                                                   int64_t n, ChunkLists cl) {
    const int e = threadIdx.x;
    int cnt = e < E ? offsets[e + 1] - offsets[e] : 0;
    if (e < E && (offsets[e] < 0 || cnt < 0 || offsets[e + 1] > n)) cnt = 0;
    int per = 0;
    const int nt = chunk_split(cnt, &per);
    const int ns = small_chunks(cnt, nt, per);
    __shared__ int4 tot4;
    const int4 pre = block_exclusive_scan4(make_int4(0, (cnt + 15) / 16 * 16, nt - ns, ns), &tot4);
    const int toff = pre.y, bpos = pre.z, spos = pre.w;
    const int total_big = tot4.z, total_small = tot4.w, total_tiled = tot4.y;
    if (e < E) {
        emit_chunks(cl, e, offsets[e], cnt, nt, per, bpos, spos, toff);
        write_first(cl, E, e, bpos, spos, toff / 16);
    }
    finish_lists(cl, E, total_big, total_small, total_tiled);
}

__global__ void row_weights_kernel(const int32_t* __restrict__ slot, const float* __restrict__ p, int64_t n,
                                   float* __restrict__ prow) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) prow[slot[i]] = p[i];
}

}  // namespace

hipError_t launch_group(const int32_t* ids, const float* p, int64_t n, int32_t K, int32_t E, int32_t* hist,
                        int32_t* base, int32_t* offsets, const ChunkLists& cl, int32_t* src, int32_t* slot,
                        float* prow, int32_t* err, hipStream_t st) {
    const int64_t nchunks = (n + kGroupChunk - 1) / kGroupChunk;
    if (nchunks > 0 && nchunks <= kGroupSmallChunks) {
        hipLaunchKernelGGL(group_small_kernel, dim3(1), dim3(1024), 0, st, ids, p, n, K, E, offsets, cl, src, slot,
                           prow, err);
    } else if (nchunks > 0) {
        hipLaunchKernelGGL(group_hist_kernel, dim3((unsigned)nchunks), dim3(256), 0, st, ids, n, E, hist, err);
        hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), 0, st, hist, nchunks, n, E, base, offsets, cl);
        hipLaunchKernelGGL(group_scatter_kernel, dim3((unsigned)nchunks), dim3(64 * kScatterWaves), 0, st, ids, p,
                           n, K, E, base, offsets, src, slot, prow);
    } else {
        hipLaunchKernelGGL(group_scan_kernel, dim3(1), dim3(1024), 0, st, hist, (int64_t)0, (int64_t)0, E, base,
                           offsets, cl);
    }
    return hipGetLastError();
}

hipError_t launch_chunks_from_offsets(const int32_t* offsets, int32_t E, int64_t n, const ChunkLists& cl,
                                      hipStream_t st) {
    hipLaunchKernelGGL(chunks_from_offsets_kernel, dim3(1), dim3(1024), 0, st, offsets, E, n, cl);
    return hipGetLastError();
}

hipError_t launch_row_weights(const int32_t* slot, const float* p, int64_t n, float* prow, hipStream_t st) {
    if (n > 0)
        hipLaunchKernelGGL(row_weights_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, slot, p, n,
                           prow);
    return hipGetLastError();
}

}  // namespace strata_moe
