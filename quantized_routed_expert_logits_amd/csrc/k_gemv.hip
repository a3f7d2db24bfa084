// Grouped expert GEMV for chunks of a few routed rows (at most max_rows, two
// per pass over the weights): the decode-window end of the prompt path,
// where most hit experts get one or two rows.  There the MFMA kernels' fp16 unpack of the 2-bit codes dominates
// (25 vector instructions per 16 codes) while the matrix unit idles; this
// kernel works on int8 codes with v_dot4_i32_i8 instead.
//
// Strata compare v0.1.35...v0.1.37 page, include/strata/prefill/moe_fused.hpp,
// experts(): per expert, gate/up on the int8 activation rows of its routed
// rows, SwiGLU, H rounded to int8 per 32 values, down into the per-slot rows
// the combine reads; the pages' int8 path multiplies s8 codes with s8 codes
// into s32 (mma.sync m16n8k32); dot4 is the same product four at a time.
//
// Arithmetic.  A weight block is 32 codes q with an fp16 d; w = d (q - z),
// z = 1.5 (symmetric map) or 1 (Q2_0).  Against an int8 activation block a
// the block's sum is an exact int32: P = sum (q - 1) a - 0 for Q2_0, and for
// the symmetric map 2 sum (q - 1.5) a = sum (2q) a - 3 sum a.  The kernel
// takes the raw codes (doubled for the symmetric map) straight out of the
// record with shifts and masks, and starts the int32 dot-product chain at the
// offset term -z' sum a (z' = 1 or 3); the output adds fp32(P) * s * d, and
// the symmetric map's factor 1/2 is applied once at the end.  The per-token
// form computes each lane's part of sum a with two more dot4 against ones;
// the per-slot q8_1 arm (the pages' MMQ form, an A/B alternative) reads
// activations quantized per routed slot with their block code sums instead,
// and only the first lane of a row adds the offset.
//
// Work split.  A workgroup (4 waves) takes one chunk and 4 / S consecutive
// 128-row slabs; the S waves of a slab split the reduction into S equal runs
// of blocks (S = 4, 2 or 1, the largest that leaves runs of at least 16
// blocks in whole ring turns).  The packed records are those of the MFMA
// kernels: lane l holds the 8 codes k = 8 (l / 16) .. + 7 of rows l % 16 +
// 16 f, f = 0..7, in its 16 record bytes.  Each lane accumulates its k range;
// the four lanes of a row add their sums, then the slab's first wave adds the
// other waves' sums from LDS in wave order (a fixed order: the result does
// not depend on timing) and stores.  Short waves in numbers well above the
// chip's resident capacity let the dispatcher balance the SIMDs; one wave
// per slab over the whole reduction left some SIMDs with a wave more than
// others and every wave a long serial chain of loads.
// Blocks stream through a register ring kDepth = 2 deep: a block's codes,
// weight scales, activation codes and activation scales (and code sums) are
// all loaded two blocks before their use, so no load is waited on in the
// block it is used (every run has even length).  A 4-deep ring measured the
// same for gate/up and 4 us slower for down at 32 tokens; the 2-deep one
// fits in 74 VGPRs, 6 waves per SIMD.
#include "internal.h"

namespace strata_moe {

namespace {

constexpr int kWaves = 4;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3 for raw dword loads on gfx9 (gfx950)
constexpr int kOnes = 0x01010101;         // four int8 ones: dot4 against them sums four codes

struct GemvArgs {
    const uint8_t* blobs;  // packed matrices: expert e at blobs + e * stride, or in its ring slot
    int64_t stride;
    int64_t ring0;
    int32_t nring;
    const Tile* chunks;      // the small-chunk list
    const int32_t* nchunks;  // its length
    const int32_t* first;    // optional expert range [e0, e1) through the grouping's first table
    int32_t e0, e1;
    int32_t nslab, Kd;
    int32_t nsplit;       // S: waves per slab, each on nblk / S consecutive blocks
    int32_t max_rows;     // the chunks of at most this many rows are this kernel's
    const int32_t* src;   // gate/up without the per-slot arm: token of each grouped row
    const int8_t* act;    // int8 activation rows [act_rows][Kd]
    int64_t act_rows;
    const float* ascale;  // their block scales [act_rows][Kd / 32]
    const int32_t* asum;  // per-slot arm: their block code sums [act_rows][Kd / 32], else null
    const float* prow;    // down: routing weight of each grouped row
    int32_t I, H;
    int8_t* hq;  // gate/up: H codes [n][I]
    float* hs;   // gate/up: H scales [n][I / 32]
    float* y;    // down: weighted routed rows [n][H]
};

__device__ __forceinline__ const uint8_t* gemv_blob(const GemvArgs& g, int e) {
    const int64_t slot = g.nring > 0 ? (g.ring0 + e) % g.nring : (int64_t)e;
    return g.blobs + slot * g.stride;
}

__device__ __forceinline__ float round_half_away(float t) {
    const float r = floorf(fabsf(t) + 0.5f);
    return copysignf(fminf(r, 127.0f), t);
}

// One record dword -> the codes of its two rows as int8 (q, or 2q for the
// symmetric map): lo[0] / hi[0] = row A (fragment 2p) k 0..3 / 4..7, lo[1] /
// hi[1] = row B.  Bits 2j, 2j+1 of each byte hold code k = 2j (bytes 0, 1:
// rows A, B) or k = 2j + 1 (bytes 2, 3).
template <bool kSym>
__device__ __forceinline__ void row_codes(uint32_t w, uint32_t (&lo)[2], uint32_t (&hi)[2]) {
    uint32_t x[4];
    if constexpr (kSym) {
        x[0] = (w << 1) & 0x06060606u;
#pragma unroll
        for (int j = 1; j < 4; ++j) x[j] = (w >> (2 * j - 1)) & 0x06060606u;
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = (w >> (2 * j)) & 0x03030303u;
    }
    lo[0] = __builtin_amdgcn_perm(x[1], x[0], 0x06040200u);  // A: k0 k1 k2 k3
    hi[0] = __builtin_amdgcn_perm(x[3], x[2], 0x06040200u);  // A: k4 k5 k6 k7
    lo[1] = __builtin_amdgcn_perm(x[1], x[0], 0x07050301u);  // B
    hi[1] = __builtin_amdgcn_perm(x[3], x[2], 0x07050301u);
}

// The loads of one block of the ring.
template <int R>
struct RingSlot {
    uint32_t c[4];     // the lane's 16 code bytes
    uint32_t sw[4];    // its row's 8 fp16 weight scales
    uint32_t a[R][2];  // per activation row its 8 codes of the lane's k range
    float s[R];        // per activation row the block scale
    int32_t A[R];      // per-slot arm: per activation row the block code sum
};

// Lane sums of the slab's other waves: [wave][row r16][fragment][row i].
constexpr int kRedFloats = 16 * 8 * kGemvRows;

// One wave: chunk tl (R rows) against slab `slab`, blocks [b0, b0 + nb) of
// the reduction.  `part` is the wave's place among the slab's waves (0: the
// one that stores); red: the workgroup's LDS sums; live: the slab exists (a
// wave without one still meets the barrier).
template <bool kGateUp, bool kQ81, bool kSym, int R, int kDepth>
__device__ __forceinline__ void gemv_wave(const GemvArgs& g, const Tile& tl, int slab, int part, int lane,
                                          bool live, float (*red)[kRedFloats]) {
    const int r16 = lane & 15, kg = lane >> 4;
    const int nblk = g.Kd / kBlock;
    const int nb = nblk / g.nsplit, b0 = part * nb;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int arow[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int row = tl.row0 + i;
        arow[i] = (kGateUp && !kQ81) ? g.src[row] : row;
    }
    const uint8_t* rec = gemv_blob(g, tl.e) + ((int64_t)(live ? slab : 0) * nblk + b0) * kRecordBytes;
    const __amdgpu_buffer_rsrc_t rrec = __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, nb * kRecordBytes,
                                                                          kBufferWord3);
    const __amdgpu_buffer_rsrc_t ract = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.act, (short)0, (int)(g.act_rows * g.Kd), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rscl = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.ascale, (short)0, (int)(g.act_rows * nblk * 4), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsum = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.asum, (short)0, kQ81 ? (int)(g.act_rows * nblk * 4) : 0, kBufferWord3);
    constexpr int zp = kSym ? 3 : 1;  // the offset's multiple of the code sum
    float acc[8][R];
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int i = 0; i < R; ++i) acc[f][i] = 0.f;

    // Block b of the run (a block beyond the run re-reads its last one, never
    // used).  The activation scale and sum addresses are the same on every
    // lane.
    auto load = [&](int b, RingSlot<R>& r) {
        b = b < nb ? b : nb - 1;
        const int ab = b0 + b;  // the block in the activation row
        const auto cv = __builtin_amdgcn_raw_buffer_load_b128(rrec, lane * 16, b * kRecordBytes, 0);
        const auto dv = __builtin_amdgcn_raw_buffer_load_b128(rrec, kRecordCodeBytes + r16 * 16, b * kRecordBytes, 0);
#pragma unroll
        for (int p = 0; p < 4; ++p) r.c[p] = cv[p], r.sw[p] = dv[p];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const auto av = __builtin_amdgcn_raw_buffer_load_b64(ract, arow[i] * g.Kd + 8 * kg, ab * kBlock, 0);
            r.a[i][0] = av[0];
            r.a[i][1] = av[1];
            r.s[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rscl, 0, (arow[i] * nblk + ab) * 4, 0));
            if constexpr (kQ81)
                r.A[i] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rsum, 0, (arow[i] * nblk + ab) * 4, 0);
        }
    };
    RingSlot<R> ring[kDepth];
    // issued slot by slot: the loop waits for a slot's loads by their count
    // (vmcnt), which only works if no later slot's loads went out before them
#pragma unroll
    for (int j = 0; j < kDepth; ++j) {
        load(j, ring[j]);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int b = 0; live && b < nb; b += kDepth) {
#pragma unroll
        for (int j = 0; j < kDepth; ++j) {
            const int blk = b + j;
            RingSlot<R>& r = ring[j];
            int32_t z[R];  // the chain's start: minus the offset term of this lane's part
#pragma unroll
            for (int i = 0; i < R; ++i) {
                if constexpr (kQ81) {
                    z[i] = kg == 0 ? -zp * r.A[i] : 0;
                } else {
                    int32_t sa = __builtin_amdgcn_sdot4((int)r.a[i][0], kOnes, 0, false);
                    sa = __builtin_amdgcn_sdot4((int)r.a[i][1], kOnes, sa, false);
                    z[i] = __mul24(sa, -zp);  // |sa| <= 8 * 127: a full-rate 24-bit multiply
                }
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t lo[2], hi[2];
                row_codes<kSym>(r.c[p], lo, hi);
                const float d0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.sw[p] & 0xffffu));
                const float d1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(r.sw[p] >> 16));
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    int32_t pa = __builtin_amdgcn_sdot4((int)lo[0], (int)r.a[i][0], z[i], false);
                    pa = __builtin_amdgcn_sdot4((int)hi[0], (int)r.a[i][1], pa, false);
                    int32_t pb = __builtin_amdgcn_sdot4((int)lo[1], (int)r.a[i][0], z[i], false);
                    pb = __builtin_amdgcn_sdot4((int)hi[1], (int)r.a[i][1], pb, false);
                    acc[2 * p][i] = fmaf((float)pa * r.s[i], d0, acc[2 * p][i]);
                    acc[2 * p + 1][i] = fmaf((float)pb * r.s[i], d1, acc[2 * p + 1][i]);
                }
            }
            // the slot's registers are free again: its next block's loads
            // go there (kept after the products, so the ring holds kDepth
            // blocks, not kDepth + 1)
            __builtin_amdgcn_sched_barrier(0);
            load(blk + kDepth, r);
        }
    }
    // the four lanes of a row (k ranges kg = 0..3) add their sums
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float v = acc[f][i];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[f][i] = v;
        }
    if (g.nsplit > 1) {  // uniform over the workgroup
        if (part != 0 && kg == 0)
#pragma unroll
            for (int f = 0; f < 8; ++f)
#pragma unroll
                for (int i = 0; i < R; ++i) red[wave][(r16 * 8 + f) * kGemvRows + i] = acc[f][i];
        __syncthreads();
        if (part == 0)
            for (int q = 1; q < g.nsplit; ++q)
#pragma unroll
                for (int f = 0; f < 8; ++f)
#pragma unroll
                    for (int i = 0; i < R; ++i) acc[f][i] += red[wave + q][(r16 * 8 + f) * kGemvRows + i];
        __syncthreads();  // red is free for the chunk's next pass
    }
    if (!live || part != 0) return;
    constexpr float half = kSym ? 0.5f : 1.0f;  // the symmetric map's codes are 2 (q - 1.5)
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int i = 0; i < R; ++i) acc[f][i] *= half;
    if constexpr (kGateUp) {
        // fragments f < 4: gate rows j = 64 slab + 16 f + r16; f + 4: the up rows of the same j.
        // H block hb (32 values) holds fragments 2 hb, 2 hb + 1 of the 16 lanes r16.
        const int nbi = g.I / kBlock;
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t row = tl.row0 + i;
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                float h[2];
                float amax = 0.f;
#pragma unroll
                for (int ff = 0; ff < 2; ++ff) {
                    const float gt = acc[2 * hb + ff][i], up = acc[4 + 2 * hb + ff][i];
                    h[ff] = gt * up * __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
                    amax = fmaxf(amax, fabsf(h[ff]));
                }
#pragma unroll
                for (int o = 1; o < 16; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
                const float sh = amax / 127.0f;
                if (kg == 0) {
#pragma unroll
                    for (int ff = 0; ff < 2; ++ff) {
                        const float q = sh != 0.0f ? round_half_away(h[ff] / sh) : 0.0f;
                        g.hq[row * g.I + 64 * slab + 32 * hb + 16 * ff + r16] = (int8_t)(int)q;
                    }
                    if (r16 == 0) g.hs[row * nbi + 2 * slab + hb] = sh;
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int64_t row = tl.row0 + i;
            const float w = g.prow[row];
            if (kg == 0)
#pragma unroll
                for (int f = 0; f < 8; ++f) g.y[row * g.H + kSlabRows * slab + 16 * f + r16] = w * acc[f][i];
        }
    }
}

// One workgroup per (chunk, group of 4 / S slabs) of the small-chunk list,
// all groups of a chunk on one XCD.  A chunk of r rows takes ceil(r / 2)
// passes (two rows, the last one or two); chunks of more than max_rows rows
// are the small-chunk MFMA kernel's and are skipped here.
template <bool kGateUp, bool kQ81, bool kSym>
__global__ void __launch_bounds__(64 * kWaves, 6) gemv_kernel(GemvArgs g) {
    __shared__ float red[kWaves][kRedFloats];
    const int per = kWaves / g.nsplit;  // slabs per workgroup
    const int ngroups = (g.nslab + per - 1) / per;
    const int id = blockIdx.x;
    const int local = id >> 3;
    const int lo = g.first ? g.first[g.e0] : 0;
    const int hi = g.first ? g.first[g.e1] : *g.nchunks;
    const int chunk = lo + (local / ngroups) * 8 + (id & 7);
    if (chunk >= hi) return;  // uniform over the workgroup, before any barrier
    const Tile tl = g.chunks[chunk];
    if (tl.nrows > g.max_rows || tl.nrows < 1) return;  // uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slab = per * (local % ngroups) + wave / g.nsplit;
    const int part = wave % g.nsplit;
    const bool live = slab < g.nslab;
    const int lane = threadIdx.x & 63;
    for (int r0 = 0; r0 < tl.nrows; r0 += kGemvRows) {  // every wave runs every pass (barriers inside)
        Tile t = tl;
        t.row0 = tl.row0 + r0;
        t.nrows = tl.nrows - r0 < kGemvRows ? tl.nrows - r0 : kGemvRows;
        if (t.nrows == 1)
            gemv_wave<kGateUp, kQ81, kSym, 1, 2>(g, t, slab, part, lane, live, red);
        else
            gemv_wave<kGateUp, kQ81, kSym, 2, 2>(g, t, slab, part, lane, live, red);
    }
}

// S for a reduction of nblk blocks (nblk even): runs of at least 16 blocks
// in whole turns of the ring.
int gemv_split(int nblk) {
    for (int S = 4; S > 1; S /= 2)
        if (nblk / S >= 16 && nblk % (2 * S) == 0) return S;
    return 1;
}

}  // namespace

hipError_t launch_gemv(const GemvLaunch& l, const ChunkLists& cl, int64_t n, int32_t E, const ExpertRange& rng,
                       hipStream_t st) {
    const int32_t ne = rng.first ? rng.e1 - rng.e0 : E;
    const int64_t cap = cl.cap < ne ? cl.cap : ne;  // at most one small chunk per expert
    if (cap <= 0 || n <= 0 || l.max_rows < 1) return hipGetLastError();
    GemvArgs g{};
    g.blobs = l.blobs;
    g.stride = l.stride;
    g.ring0 = rng.ring0;
    g.nring = rng.nring;
    g.chunks = cl.tiles + cl.cap;
    g.nchunks = cl.sched + 1;
    g.first = rng.first ? rng.first + ((int64_t)rng.E + 1) : nullptr;  // the small list's row of the table
    g.e0 = rng.e0;
    g.e1 = rng.e1;
    g.nslab = l.gate_up ? 2 * l.I / kSlabRows : l.H / kSlabRows;
    g.Kd = l.gate_up ? l.H : l.I;
    g.nsplit = gemv_split(g.Kd / kBlock);
    g.max_rows = l.max_rows;
    g.src = l.src;
    g.act = l.act;
    g.act_rows = l.act_rows;
    g.ascale = l.ascale;
    g.asum = l.asum;
    g.prow = l.prow;
    g.I = l.I;
    g.H = l.H;
    g.hq = l.hq;
    g.hs = l.hs;
    g.y = l.y;
    const int per = kWaves / g.nsplit;
    const int ngroups = (g.nslab + per - 1) / per;
    const dim3 grid((unsigned)(8 * ((cap + 7) / 8) * ngroups));
    void (*kernel)(GemvArgs);
    if (l.gate_up && l.asum)
        kernel = l.sym ? gemv_kernel<true, true, true> : gemv_kernel<true, true, false>;
    else if (l.gate_up)
        kernel = l.sym ? gemv_kernel<true, false, true> : gemv_kernel<true, false, false>;
    else
        kernel = l.sym ? gemv_kernel<false, false, true> : gemv_kernel<false, false, false>;
    hipLaunchKernelGGL(kernel, grid, dim3(64 * kWaves), 0, st, g);
    return hipGetLastError();
}

}  // namespace strata_moe
