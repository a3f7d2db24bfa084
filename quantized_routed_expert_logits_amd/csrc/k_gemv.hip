// Grouped expert GEMV for chunks of at most kGemvRows routed rows: the
// decode-window end of the prompt path, where most hit experts get one or two
// rows.  There the MFMA kernels' fp16 unpack of the 2-bit codes dominates
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
// z = 1.5 (symmetric map) or 1 (Q2_0).  The codes become int8 c = 2q - 3
// (symmetric) or q - 1 (Q2_0) by a byte lookup (v_perm), so a block's sum
// over an int8 activation block a is an exact int32 P = sum c a; the output
// adds fp32(P) * s * d (times 1/2 for the symmetric map, once at the end).
// The per-slot q8_1 arm (the pages' MMQ form, an A/B alternative) reads
// activations quantized per routed slot with their block code sums A, keeps
// the raw codes q and subtracts z * A instead: P = sum q a - z A (2 sum q a -
// 3 A for the symmetric map).
//
// Work split.  A workgroup takes one chunk and 4 consecutive 128-row slabs,
// one per wave, as the small-chunk MFMA kernel does (same packed records:
// lane l holds the 8 codes k = 8 (l / 16) .. + 7 of rows l % 16 + 16 f,
// f = 0..7, in its 16 record bytes).  Each lane accumulates its k range; the
// four lanes of a row add their sums at the end.
#include "internal.h"

namespace strata_moe {

namespace {

constexpr int kWaves = 4;
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3 for raw dword loads on gfx9 (gfx950)
constexpr uint32_t kLookupSym = 0x0301FFFDu;  // bytes -3, -1, 1, 3: 2q - 3 for q = 0..3
constexpr uint32_t kLookupQ20 = 0x020100FFu;  // bytes -1, 0, 1, 2: q - 1

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
    const int32_t* src;   // gate/up without the per-slot arm: token of each grouped row
    const int8_t* act;    // int8 activation rows [act_rows][Kd]
    int64_t act_rows;
    const float* ascale;  // their block scales [act_rows][Kd / 32]
    const int32_t* asum;  // per-slot arm: their block code sums [act_rows][Kd / 32], else null
    int32_t sym;          // 1: w = d (q - 1.5), 0: w = d (q - 1)
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

// One record dword -> the int8 codes of its two rows: lo[0] / hi[0] = row A
// (fragment 2p) k 0..3 / 4..7, lo[1] / hi[1] = row B.  Bits 2j, 2j+1 of each
// byte hold code k = 2j (bytes 0, 1: rows A, B) or k = 2j + 1 (bytes 2, 3).
template <bool kLookup>
__device__ __forceinline__ void row_codes(uint32_t w, uint32_t lut, uint32_t (&lo)[2], uint32_t (&hi)[2]) {
    uint32_t x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[j] = (w >> (2 * j)) & 0x03030303u;
        if constexpr (kLookup) x[j] = __builtin_amdgcn_perm(lut, lut, x[j]);  // byte q -> its int8 code
    }
    lo[0] = __builtin_amdgcn_perm(x[1], x[0], 0x06040200u);  // A: k0 k1 k2 k3
    hi[0] = __builtin_amdgcn_perm(x[3], x[2], 0x06040200u);  // A: k4 k5 k6 k7
    lo[1] = __builtin_amdgcn_perm(x[1], x[0], 0x07050301u);  // B
    hi[1] = __builtin_amdgcn_perm(x[3], x[2], 0x07050301u);
}

// One wave: chunk tl (R rows) against slab `slab`.
template <bool kGateUp, bool kQ81, int R>
__device__ __forceinline__ void gemv_wave(const GemvArgs& g, const Tile& tl, int slab, int lane) {
    const int r16 = lane & 15, kg = lane >> 4;
    const int nblk = g.Kd / kBlock;
    int64_t arow[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int row = tl.row0 + i;
        arow[i] = (kGateUp && !kQ81) ? (int64_t)g.src[row] : (int64_t)row;
    }
    const uint8_t* rec = gemv_blob(g, tl.e) + (int64_t)slab * nblk * kRecordBytes;
    const __amdgpu_buffer_rsrc_t rrec = __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, nblk * kRecordBytes,
                                                                          kBufferWord3);
    const __amdgpu_buffer_rsrc_t ract = __builtin_amdgcn_make_buffer_rsrc(
        (void*)g.act, (short)0, (int)(g.act_rows * g.Kd), kBufferWord3);
    const uint32_t lut = g.sym ? kLookupSym : kLookupQ20;
    float acc[8][R];
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int i = 0; i < R; ++i) acc[f][i] = 0.f;

    // loads of block b: the lane's 16 code bytes and its row's 16 scale
    // bytes, and per activation row its 8 codes of the lane's k range
    auto load = [&](int b, uint32_t (&c)[4], uint32_t (&sw)[4], uint32_t (&a)[R][2]) {
        b = b < nblk ? b : nblk - 1;
        const auto cv = __builtin_amdgcn_raw_buffer_load_b128(rrec, lane * 16, b * kRecordBytes, 0);
        const auto dv = __builtin_amdgcn_raw_buffer_load_b128(rrec, kRecordCodeBytes + r16 * 16, b * kRecordBytes, 0);
#pragma unroll
        for (int p = 0; p < 4; ++p) c[p] = cv[p], sw[p] = dv[p];
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const auto av = __builtin_amdgcn_raw_buffer_load_b64(ract, (int)(arow[i] * g.Kd) + 8 * kg, b * kBlock, 0);
            a[i][0] = av[0];
            a[i][1] = av[1];
        }
    };
    uint32_t c[2][4], sw[2][4], a[2][R][2];
    load(0, c[0], sw[0], a[0]);
    for (int b = 0; b < nblk; b += 2) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int blk = b + u;
            if (blk >= nblk) break;  // uniform
            load(blk + 1, c[u ^ 1], sw[u ^ 1], a[u ^ 1]);
            float s[R];
            int32_t zs[R];  // per-slot arm: the offset term z * A (2z for the symmetric map), on lanes kg == 0
#pragma unroll
            for (int i = 0; i < R; ++i) {
                s[i] = g.ascale[arow[i] * nblk + blk];
                zs[i] = 0;
                if constexpr (kQ81) {
                    const int32_t A = g.asum[arow[i] * nblk + blk];
                    zs[i] = kg == 0 ? (g.sym ? 3 * A : A) : 0;
                }
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint32_t lo[2], hi[2];
                row_codes<!kQ81>(c[u][p], lut, lo, hi);
                const float d0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(sw[u][p] & 0xffffu));
                const float d1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(sw[u][p] >> 16));
#pragma unroll
                for (int i = 0; i < R; ++i) {
                    int32_t pa = __builtin_amdgcn_sdot4((int)lo[0], (int)a[u][i][0], 0, false);
                    pa = __builtin_amdgcn_sdot4((int)hi[0], (int)a[u][i][1], pa, false);
                    int32_t pb = __builtin_amdgcn_sdot4((int)lo[1], (int)a[u][i][0], 0, false);
                    pb = __builtin_amdgcn_sdot4((int)hi[1], (int)a[u][i][1], pb, false);
                    if constexpr (kQ81) {
                        if (g.sym) pa = 2 * pa, pb = 2 * pb;
                        pa -= zs[i];
                        pb -= zs[i];
                    }
                    acc[2 * p][i] = fmaf((float)pa * s[i], d0, acc[2 * p][i]);
                    acc[2 * p + 1][i] = fmaf((float)pb * s[i], d1, acc[2 * p + 1][i]);
                }
            }
        }
    }
    // the four lanes of a row (k ranges kg = 0..3) add their sums
    const float half = g.sym ? 0.5f : 1.0f;  // the symmetric map's codes are 2 (q - 1.5)
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float v = acc[f][i];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            acc[f][i] = v * half;
        }

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

// One workgroup per (chunk, group of 4 slabs) of the small-chunk list, all
// groups of a chunk on one XCD; chunks of more than kGemvRows rows are the
// small-chunk MFMA kernel's and are skipped here.
template <bool kGateUp, bool kQ81>
__global__ void __launch_bounds__(64 * kWaves) gemv_kernel(GemvArgs g) {
    const int ngroups = (g.nslab + kWaves - 1) / kWaves;
    const int id = blockIdx.x;
    const int local = id >> 3;
    const int lo = g.first ? g.first[g.e0] : 0;
    const int hi = g.first ? g.first[g.e1] : *g.nchunks;
    const int chunk = lo + (local / ngroups) * 8 + (id & 7);
    if (chunk >= hi) return;
    const Tile tl = g.chunks[chunk];
    if (tl.nrows > kGemvRows || tl.nrows < 1) return;  // uniform over the workgroup
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slab = kWaves * (local % ngroups) + wave;
    if (slab >= g.nslab) return;  // waves are independent: no barrier follows
    const int lane = threadIdx.x & 63;
    if (tl.nrows == 1)
        gemv_wave<kGateUp, kQ81, 1>(g, tl, slab, lane);
    else
        gemv_wave<kGateUp, kQ81, 2>(g, tl, slab, lane);
}

}  // namespace

hipError_t launch_gemv(const GemvLaunch& l, const ChunkLists& cl, int64_t n, int32_t E, const ExpertRange& rng,
                       hipStream_t st) {
    const int32_t ne = rng.first ? rng.e1 - rng.e0 : E;
    const int64_t cap = cl.cap < ne ? cl.cap : ne;  // at most one small chunk per expert
    if (cap <= 0 || n <= 0) return hipGetLastError();
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
    g.src = l.src;
    g.act = l.act;
    g.act_rows = l.act_rows;
    g.ascale = l.ascale;
    g.asum = l.asum;
    g.sym = l.sym;
    g.prow = l.prow;
    g.I = l.I;
    g.H = l.H;
    g.hq = l.hq;
    g.hs = l.hs;
    g.y = l.y;
    const int ngroups = (g.nslab + kWaves - 1) / kWaves;
    const dim3 grid((unsigned)(8 * ((cap + 7) / 8) * ngroups));
    if (l.gate_up) {
        if (l.asum)
            hipLaunchKernelGGL((gemv_kernel<true, true>), grid, dim3(64 * kWaves), 0, st, g);
        else
            hipLaunchKernelGGL((gemv_kernel<true, false>), grid, dim3(64 * kWaves), 0, st, g);
    } else {
        hipLaunchKernelGGL((gemv_kernel<false, false>), grid, dim3(64 * kWaves), 0, st, g);
    }
    return hipGetLastError();
}

}  // namespace strata_moe
