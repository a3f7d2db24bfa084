// Per-32 int8 rounding of fp32 rows (the layer input, once per token), the
// fp16 code operands of the expert GEMMs built from int8 codes, and a fill
// helper.
//
// Strata compare v0.1.35...v0.1.37 page, include/strata/prefill/moe_fused.hpp,
// header comment and quantize_act: on the fused path each token's input is
// quantized a single time (not once per routed slot as on the MMQ path), to
// int8 codes with one scale for every 32 consecutive values.  The pages do not
// give the rounding; the kernels take s = max|v| / 127 and
// q = round-half-away-from-zero(v / s), both divisions correctly rounded fp32
// (IEEE), |q| <= 127, s = 0 and q = 0 for an all-zero block.
//
// Quantize layout: 8 lanes cover one block of 32 values, one float4 each, so a
// wave reads 1 KiB of contiguous input per instruction.  Outputs per block:
// the int8 codes and the scale.
//
// Operands of the expert GEMMs: the int8 codes q themselves as fp16
// (exact), either as rows [rows][cols] (the layer input, read in place by the
// small-chunk gate/up kernel) or in the tiled layout of the grouped rows (the
// gate/up input of big chunks, gathered through src, and the down input); the
// GEMMs apply the block scales in fp32 after each block's products.  The
// layer input also gets a row multiplier 2^e_r (127 * the row's largest block
// scale in [2^14, 2^15) after scaling by 2^-e_r), which the router takes for
// its fp16 operand.
//
// The kernels also write the operand of the GEMMs' offset pass: per block,
// u = -uoff * s * (sum of the block's codes) (the 2-bit weight offset's share
// beyond the GEMM's q - 1: uoff = 0.5 for w = d (q - 1.5), 0 for the pages'
// Q2_0 map w = d (q - 1); see k_experts.hip), the row's u scaled by a power of two into (-1, 1) and
// split hi/lo, in a hi 8 / lo 8 layout over the block index (padded with
// zeros to a multiple of 32 blocks), plus that power of two.
#include "internal.h"

namespace strata_moe {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float round_half_away(float t) {
    const float r = floorf(fabsf(t) + 0.5f);  // exact: |t| <= 127.00002
    return copysignf(fminf(r, 127.0f), t);
}

__global__ void __launch_bounds__(256) quantize_kernel(const float4* __restrict__ v, int64_t n4,
                                                       int8_t* __restrict__ q8, float* __restrict__ s_out,
                                                       ZeroWords z) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < 2 && z.p[g]) *z.p[g] = 0;  // the call's flag words (saves a launch)
    const bool valid = g < n4;
    const float4 x = valid ? v[g] : make_float4(0.f, 0.f, 0.f, 0.f);
    float a = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    const float s = a / 127.0f;
    float q[4] = {0.f, 0.f, 0.f, 0.f};
    if (s != 0.0f) {
        q[0] = round_half_away(x.x / s);
        q[1] = round_half_away(x.y / s);
        q[2] = round_half_away(x.z / s);
        q[3] = round_half_away(x.w / s);
    }
    if (!valid) return;
    const uint32_t packed = ((uint32_t)(uint8_t)(int8_t)(int)q[0]) | ((uint32_t)(uint8_t)(int8_t)(int)q[1] << 8) |
                            ((uint32_t)(uint8_t)(int8_t)(int)q[2] << 16) | ((uint32_t)(uint8_t)(int8_t)(int)q[3] << 24);
    reinterpret_cast<uint32_t*>(q8)[g] = packed;
    if ((g & 7) == 0) s_out[g >> 3] = s;
}

// The per-slot q8_1 form: row r takes token src[r]'s input and rounds it as
// quantize_kernel does (8 lanes per 32-value block, one float4 each, the same
// arithmetic), so the codes and scales equal that token's; it also writes
// each block's code sum.  One thread per float4 of the n x cols output.
__global__ void __launch_bounds__(256) quantize_slots_kernel(const float* __restrict__ x,
                                                             const int32_t* __restrict__ src, int64_t n,
                                                             int32_t cols, int8_t* __restrict__ q8,
                                                             float* __restrict__ s_out, int32_t* __restrict__ sum_out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t n4 = n * (cols / 4);
    const bool valid = g < n4;
    const int64_t row = valid ? g / (cols / 4) : 0;
    const int64_t c4 = valid ? g - row * (cols / 4) : 0;
    const float4 v = valid ? reinterpret_cast<const float4*>(x + (int64_t)src[row] * cols)[c4]
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 1));
    a = fmaxf(a, __shfl_xor(a, 2));
    a = fmaxf(a, __shfl_xor(a, 4));
    const float s = a / 127.0f;
    float q[4] = {0.f, 0.f, 0.f, 0.f};
    if (s != 0.0f) {
        q[0] = round_half_away(v.x / s);
        q[1] = round_half_away(v.y / s);
        q[2] = round_half_away(v.z / s);
        q[3] = round_half_away(v.w / s);
    }
    int sum = (int)q[0] + (int)q[1] + (int)q[2] + (int)q[3];
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    if (!valid) return;
    const uint32_t packed = ((uint32_t)(uint8_t)(int8_t)(int)q[0]) | ((uint32_t)(uint8_t)(int8_t)(int)q[1] << 8) |
                            ((uint32_t)(uint8_t)(int8_t)(int)q[2] << 16) | ((uint32_t)(uint8_t)(int8_t)(int)q[3] << 24);
    reinterpret_cast<uint32_t*>(q8)[g] = packed;
    if ((g & 7) == 0) {
        s_out[g >> 3] = s;
        sum_out[g >> 3] = sum;
    }
}

// fp16 hi/lo split of an fp32 value.  The asm barrier keeps v an fp32-rounded
// value: otherwise the compiler fuses a producing multiply into the fp16
// conversion (one rounding), and hi can differ by one ulp from the hi that lo
// is measured against when the fp32 value sits on an fp16 rounding tie.
__device__ __forceinline__ void split_hi_lo(float v, _Float16& hi, _Float16& lo) {
    asm volatile("" : "+v"(v));
    hi = (_Float16)v;
    lo = (_Float16)(v - (float)hi);
}

// One wave per row: the row multiplier from the block scales, then 16 codes
// per lane per step (16 contiguous bytes in, 32 contiguous bytes of fp16
// codes out); the block sums go through LDS to the lanes that write the
// offset operand.
__global__ void __launch_bounds__(256) prescale_kernel(const int8_t* __restrict__ q, const float* __restrict__ s,
                                                       int64_t rows, int32_t cols, float uoff,
                                                       _Float16* __restrict__ out, float* __restrict__ mult,
                                                       _Float16* __restrict__ uop, float* __restrict__ umult) {
    __shared__ float ush[4][kMaxOffsetChunks * 32];
    const int w = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * 4 + w;
    if (row >= rows) return;  // wave-uniform; only wave-level synchronisation below
    const int lane = threadIdx.x & 63;
    const int nb = cols / kBlock;
    const int nch = (nb + 31) / 32;
    const float* srow = s + row * nb;
    // the row multiplier 2^e, written when mult is given (the router takes the
    // input rows' multipliers from here)
    float m = 0.0f;
    for (int b = lane; b < nb; b += 64) m = fmaxf(m, srow[b]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float bound = 127.0f * m;  // >= every |q * s| of the row
    float back = 1.0f;
    if (bound > 0.0f) {
        int ex = 0;
        frexpf(bound, &ex);        // bound in [2^(ex-1), 2^ex)
        ex = ex < -96 ? -96 : ex;  // keeps 2^(ex-15) a normal float
        back = ldexpf(1.0f, ex - 15);
    }
    if (mult && lane == 0) mult[row] = back;
    const int8_t* qrow = q + row * cols;
    float umax = 0.0f;
    for (int j0 = 0; j0 < cols / 16; j0 += 64) {  // uniform trip count: the shuffle below sees whole waves
        const int j = j0 + lane;
        const bool on = j < cols / 16;
        uint4 wv = make_uint4(0, 0, 0, 0);
        if (on) wv = *reinterpret_cast<const uint4*>(qrow + 16 * j);
        const float sraw = on ? srow[j >> 1] : 0.0f;
        const uint32_t ws[4] = {wv.x, wv.y, wv.z, wv.w};
        half8_t cq[2];
        int sum = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c = (int8_t)(ws[i >> 2] >> (8 * (i & 3)));
            sum += c;
            cq[i >> 3][i & 7] = (_Float16)c;  // exact: |c| <= 127
        }
        sum += __shfl_xor(sum, 1);  // lanes 2m, 2m+1 hold the two halves of one block
        if (on && (j & 1) == 0) {
            const float u = -uoff * sraw * (float)sum;
            ush[w][j >> 1] = u;
            umax = fmaxf(umax, fabsf(u));
        }
        if (!on) continue;
        if (out) {
            half8_t* dst = reinterpret_cast<half8_t*>(out + row * cols + 16 * j);
            dst[0] = cq[0];
            dst[1] = cq[1];
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) umax = fmaxf(umax, __shfl_xor(umax, o));
    if (!uop) return;  // no offset operand (the Q2_0 map)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // offset operand: lane g < 4*nch writes value group g (blocks 8g..8g+7)
    int eu = 0;
    if (umax > 0.0f) frexpf(umax, &eu);  // |u| * 2^-eu < 1
    eu = eu < -100 ? -100 : eu;           // keeps 2^-eu finite
    const float dn = ldexpf(1.0f, -eu);
    if (lane == 0) umult[row] = ldexpf(1.0f, eu);
    if (lane < 4 * nch) {
        half8_t hi, lo;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int b = 8 * lane + t;
            const float un = b < nb ? ush[w][b] * dn : 0.0f;  // exact: a power-of-two scaling
            _Float16 h, l;
            split_hi_lo(un, h, l);
            hi[t] = h;
            lo[t] = l;
        }
        half8_t* dst = reinterpret_cast<half8_t*>(uop + row * (int64_t)nch * 64 + 16 * lane);
        dst[0] = hi;
        dst[1] = lo;
    }
}

// The down GEMM's operand of grouped rows in the tiled layout: the int8 H
// codes as fp16 (exact) in [tile][block][group g][row within the tile][8],
// their block scales in [tile][block / 4][row within the tile][4] (blocks
// padded with zeros to a multiple of 4), plus the offset operand as
// prescale_kernel builds it.  One workgroup per 16-row tile of the tile
// table.  The tile's rows are consecutive grouped rows: their codes and
// scales are read coalesced into LDS, kStageCols columns at a time (rows
// padded by 8 bytes / 1 float against bank conflicts), then lane 16 g + r of
// a wave takes tile row r, value group g (8 codes) of a block, so each
// block's fragment is one contiguous 1 KiB store; wave w takes blocks w,
// w + 4, ...  Wider rows than kStageCols are staged twice (once per pass).
constexpr int kStageCols = 2048;
inline size_t tile_h_lds_bytes(int32_t cols) {
    const int sc = cols < kStageCols ? cols : kStageCols;
    return (size_t)16 * (sc + 8) + (size_t)16 * (sc / kBlock + 1) * sizeof(float);
}

__global__ void __launch_bounds__(256) tile_h_kernel(const int8_t* __restrict__ q, const float* __restrict__ s,
                                                     const TileRows* __restrict__ trows,
                                                     const int32_t* __restrict__ ntiles, int32_t cols, float uoff,
                                                     _Float16* __restrict__ out, float* __restrict__ sout,
                                                     _Float16* __restrict__ uop, float* __restrict__ umult,
                                                     const int32_t* __restrict__ first_tile, int32_t e0, int32_t e1) {
    extern __shared__ __align__(16) unsigned char lds[];  // codes [16][sc + 8], scales [16][sc / 32 + 1]
    __shared__ float ush[16][kMaxOffsetChunks * 32];      // u of each row and block
    __shared__ float umx[4][16];                          // per wave: max |u| of each row
    // all tiles, or (first_tile) those of experts [e0, e1)
    const int64_t t = (first_tile ? first_tile[e0] : 0) + (int64_t)blockIdx.x;
    if (t >= (first_tile ? first_tile[e1] : *ntiles)) return;  // uniform over the workgroup, before any barrier
    const TileRows tr = trows[t];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int nb = cols / kBlock, nch = (nb + 31) / 32, nq = (nb + 3) / 4;
    const int sc = cols < kStageCols ? cols : kStageCols, sb = sc / kBlock;
    const int qstride = sc + 8, sstride = sb + 1;
    float* sl = reinterpret_cast<float*>(lds + (size_t)16 * qstride);
    // block scales, tiled: thread i takes row i / nq, 4-block group i % nq
    for (int i = tid; i < 16 * nq; i += 256) {
        const int rr = i / nq, qb = i - rr * nq;
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int b = 4 * qb + j;
            v[j] = rr < tr.nrows && b < nb ? s[((int64_t)tr.row0 + rr) * nb + b] : 0.0f;
        }
        *reinterpret_cast<float4*>(sout + ((t * nq + qb) * 16 + rr) * 4) = make_float4(v[0], v[1], v[2], v[3]);
    }
    // columns [c0, c0 + sc) of the tile's rows into LDS; rows past nrows as zeros
    auto stage = [&](int c0) {  // all of a thread's loads first, then its LDS stores
        const int pieces = sc / 16;
        constexpr int kPer = 16 * (kStageCols / 16) / 256;
        uint4 v[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = tid + 256 * k, rr = i / pieces, c = i - rr * pieces;
            v[k] = make_uint4(0, 0, 0, 0);
            if (i < 16 * pieces && rr < tr.nrows && c0 + 16 * c < cols)
                v[k] = *reinterpret_cast<const uint4*>(q + ((int64_t)tr.row0 + rr) * cols + c0 + 16 * c);
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = tid + 256 * k, rr = i / pieces, c = i - rr * pieces;
            if (i < 16 * pieces) {
                *reinterpret_cast<uint2*>(lds + rr * qstride + 16 * c) = make_uint2(v[k].x, v[k].y);
                *reinterpret_cast<uint2*>(lds + rr * qstride + 16 * c + 8) = make_uint2(v[k].z, v[k].w);
            }
        }
        for (int i = tid; i < 16 * sb; i += 256) {
            const int rr = i / sb, b = i - rr * sb, bg = c0 / kBlock + b;
            sl[rr * sstride + b] = rr < tr.nrows && bg < nb ? s[((int64_t)tr.row0 + rr) * nb + bg] : 0.0f;
        }
    };
    const bool valid = r < tr.nrows;
    const int64_t row = (int64_t)tr.row0 + r;
    half8_t* tile = reinterpret_cast<half8_t*>(out) + t * nb * 64;
    // one pass per slice: the fp16 codes, and the block sums -> u, max |u|
    float umax = 0.0f;
    for (int c0 = 0; c0 < cols; c0 += sc) {
        if (c0 > 0) __syncthreads();  // the previous slice is read
        stage(c0);
        __syncthreads();
        const int b1 = (cols - c0) / kBlock < sb ? (cols - c0) / kBlock : sb;
        for (int b = w; b < b1; b += 4) {  // uniform trip count: the shuffles see whole waves
            const uint2 c8 = *reinterpret_cast<const uint2*>(lds + r * qstride + kBlock * b + 8 * g);
            const float sraw = sl[r * sstride + b];
            int sum = 0;
            half8_t h;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int c = (int8_t)((i < 4 ? c8.x : c8.y) >> (8 * (i & 3)));
                sum += c;
                h[i] = (_Float16)c;  // exact; rows past nrows: zero codes
            }
            tile[(c0 / kBlock + b) * 64 + lane] = h;
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            const float u = -uoff * sraw * (float)sum;
            if (g == 0) ush[r][c0 / kBlock + b] = u;
            umax = fmaxf(umax, fabsf(u));
        }
    }
    if (!uop) return;  // no offset operand (the Q2_0 map)
    if (g == 0) umx[w][r] = umax;
    __syncthreads();
    umax = fmaxf(fmaxf(umx[0][r], umx[1][r]), fmaxf(umx[2][r], umx[3][r]));
    int eu = 0;
    if (umax > 0.0f) frexpf(umax, &eu);
    eu = eu < -100 ? -100 : eu;
    const float dn = ldexpf(1.0f, -eu);
    if (valid && w == 0 && g == 0) umult[row] = ldexpf(1.0f, eu);
    // offset operand: value group G (blocks 8G .. 8G + 7) of row r, hi then lo
    if (valid)
        for (int G = 4 * w + g; G < 4 * nch; G += 16) {
            half8_t hi, lo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int b = 8 * G + i;
                const float un = b < nb ? ush[r][b] * dn : 0.0f;  // exact: a power-of-two scaling
                _Float16 h, l;
                split_hi_lo(un, h, l);
                hi[i] = h;
                lo[i] = l;
            }
            half8_t* dst = reinterpret_cast<half8_t*>(uop + row * (int64_t)nch * 64 + 16 * G);
            dst[0] = hi;
            dst[1] = lo;
        }
}

// launch_offset_rows: L lanes per row (L = 4 nch rounded up to a power of
// two), lane G of a row takes value group G (blocks 8G .. 8G + 7): its 8
// floats in, the row's largest |u| (a shuffle over the L lanes), its
// multiplier, then the group's hi and lo halves written over the same 32
// bytes it read.
__global__ void __launch_bounds__(256) offset_rows_kernel(float* __restrict__ hu, int64_t n, int32_t nb,
                                                          float* __restrict__ umult) {
    const int nch = (nb + 31) / 32, L = nch == 1 ? 4 : nch == 2 ? 8 : 16;
    const int lane = threadIdx.x & 63, G = lane & (L - 1);
    const int64_t row = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / L) + lane / L;
    const bool mine = row < n && G < 4 * nch;
    float* ug = hu + row * (int64_t)nch * 32 + 8 * G;
    float u[8];
    if (mine) {
        const float4 u0 = reinterpret_cast<const float4*>(ug)[0], u1 = reinterpret_cast<const float4*>(ug)[1];
        u[0] = u0.x; u[1] = u0.y; u[2] = u0.z; u[3] = u0.w;
        u[4] = u1.x; u[5] = u1.y; u[6] = u1.z; u[7] = u1.w;
    }
    float umax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (!mine || 8 * G + i >= nb) u[i] = 0.0f;  // padding blocks: zero operand
        umax = fmaxf(umax, fabsf(u[i]));
    }
    for (int off = 1; off < L; off <<= 1) umax = fmaxf(umax, __shfl_xor(umax, off));
    if (!mine) return;
    int eu = 0;
    if (umax > 0.0f) frexpf(umax, &eu);
    eu = eu < -100 ? -100 : eu;
    const float dn = ldexpf(1.0f, -eu);
    if (G == 0) umult[row] = ldexpf(1.0f, eu);
    half8_t hi, lo;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        _Float16 h, l;
        split_hi_lo(u[i] * dn, h, l);  // exact: a power-of-two scaling
        hi[i] = h;
        lo[i] = l;
    }
    half8_t* dst = reinterpret_cast<half8_t*>(ug);
    dst[0] = hi;
    dst[1] = lo;
}

// The 4-wave gate/up kernel's operand in the tiled layout: tile t of the
// tile table (if its chunk is big) holds grouped rows trows[t], each the
// token src[row]; its int8 codes become fp16 (exact) in [tile][block][group
// g][row within the tile][8] and its block scales [tile][block / 4][row
// within the tile][4] (one 16-byte load per lane and 4 blocks).  One
// workgroup per tile and slice of kGatherCols columns (grid y): the 16 token
// rows' codes of the slice are staged in LDS with coalesced loads (rows
// padded by 8 bytes), then lane 16 g + r of a wave writes row r, group g of
// a block, so each block's fragment is one contiguous 1 KiB store; wave w
// takes blocks w, w + 4, ...  Rows past a tile's nrows are zeros.
constexpr int kGatherCols = 1280;  // columns per slice (40 blocks, 10 scale groups; 640 measured 4 us slower at T = 8192)
constexpr int kGatherPer = (16 * (kGatherCols / 16) + 255) / 256;  // 16-byte pieces per thread
inline size_t gather_tiles_lds_bytes(int32_t cols) {
    const int sc = cols < kGatherCols ? cols : kGatherCols;
    return (size_t)16 * (sc + 8);
}

__global__ void __launch_bounds__(256) gather_tiles_kernel(const int8_t* __restrict__ q, const float* __restrict__ s,
                                                           const int32_t* __restrict__ src,
                                                           const TileRows* __restrict__ trows,
                                                           const int32_t* __restrict__ ntiles, int32_t cols,
                                                           _Float16* __restrict__ out, float* __restrict__ sout) {
    extern __shared__ __align__(16) unsigned char lds[];  // codes [16][sc + 8]
    const int64_t t = blockIdx.x;
    if (t >= *ntiles) return;  // uniform over the workgroup, before any barrier
    const TileRows tr = trows[t];
    if (!tr.big) return;  // the small-chunk kernel reads its rows in place
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, r = lane & 15, g = lane >> 4;
    const int nb = cols / kBlock;
    const int sc = cols < kGatherCols ? cols : kGatherCols, qstride = sc + 8;
    const int c0 = blockIdx.y * sc;                                     // the slice's first column
    const int b0 = c0 / kBlock, b1 = (cols - c0 < sc ? cols - c0 : sc) / kBlock;  // its blocks [b0, b0 + b1)
    // block scales of the slice's 4-block groups: thread i takes row i / ng, group i % ng
    const int nq = nb / 4, ng = (b1 + 3) / 4;
    for (int i = tid; i < 16 * ng; i += 256) {
        const int rr = i / ng, qb = b0 / 4 + i - rr * ng;
        if (qb >= nq) continue;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (rr < tr.nrows) v = *reinterpret_cast<const float4*>(s + (int64_t)src[tr.row0 + rr] * nb + 4 * qb);
        *reinterpret_cast<float4*>(sout + ((t * nq + qb) * 16 + rr) * 4) = v;
    }
    // all of a thread's loads first, then its LDS stores
    const int pieces = sc / 16;
    uint4 v[kGatherPer];
#pragma unroll
    for (int k = 0; k < kGatherPer; ++k) {
        const int i = tid + 256 * k, rr = i / pieces, c = i - rr * pieces;
        v[k] = make_uint4(0, 0, 0, 0);
        if (i < 16 * pieces && rr < tr.nrows && c0 + 16 * c < cols)
            v[k] = *reinterpret_cast<const uint4*>(q + (int64_t)src[tr.row0 + rr] * cols + c0 + 16 * c);
    }
#pragma unroll
    for (int k = 0; k < kGatherPer; ++k) {
        const int i = tid + 256 * k, rr = i / pieces, c = i - rr * pieces;
        if (i < 16 * pieces) {
            *reinterpret_cast<uint2*>(lds + rr * qstride + 16 * c) = make_uint2(v[k].x, v[k].y);
            *reinterpret_cast<uint2*>(lds + rr * qstride + 16 * c + 8) = make_uint2(v[k].z, v[k].w);
        }
    }
    __syncthreads();
    half8_t* tile = reinterpret_cast<half8_t*>(out) + t * nb * 64;
    for (int b = w; b < b1; b += 4) {
        const uint2 c8 = *reinterpret_cast<const uint2*>(lds + r * qstride + kBlock * b + 8 * g);
        half8_t h;
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (_Float16)(int8_t)((i < 4 ? c8.x : c8.y) >> (8 * (i & 3)));  // exact
        tile[(b0 + b) * 64 + lane] = h;
    }
}

// The layer input in one pass: quantize_kernel's int8 codes and scales and
// prescale_kernel's outputs (fp16 codes, row multiplier, offset operand)
// from the fp32 rows, one wave per row.  Lane pairs own a 32-value block, 16
// values each (four float4 loads: the wave reads 4 KiB of the row per step);
// the arithmetic of each output is that of the two separate kernels.
// 8 waves per SIMD (60 VGPRs, no spills): 8192 rows fit one round; 36-37 vs
// 39 us at 8192 rows, 126 vs 124 at 32768.
__global__ void __launch_bounds__(256, 8) quantize_prescale_kernel(const float* __restrict__ x, int64_t rows,
                                                                   int32_t cols, float uoff, int8_t* __restrict__ q8,
                                                                   float* __restrict__ s_out, _Float16* __restrict__ out,
                                                                   float* __restrict__ mult, float* __restrict__ xn,
                                                                   _Float16* __restrict__ uop, float* __restrict__ umult,
                                                                   ZeroWords z) {
    __shared__ float ush[4][kMaxOffsetChunks * 32];
    if (blockIdx.x == 0 && threadIdx.x < 2 && z.p[threadIdx.x]) *z.p[threadIdx.x] = 0;  // the call's flag words
    const int w = threadIdx.x >> 6;
    const int64_t row = (int64_t)blockIdx.x * 4 + w;
    if (row >= rows) return;  // wave-uniform; only wave-level synchronisation below
    const int lane = threadIdx.x & 63;
    const int nb = cols / kBlock;
    const int nch = (nb + 31) / 32;
    const float* xrow = x + row * cols;
    float smax = 0.0f, umax = 0.0f, sq = 0.0f;
    for (int j0 = 0; j0 < cols / 16; j0 += 64) {  // uniform trip count: the shuffles see whole waves
        const int j = j0 + lane;                  // 16-value group j: block j / 2, half j % 2
        const bool on = j < cols / 16;
        float v[16];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const float4 x4 = on ? reinterpret_cast<const float4*>(xrow + 16 * j)[f] : make_float4(0.f, 0.f, 0.f, 0.f);
            v[4 * f] = x4.x, v[4 * f + 1] = x4.y, v[4 * f + 2] = x4.z, v[4 * f + 3] = x4.w;
        }
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            a = fmaxf(a, fabsf(v[i]));
            sq = fmaf(v[i], v[i], sq);  // zeros past the row
        }
        a = fmaxf(a, __shfl_xor(a, 1));
        const float s = a / 127.0f;
        int sum = 0;
        uint32_t packed[4] = {0, 0, 0, 0};
        half8_t cq[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float qf = s != 0.0f ? round_half_away(v[i] / s) : 0.0f;
            const int c = (int)qf;
            sum += c;
            packed[i >> 2] |= (uint32_t)(uint8_t)(int8_t)c << (8 * (i & 3));
            cq[i >> 3][i & 7] = (_Float16)c;  // exact: |c| <= 127
        }
        sum += __shfl_xor(sum, 1);
        if (!on) continue;
        smax = fmaxf(smax, s);
        *reinterpret_cast<uint4*>(q8 + row * cols + 16 * j) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        if (out) {
            half8_t* dst = reinterpret_cast<half8_t*>(out + row * cols + 16 * j);
            dst[0] = cq[0];
            dst[1] = cq[1];
        }
        if ((j & 1) == 0) {
            s_out[row * nb + (j >> 1)] = s;
            const float u = -uoff * s * (float)sum;
            ush[w][j >> 1] = u;
            umax = fmaxf(umax, fabsf(u));
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        smax = fmaxf(smax, __shfl_xor(smax, o));
        umax = fmaxf(umax, __shfl_xor(umax, o));
        sq += __shfl_xor(sq, o);
    }
    if (lane == 0 && xn) xn[row] = sqrtf(sq);
    // the row multiplier, as prescale_kernel computes it from the block scales
    const float bound = 127.0f * smax;
    float back = 1.0f;
    if (bound > 0.0f) {
        int ex = 0;
        frexpf(bound, &ex);
        ex = ex < -96 ? -96 : ex;
        back = ldexpf(1.0f, ex - 15);
    }
    if (lane == 0) mult[row] = back;
    if (!uop) return;  // no offset operand (the Q2_0 map)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int eu = 0;
    if (umax > 0.0f) frexpf(umax, &eu);
    eu = eu < -100 ? -100 : eu;
    const float dn = ldexpf(1.0f, -eu);
    if (lane == 0) umult[row] = ldexpf(1.0f, eu);
    if (lane < 4 * nch) {
        half8_t hi, lo;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int b = 8 * lane + t;
            const float un = b < nb ? ush[w][b] * dn : 0.0f;
            _Float16 h, l;
            split_hi_lo(un, h, l);
            hi[t] = h;
            lo[t] = l;
        }
        half8_t* dst = reinterpret_cast<half8_t*>(uop + row * (int64_t)nch * 64 + 16 * lane);
        dst[0] = hi;
        dst[1] = lo;
    }
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t count) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < count) p[g] = 0.0f;
}

inline unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_quantize(const float* v, int64_t rows, int32_t cols, int8_t* q8, float* s, hipStream_t st,
                           ZeroWords z) {
    const int64_t n4 = rows * cols / 4;
    if (n4 > 0)
        hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(n4, 256)), dim3(256), 0, st,
                           reinterpret_cast<const float4*>(v), n4, q8, s, z);
    return hipGetLastError();
}

hipError_t launch_prescale(const int8_t* q, const float* s, int64_t rows, int32_t cols, float uoff, _Float16* out,
                           float* mult, _Float16* uop, float* umult, hipStream_t st) {
    if (rows > 0)
        hipLaunchKernelGGL(prescale_kernel, dim3(grid_for(rows, 4)), dim3(256), 0, st, q, s, rows, cols, uoff, out,
                           mult, uop, umult);
    return hipGetLastError();
}

hipError_t launch_gather_tiles(const int8_t* q, const float* s, const int32_t* src, const ChunkLists& cl,
                               int64_t tiles_cap, int32_t cols, _Float16* out, float* sout, hipStream_t st) {
    if (tiles_cap > 0)
        hipLaunchKernelGGL(gather_tiles_kernel,
                           dim3((unsigned)tiles_cap, (unsigned)((cols + kGatherCols - 1) / kGatherCols)), dim3(256),
                           gather_tiles_lds_bytes(cols), st, q, s, src, cl.trows, cl.sched + 2, cols, out, sout);
    return hipGetLastError();
}

hipError_t launch_tile_h(const int8_t* q, const float* s, const ChunkLists& cl, int64_t tiles_cap, int32_t cols,
                         float uoff, _Float16* out, float* sout, _Float16* uop, float* umult, hipStream_t st,
                         const ExpertRange& rng) {
    const int32_t* first_tile = rng.first ? rng.first + 2 * ((int64_t)rng.E + 1) : nullptr;
    if (tiles_cap > 0)
        hipLaunchKernelGGL(tile_h_kernel, dim3((unsigned)tiles_cap), dim3(256), tile_h_lds_bytes(cols), st, q, s,
                           cl.trows, cl.sched + 2, cols, uoff, out, sout, uop, umult, first_tile, rng.e0, rng.e1);
    return hipGetLastError();
}

hipError_t launch_offset_rows(float* hu, int64_t n, int32_t cols, float* umult, hipStream_t st) {
    if (n > 0)
    {
        const int nch = (cols / kBlock + 31) / 32, L = nch == 1 ? 4 : nch == 2 ? 8 : 16, rows = 4 * (64 / L);
        hipLaunchKernelGGL(offset_rows_kernel, dim3((unsigned)((n + rows - 1) / rows)), dim3(256), 0, st, hu, n,
                           cols / kBlock, umult);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_prescale(const float* x, int64_t rows, int32_t cols, float uoff, int8_t* q8, float* s,
                                   _Float16* codes16, float* mult, float* xn, _Float16* uop, float* umult,
                                   hipStream_t st, ZeroWords z) {
    if (rows > 0)
        hipLaunchKernelGGL(quantize_prescale_kernel, dim3(grid_for(rows, 4)), dim3(256), 0, st, x, rows, cols, uoff,
                           q8, s, codes16, mult, xn, uop, umult, z);
    return hipGetLastError();
}

hipError_t launch_quantize_slots(const float* x, const int32_t* src, int64_t n, int32_t cols, int8_t* q8, float* s,
                                 int32_t* sum, hipStream_t st) {
    const int64_t n4 = n * (cols / 4);
    if (n4 > 0)
        hipLaunchKernelGGL(quantize_slots_kernel, dim3(grid_for(n4, 256)), dim3(256), 0, st, x, src, n, cols, q8, s,
                           sum);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t st) {
    if (count > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(count, 256)), dim3(256), 0, st, p, count);
    return hipGetLastError();
}

}  // namespace strata_moe
