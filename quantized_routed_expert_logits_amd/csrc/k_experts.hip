// Grouped expert GEMMs: gate/up with SwiGLU and the int8 rounding of H fused
// in the epilogue, and down with the weighted scatter-add combine fused in its
// epilogue.
//
// Strata compare v0.1.35...v0.1.37 page, include/strata/prefill/moe_fused.hpp,
// experts: per expert, gate/up on the int8 activations of its grouped rows
// (through src), SwiGLU, H rounded to int8 per 32 values in the epilogue, then
// down into the rows the combine reads; each expert is read where it is (no
// gather), in 64-row tiles; the 2-bit codes are unpacked in registers.
//
// Arithmetic.  One weight block is 32 codes q of one row with one fp16 scale
// d, w = d * (q - 1.5); one activation block is 32 int8 codes a with an fp32
// scale s.  Their contribution to an output is
//     s * d * sum(q - 1.5) * a = s * [d * sum (q - 1) * a] + d * u,
//     u = -0.5 * s * sum(a)  (computed once per activation block).
// The bracket is one v_mfma_f32_16x16x32_f16 (K = 32 = one block): the A
// operand d*(q-1) is exact in fp16 (q - 1 in {-1, 0, 1, 2}), the B operand
// holds the integer codes (exact in fp16), products are exact and every
// partial sum is a multiple of d's last place below 2^24 of them, so the fp32
// result is exact.  The per-block scale s then needs one fp32 FMA per output
// (s differs per token and per block, so it cannot enter the MFMA exactly);
// the offset term d*u a second one.
//
// Operand roles: A = weights (rows = weight rows, 16 per fragment), B =
// activations (columns = routed rows).  Lane l of the 16x16 output holds
// column l % 16 (one routed row) and rows 4*(l/16) + v, v = 0..3, so the
// activation scale s and u are one value per lane per block.
//
// Work split: a workgroup (4 waves) takes one 64-row tile of one expert
// (its rows in the grouped order) and 4 consecutive weight slices of 64 rows;
// each wave one slice: 4 fragments x 4 token tiles = 16 MFMAs per block.
#include "internal.h"

namespace strata_moe {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;

__device__ __forceinline__ _Float16 lo_half(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ _Float16 hi_half(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// One packed dword (16 codes) -> two A fragments of 8 fp16 values d*(q-1).
// Pair m (0..7) of the dword fills fragment m/4, elements 2(m%4) and
// 2(m%4)+1; its codes sit at bits [2m, 2m+1] and [16+2m, 17+2m].  OR-ing the
// code into the mantissa of 1024.0 (0x6400) gives 1024 + q exactly; minus
// 1025 gives q - 1; times d is exact.
__device__ __forceinline__ void unpack_pair(uint32_t x, _Float16 d0, _Float16 d1, half8_t& a0, half8_t& a1) {
#pragma clang fp contract(off)
    const half2_t bias = {(_Float16)1025.0f, (_Float16)1025.0f};
    const half2_t s0 = {d0, d0}, s1 = {d1, d1};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const uint32_t y = ((x >> (2 * m)) & 0x00030003u) | 0x64006400u;
        const half2_t h = (__builtin_bit_cast(half2_t, y) - bias) * (m < 4 ? s0 : s1);
        if (m < 4) {
            a0[2 * (m & 3)] = h[0];
            a0[2 * (m & 3) + 1] = h[1];
        } else {
            a1[2 * (m & 3)] = h[0];
            a1[2 * (m & 3) + 1] = h[1];
        }
    }
}

// The block loop shared by both GEMMs.  blob: one expert's packed matrix
// (M rows, reduction Kd); slice: this wave's 64-row slice; act [rows][Kd]
// fp16 integer codes with as/au [rows][Kd/32]; arow[tt]: the activation row
// of this lane's column in token tile tt (-1: padding).
__device__ __forceinline__ void block_loop(const uint8_t* __restrict__ blob, int32_t M, int32_t Kd, int slice,
                                           int lane, const int64_t (&arow)[4], const _Float16* __restrict__ act,
                                           const float* __restrict__ as, const float* __restrict__ au,
                                           float4_t (&acc)[4][4]) {
    const int nblk = Kd / kBlock;
    const uint2* codes = reinterpret_cast<const uint2*>(blob) + (int64_t)slice * nblk * 64 + lane;
    const uint16_t* scl = reinterpret_cast<const uint16_t*>(blob + (int64_t)M * Kd / 4) + (int64_t)slice * nblk * 64;
    const int r16 = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[f][tt] = (float4_t){0.f, 0.f, 0.f, 0.f};
    for (int b = 0; b < nblk; ++b) {
        const uint2 c = codes[(int64_t)b * 64];
        const uint16_t* sb = scl + (int64_t)b * 64;
        const uint2 du = *reinterpret_cast<const uint2*>(sb + r16 * 4);
        const uint4 dc0 = *reinterpret_cast<const uint4*>(sb + kg * 16);
        const uint4 dc1 = *reinterpret_cast<const uint4*>(sb + kg * 16 + 8);
        half8_t A[4];
        unpack_pair(c.x, lo_half(du.x), hi_half(du.x), A[0], A[1]);
        unpack_pair(c.y, lo_half(du.y), hi_half(du.y), A[2], A[3]);
        // correction scales d of output rows 4*kg + v, fragment f: halves [v*4 + f]
        const uint32_t dw[8] = {dc0.x, dc0.y, dc0.z, dc0.w, dc1.x, dc1.y, dc1.z, dc1.w};
        float dcorr[4][4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const uint32_t w = dw[(v * 4 + f) >> 1];
                dcorr[f][v] = (float)(((v * 4 + f) & 1) ? hi_half(w) : lo_half(w));
            }
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            half8_t B = {};
            float s = 0.f, u = 0.f;
            if (arow[tt] >= 0) {
                B = *reinterpret_cast<const half8_t*>(act + arow[tt] * Kd + b * kBlock + kg * 8);
                s = as[arow[tt] * nblk + b];
                u = au[arow[tt] * nblk + b];
            }
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const float4_t q = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[f], B, (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[f][tt][v] = fmaf(q[v], s, fmaf(dcorr[f][v], u, acc[f][tt][v]));
            }
        }
    }
}

__device__ __forceinline__ float round_half_away(float t) {
    const float r = floorf(fabsf(t) + 0.5f);
    return copysignf(fminf(r, 127.0f), t);
}

// Gate/up: M = 2I rows stacked per slice as [gate 32 | up 32]; fragments 0,1
// are gate rows j0 + 16f + 4*kg + v, fragments 2,3 the up rows of the same j.
// The 32 SwiGLU outputs of one slice are exactly one int8 block of H.
__global__ void __launch_bounds__(256) gate_up_kernel(const uint8_t* __restrict__ blobs, int64_t stride,
                                                      const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles,
                                                      const int32_t* __restrict__ src, const _Float16* __restrict__ xq,
                                                      const float* __restrict__ xs, const float* __restrict__ xu,
                                                      int32_t H, int32_t I, _Float16* __restrict__ hq,
                                                      float* __restrict__ hs, float* __restrict__ hu) {
    if ((int)blockIdx.x >= *ntiles) return;
    const Tile tl = tiles[blockIdx.x];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int slice = blockIdx.y * kWaves + wave;
    if (slice >= I / 32) return;  // waves are independent: no LDS, no barrier
    const int r16 = lane & 15, kg = lane >> 4;
    int64_t arow[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int r = tt * 16 + r16;
        arow[tt] = r < tl.nrows ? (int64_t)src[tl.row0 + r] : -1;
    }
    float4_t acc[4][4];
    block_loop(blobs + (int64_t)tl.e * stride, 2 * I, H, slice, lane, arow, xq, xs, xu, acc);

    const int nbi = I / kBlock;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        float h[2][4];
        float amax = 0.f;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float g = acc[f][tt][v], up = acc[f + 2][tt][v];
                h[f][v] = g / (1.0f + expf(-g)) * up;
                amax = fmaxf(amax, fabsf(h[f][v]));
            }
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const float sh = amax / 127.0f;
        float q[2][4];
        int qsum = 0;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                q[f][v] = sh != 0.0f ? round_half_away(h[f][v] / sh) : 0.0f;
                qsum += (int)q[f][v];
            }
        qsum += __shfl_xor(qsum, 16);
        qsum += __shfl_xor(qsum, 32);
        const int r = tt * 16 + r16;
        if (r < tl.nrows) {
            const int64_t row = tl.row0 + r;
            _Float16* dst = hq + row * I + slice * 32 + 4 * kg;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const half4_t hv = {(_Float16)q[f][0], (_Float16)q[f][1], (_Float16)q[f][2], (_Float16)q[f][3]};
                *reinterpret_cast<half4_t*>(dst + 16 * f) = hv;
            }
            if (kg == 0) {
                hs[row * nbi + slice] = sh;
                hu[row * nbi + slice] = -0.5f * sh * (float)qsum;
            }
        }
    }
}

// Down: M = H rows, slice rows o0 + 16f + 4*kg + v; the epilogue adds each
// routed row, times its routing weight, into the output row of its token.
__global__ void __launch_bounds__(256) down_kernel(const uint8_t* __restrict__ blobs, int64_t stride,
                                                   const Tile* __restrict__ tiles, const int32_t* __restrict__ ntiles,
                                                   const int32_t* __restrict__ src, const float* __restrict__ prow,
                                                   const _Float16* __restrict__ hq, const float* __restrict__ hs,
                                                   const float* __restrict__ hu, int32_t H, int32_t I,
                                                   float* __restrict__ y) {
    if ((int)blockIdx.x >= *ntiles) return;
    const Tile tl = tiles[blockIdx.x];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int slice = blockIdx.y * kWaves + wave;
    if (slice >= H / 64) return;
    const int r16 = lane & 15, kg = lane >> 4;
    int64_t arow[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int r = tt * 16 + r16;
        arow[tt] = r < tl.nrows ? (int64_t)(tl.row0 + r) : -1;
    }
    float4_t acc[4][4];
    block_loop(blobs + (int64_t)tl.e * stride, H, I, slice, lane, arow, hq, hs, hu, acc);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        if (arow[tt] < 0) continue;
        const int64_t t = src[arow[tt]];
        const float w = prow[arow[tt]];
        float* dst = y + t * H + slice * 64 + 4 * kg;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int v = 0; v < 4; ++v) unsafeAtomicAdd(dst + 16 * f + v, w * acc[f][tt][v]);
    }
}

}  // namespace

hipError_t launch_gate_up(const uint8_t* blobs, int64_t stride, const Tile* tiles, const int32_t* ntiles,
                          int64_t tiles_cap, const int32_t* src, const _Float16* xq, const float* xs,
                          const float* xu, int32_t H, int32_t I, _Float16* hq, float* hs, float* hu,
                          hipStream_t st) {
    const int nslices = I / 32;
    if (tiles_cap > 0)
        hipLaunchKernelGGL(gate_up_kernel, dim3((unsigned)tiles_cap, (nslices + kWaves - 1) / kWaves), dim3(256), 0,
                           st, blobs, stride, tiles, ntiles, src, xq, xs, xu, H, I, hq, hs, hu);
    return hipGetLastError();
}

hipError_t launch_down(const uint8_t* blobs, int64_t stride, const Tile* tiles, const int32_t* ntiles,
                       int64_t tiles_cap, const int32_t* src, const float* prow, const _Float16* hq,
                       const float* hs, const float* hu, int32_t H, int32_t I, float* y, hipStream_t st) {
    const int nslices = H / 64;
    if (tiles_cap > 0)
        hipLaunchKernelGGL(down_kernel, dim3((unsigned)tiles_cap, (nslices + kWaves - 1) / kWaves), dim3(256), 0, st,
                           blobs, stride, tiles, ntiles, src, prow, hq, hs, hu, H, I, y);
    return hipGetLastError();
}

}  // namespace strata_moe
