// Expert packing: canonical 2-bit codes and fp16 scales -> the GEMM kernels'
// blob layout, and the inverse for round-trip checks.
//
// The pages pass each expert to the fused kernels as one blob in its own
// (Q2_0 / GGUF) layout, 16-byte aligned (Strata compare v0.1.35...v0.1.37
// page, moe_fused.hpp, Batch).  This layout is this library's own: it is laid
// out so that one wave reads one contiguous 512-byte run of codes and one
// 128-byte run of scales per 32-wide block of the reduction dimension.
//
// For an M x Kd matrix (reduction over Kd), per 64-row slice s and block b:
//   codes  [64 lanes][2 x u32]: lane l (row r = l % 16 of each fragment,
//          k-group g = l / 16, k = 32b + 8g + i) holds 16 codes per word,
//          word w covering fragments 2w and 2w+1; element m' = 8*(f - 2w) + i
//          sits at bits 16*(m' % 2) + 2*(m' / 2).
//   scales [16 rows][4 fragments] fp16.
// Row map: gate/up (M = 2I): fragment f, row r of slice s is gate row
// 32s + 16f + r (f = 0, 1) or up row I + 32s + 16(f-2) + r (f = 2, 3);
// down (M = H): row 64s + 16f + r.
#include "internal.h"

namespace strata_moe {

namespace {

__device__ __forceinline__ int row_of(int f, int r, int s, int gate_up_I) {
    if (gate_up_I > 0) return f < 2 ? 32 * s + 16 * f + r : gate_up_I + 32 * s + 16 * (f - 2) + r;
    return 64 * s + 16 * f + r;
}

__global__ void pack_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int32_t nexp,
                            int32_t M, int32_t Kd, int32_t gate_up_I, uint8_t* __restrict__ dst, int64_t stride) {
    const int nslice = M / kSliceRows, nblk = Kd / kBlock;
    const int64_t total = (int64_t)nexp * nslice * nblk * 64;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int lane = (int)(g % 64);
    int64_t rest = g / 64;
    const int b = (int)(rest % nblk);
    rest /= nblk;
    const int s = (int)(rest % nslice);
    const int64_t e = rest / nslice;
    const int r16 = lane & 15, kg = lane >> 4;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int word = 0; word < 2; ++word)
#pragma unroll
        for (int mp = 0; mp < 16; ++mp) {
            const int f = 2 * word + mp / 8;
            const int row = row_of(f, r16, s, gate_up_I);
            const int k = kBlock * b + 8 * kg + (mp & 7);
            const uint32_t c = codes[(e * M + row) * Kd + k] & 3u;
            w[word] |= c << (16 * (mp & 1) + 2 * (mp >> 1));
        }
    uint8_t* blob = dst + e * stride;
    reinterpret_cast<uint2*>(blob)[((int64_t)s * nblk + b) * 64 + lane] = make_uint2(w[0], w[1]);
    uint16_t* sd = reinterpret_cast<uint16_t*>(blob + (int64_t)M * Kd / 4);
    sd[((int64_t)s * nblk + b) * 64 + lane] = scales[(e * M + row_of(lane & 3, lane >> 2, s, gate_up_I)) * nblk + b];
}

__global__ void unpack_kernel(const uint8_t* __restrict__ src, int64_t stride, int32_t nexp, int32_t M, int32_t Kd,
                              int32_t gate_up_I, uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
    const int nslice = M / kSliceRows, nblk = Kd / kBlock;
    const int64_t total = (int64_t)nexp * nslice * nblk * 64;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int lane = (int)(g % 64);
    int64_t rest = g / 64;
    const int b = (int)(rest % nblk);
    rest /= nblk;
    const int s = (int)(rest % nslice);
    const int64_t e = rest / nslice;
    const int r16 = lane & 15, kg = lane >> 4;
    const uint8_t* blob = src + e * stride;
    const uint2 wv = reinterpret_cast<const uint2*>(blob)[((int64_t)s * nblk + b) * 64 + lane];
    const uint32_t w[2] = {wv.x, wv.y};
#pragma unroll
    for (int word = 0; word < 2; ++word)
#pragma unroll
        for (int mp = 0; mp < 16; ++mp) {
            const int f = 2 * word + mp / 8;
            const int row = row_of(f, r16, s, gate_up_I);
            const int k = kBlock * b + 8 * kg + (mp & 7);
            codes[(e * M + row) * Kd + k] = (uint8_t)((w[word] >> (16 * (mp & 1) + 2 * (mp >> 1))) & 3u);
        }
    const uint16_t* sd = reinterpret_cast<const uint16_t*>(blob + (int64_t)M * Kd / 4);
    scales[(e * M + row_of(lane & 3, lane >> 2, s, gate_up_I)) * nblk + b] = sd[((int64_t)s * nblk + b) * 64 + lane];
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, const uint16_t* scales, int32_t nexp, int32_t M, int32_t Kd,
                       int32_t gate_up_I, uint8_t* dst, int64_t stride, hipStream_t st) {
    const int64_t total = (int64_t)nexp * (M / kSliceRows) * (Kd / kBlock) * 64;
    if (total > 0)
        hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, codes, scales, nexp,
                           M, Kd, gate_up_I, dst, stride);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* src, int64_t stride, int32_t nexp, int32_t M, int32_t Kd, int32_t gate_up_I,
                         uint8_t* codes, uint16_t* scales, hipStream_t st) {
    const int64_t total = (int64_t)nexp * (M / kSliceRows) * (Kd / kBlock) * 64;
    if (total > 0)
        hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, src, stride, nexp,
                           M, Kd, gate_up_I, codes, scales);
    return hipGetLastError();
}

}  // namespace strata_moe
