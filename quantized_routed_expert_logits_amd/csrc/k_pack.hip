// Expert packing: canonical 2-bit codes and fp16 scales -> the GEMM kernels'
// blob layout, and the inverse for round-trip checks.
//
// The pages pass each expert to the fused kernels as one blob in its own
// (Q2_0 / GGUF) layout, 16-byte aligned (Strata compare v0.1.35...v0.1.37
// page, moe_fused.hpp, Batch).  This layout is this library's own: a
// GEMM work item streams one 1280-byte record per 32-wide block of the
// reduction dimension for its 128-row slab (256 code dwords and 128 scales).
//
// For an M x Kd matrix (reduction over Kd), slab s (128 rows = 8 MFMA
// fragments of 16 rows), block b, the record at ((s * Kd/32) + b) * 1280:
//   codes  [64 lanes l][4 fragment pairs p] u32 -- 16 codes of fragments 2p
//          and 2p+1 for row r = l % 16 and k = 32b + 8*(l/16) + i (i < 8);
//          element m' = 8*(f - 2p) + i sits at bits 16*(m' % 2) + 2*(m' / 2);
//          so one lane's four dwords (all 8 fragments) are 16 contiguous bytes;
//   scales [16 rows r][4 pairs p][2] fp16 -- d of fragment 2p + w, row r; so
//          the 8 scales a lane of row r needs are 16 contiguous bytes.
// Row map: gate/up (M = 2I, slab = 64 gate + 64 up rows): fragment f < 4 is
// gate row 64s + 16f + r, f >= 4 is up row I + 64s + 16(f-4) + r; down
// (M = H): row 128s + 16f + r.
#include "internal.h"

namespace strata_moe {

namespace {

__device__ __forceinline__ int row_of(int f, int r, int s, int gate_up_I) {
    if (gate_up_I > 0) return f < 4 ? 64 * s + 16 * f + r : gate_up_I + 64 * s + 16 * (f - 4) + r;
    return kSlabRows * s + 16 * f + r;
}

// One thread per (expert, slab, block, lane, pair): one code dword, and the
// 2 scales of (row, pair) for lanes < 16.
__global__ void pack_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int32_t nexp,
                            int32_t M, int32_t Kd, int32_t gate_up_I, uint8_t* __restrict__ dst, int64_t stride) {
    const int nslab = M / kSlabRows, nblk = Kd / kBlock;
    const int64_t total = (int64_t)nexp * nslab * nblk * 256;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int tau = (int)(g % 256);
    int64_t rest = g / 256;
    const int b = (int)(rest % nblk);
    rest /= nblk;
    const int s = (int)(rest % nslab);
    const int64_t e = rest / nslab;
    const int p = tau & 3, lane = tau >> 2, r16 = lane & 15, kg = lane >> 4;
    uint32_t w = 0u;
#pragma unroll
    for (int mp = 0; mp < 16; ++mp) {
        const int f = 2 * p + mp / 8;
        const int row = row_of(f, r16, s, gate_up_I);
        const int k = kBlock * b + 8 * kg + (mp & 7);
        w |= ((uint32_t)codes[(e * M + row) * Kd + k] & 3u) << (16 * (mp & 1) + 2 * (mp >> 1));
    }
    uint8_t* rec = dst + e * stride + ((int64_t)s * nblk + b) * kRecordBytes;
    reinterpret_cast<uint32_t*>(rec)[tau] = w;
    if (kg == 0) {
        uint16_t* sc = reinterpret_cast<uint16_t*>(rec + kRecordCodeBytes) + (r16 * 4 + p) * 2;
        sc[0] = scales[(e * M + row_of(2 * p, r16, s, gate_up_I)) * nblk + b];
        sc[1] = scales[(e * M + row_of(2 * p + 1, r16, s, gate_up_I)) * nblk + b];
    }
}

__global__ void unpack_kernel(const uint8_t* __restrict__ src, int64_t stride, int32_t nexp, int32_t M, int32_t Kd,
                              int32_t gate_up_I, uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
    const int nslab = M / kSlabRows, nblk = Kd / kBlock;
    const int64_t total = (int64_t)nexp * nslab * nblk * 256;
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int tau = (int)(g % 256);
    int64_t rest = g / 256;
    const int b = (int)(rest % nblk);
    rest /= nblk;
    const int s = (int)(rest % nslab);
    const int64_t e = rest / nslab;
    const int p = tau & 3, lane = tau >> 2, r16 = lane & 15, kg = lane >> 4;
    const uint8_t* rec = src + e * stride + ((int64_t)s * nblk + b) * kRecordBytes;
    const uint32_t w = reinterpret_cast<const uint32_t*>(rec)[tau];
#pragma unroll
    for (int mp = 0; mp < 16; ++mp) {
        const int f = 2 * p + mp / 8;
        const int row = row_of(f, r16, s, gate_up_I);
        const int k = kBlock * b + 8 * kg + (mp & 7);
        codes[(e * M + row) * Kd + k] = (uint8_t)((w >> (16 * (mp & 1) + 2 * (mp >> 1))) & 3u);
    }
    if (kg == 0) {
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec + kRecordCodeBytes) + (r16 * 4 + p) * 2;
        scales[(e * M + row_of(2 * p, r16, s, gate_up_I)) * nblk + b] = sc[0];
        scales[(e * M + row_of(2 * p + 1, r16, s, gate_up_I)) * nblk + b] = sc[1];
    }
}

}  // namespace

hipError_t launch_pack(const uint8_t* codes, const uint16_t* scales, int32_t nexp, int32_t M, int32_t Kd,
                       int32_t gate_up_I, uint8_t* dst, int64_t stride, hipStream_t st) {
    const int64_t total = (int64_t)nexp * (M / kSlabRows) * (Kd / kBlock) * 256;
    if (total > 0)
        hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, codes, scales, nexp,
                           M, Kd, gate_up_I, dst, stride);
    return hipGetLastError();
}

hipError_t launch_unpack(const uint8_t* src, int64_t stride, int32_t nexp, int32_t M, int32_t Kd, int32_t gate_up_I,
                         uint8_t* codes, uint16_t* scales, hipStream_t st) {
    const int64_t total = (int64_t)nexp * (M / kSlabRows) * (Kd / kBlock) * 256;
    if (total > 0)
        hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, src, stride, nexp,
                           M, Kd, gate_up_I, codes, scales);
    return hipGetLastError();
}

}  // namespace strata_moe
