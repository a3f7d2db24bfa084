// Per-32 int8 rounding of fp32 rows (the layer input, once per token), plus
// small conversion kernels.
//
// Strata compare v0.1.35...v0.1.37 page, include/strata/prefill/moe_fused.hpp,
// quantize_act: the activations are rounded to int8 once per token with one
// scale per 32 values.  The rounding is not on the pages; the kernels take
// s = max|v| / 127 and q = round-half-away-from-zero(v / s), both divisions
// correctly rounded fp32 (IEEE), |q| <= 127, s = 0 and q = 0 for an all-zero
// block.
//
// Layout: 8 lanes cover one block of 32 values, one float4 each, so a wave
// reads 1 KiB of contiguous input per instruction.  Outputs per block: the
// codes as exact fp16 integers (the GEMM operand), optionally as int8, the
// scale, and u = -0.5 * s * (sum of the block's codes), the term the 2-bit
// weight offset contributes (see k_experts.hip).
#include "internal.h"

namespace strata_moe {

namespace {

__device__ __forceinline__ float round_half_away(float t) {
    const float r = floorf(fabsf(t) + 0.5f);  // exact: |t| <= 127.00002
    return copysignf(fminf(r, 127.0f), t);
}

__global__ void __launch_bounds__(256) quantize_kernel(const float4* __restrict__ v, int64_t n4,
                                                       _Float16* __restrict__ q16, int8_t* __restrict__ q8,
                                                       float* __restrict__ s_out, float* __restrict__ u_out,
                                                       float4* __restrict__ zero_out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
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
    int sum = (int)q[0] + (int)q[1] + (int)q[2] + (int)q[3];
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    sum += __shfl_xor(sum, 4);
    if (!valid) return;
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    if (q16) {
        half4_t h = {(_Float16)q[0], (_Float16)q[1], (_Float16)q[2], (_Float16)q[3]};
        reinterpret_cast<half4_t*>(q16)[g] = h;
    }
    if (q8) {
        const uint32_t packed = ((uint32_t)(uint8_t)(int8_t)(int)q[0]) | ((uint32_t)(uint8_t)(int8_t)(int)q[1] << 8) |
                                ((uint32_t)(uint8_t)(int8_t)(int)q[2] << 16) | ((uint32_t)(uint8_t)(int8_t)(int)q[3] << 24);
        reinterpret_cast<uint32_t*>(q8)[g] = packed;
    }
    if ((g & 7) == 0) {
        s_out[g >> 3] = s;
        if (u_out) u_out[g >> 3] = -0.5f * s * (float)sum;
    }
    if (zero_out) zero_out[g] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ void f16_to_i8_kernel(const _Float16* __restrict__ v, int64_t count, int8_t* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < count) out[g] = (int8_t)(int)v[g];
}

__global__ void i8_to_f16_kernel(const int8_t* __restrict__ v, int64_t count, _Float16* __restrict__ out) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < count) out[g] = (_Float16)(int)v[g];
}

__global__ void fill_zero_kernel(float* __restrict__ p, int64_t count) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g < count) p[g] = 0.0f;
}

// u = -0.5 * s * (sum of the block's codes) for given int8 codes and scales.
__global__ void block_correction_kernel(const int8_t* __restrict__ q, const float* __restrict__ s, int64_t nblocks,
                                        float* __restrict__ u) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= nblocks) return;
    int sum = 0;
    for (int i = 0; i < kBlock; ++i) sum += q[g * kBlock + i];
    u[g] = -0.5f * s[g] * (float)sum;
}

inline unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_quantize(const float* v, int64_t rows, int32_t cols, _Float16* q16, int8_t* q8, float* s, float* u,
                           float* zero_out, hipStream_t st) {
    const int64_t n4 = rows * cols / 4;
    if (n4 > 0)
        hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(n4, 256)), dim3(256), 0, st,
                           reinterpret_cast<const float4*>(v), n4, q16, q8, s, u,
                           reinterpret_cast<float4*>(zero_out));
    return hipGetLastError();
}

hipError_t launch_f16_to_i8(const _Float16* v, int64_t count, int8_t* out, hipStream_t st) {
    if (count > 0) hipLaunchKernelGGL(f16_to_i8_kernel, dim3(grid_for(count, 256)), dim3(256), 0, st, v, count, out);
    return hipGetLastError();
}

hipError_t launch_i8_to_f16(const int8_t* v, int64_t count, _Float16* out, hipStream_t st) {
    if (count > 0) hipLaunchKernelGGL(i8_to_f16_kernel, dim3(grid_for(count, 256)), dim3(256), 0, st, v, count, out);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t st) {
    if (count > 0) hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(count, 256)), dim3(256), 0, st, p, count);
    return hipGetLastError();
}

hipError_t launch_block_correction(const int8_t* q, const float* s, int64_t rows, int32_t cols, float* u,
                                   hipStream_t st) {
    const int64_t nb = rows * (cols / kBlock);
    if (nb > 0)
        hipLaunchKernelGGL(block_correction_kernel, dim3(grid_for(nb, 256)), dim3(256), 0, st, q, s, nb, u);
    return hipGetLastError();
}

}  // namespace strata_moe
