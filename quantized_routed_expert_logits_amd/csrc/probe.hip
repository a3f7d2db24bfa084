// libstrata_probe: measurements of the matrix unit that the layer's design
// and its error model rest on.  Not part of the layer (no layer entry point
// calls into it); the benchmark and the tests load it beside libstrata_moe.
//
//   strata_probe_mfma_rate: the issue rate of one MFMA form (8 independent
//     accumulator chains per wave, every SIMD busy), as ops per second.  This
//     is the measured peak next to the published one.
//   strata_probe_scaled_blocks: the rate of "per-32-block products, each
//     scaled into an fp32 accumulator" on register-resident operands, in two
//     formulations: fp16 MFMA with the weight scale inside the operand and
//     one FMA per output (the layer's form), and int8 MFMA with both scales
//     applied per output (convert, multiply, FMA).  Output-blocks per second.
//   strata_probe_scaled_tiles: the same fp16 form at the shape of the 4-wave
//     gate/up kernel (6 output tiles of 32 x 32 per wave and block: 24
//     v_mfma_f32_16x16x32_f16 and 96 FMAs), or with v_mfma_f32_32x32x16_f16
//     (two chained per tile and block, 16 FMAs per lane), operands in
//     registers: the ceiling of the exact block-scaled products before any
//     load, unpack or barrier.
//   strata_probe_block_step: that shape built up toward the kernel's block
//     step: (0) the products and FMAs with the three activation fragments of
//     each block loaded from a small buffer; (1) plus a stand-in for the
//     weight unpack (one dword per lane, 25 VALU into two fragments) whose
//     fragments the four waves exchange through LDS with one barrier per
//     block; (2) the same with one barrier per two blocks.
//   strata_probe_mfma_f16: one v_mfma_f32_16x16x32_f16 on given operands
//     (row-major A [16][32], B [32][16], C [16][16]), to check how it rounds.
//   strata_probe_hbm_read: the read bandwidth a plain streaming kernel gets
//     from HBM (16-byte loads, four in flight per thread, a grid-stride
//     loop), the measured ceiling beside the published 8 TB/s.
#include <hip/hip_runtime.h>

#include <cstdint>

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int16v_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int kChains = 8;
constexpr int kWavesPerGroup = 4;

enum Kind { kF16_16x16x32, kF16_32x32x16, kI8_16x16x64, kI8_32x32x32, kI8_16x16x32, kI8_32x32x16, kKinds };

// 2 M N K of each form
__host__ __device__ constexpr double kind_ops(int k) {
    return k == kF16_16x16x32 ? 2.0 * 16 * 16 * 32
         : k == kF16_32x32x16 ? 2.0 * 32 * 32 * 16
         : k == kI8_16x16x64  ? 2.0 * 16 * 16 * 64
         : k == kI8_32x32x32  ? 2.0 * 32 * 32 * 32
         : k == kI8_16x16x32  ? 2.0 * 16 * 16 * 32
                              : 2.0 * 32 * 32 * 16;
}

// seed: a value the host passes as 0 (operands stay data-dependent, so the
// compiler keeps every MFMA); out receives one word per wave.
template <int kKind>
__global__ void __launch_bounds__(64 * kWavesPerGroup) mfma_rate_kernel(int32_t iters, int32_t seed,
                                                                        float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int s = seed + lane;
    float r = 0.f;
    if constexpr (kKind == kF16_16x16x32 || kKind == kF16_32x32x16) {
        half8_t a, b;
        for (int i = 0; i < 8; ++i) a[i] = (_Float16)(float)(s + i), b[i] = (_Float16)(float)(s - i);
        if constexpr (kKind == kF16_16x16x32) {
            float4_t c[kChains] = {};
            for (int it = 0; it < iters; ++it)
#pragma unroll
                for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kChains; ++j) r += c[j][0];
        } else {
            float16_t c[kChains / 2] = {};
            for (int it = 0; it < iters; ++it)
#pragma unroll
                for (int j = 0; j < kChains / 2; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kChains / 2; ++j) r += c[j][0];
        }
    } else if constexpr (kKind == kI8_16x16x64 || kKind == kI8_32x32x32) {
        const int4_t a = {s, s + 1, s + 2, s + 3}, b = {s ^ 5, s ^ 6, s ^ 7, s ^ 8};
        if constexpr (kKind == kI8_16x16x64) {
            int4_t c[kChains] = {};
            for (int it = 0; it < iters; ++it)
#pragma unroll
                for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kChains; ++j) r += (float)c[j][0];
        } else {
            int16v_t c[kChains / 2] = {};
            for (int it = 0; it < iters; ++it)
#pragma unroll
                for (int j = 0; j < kChains / 2; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kChains / 2; ++j) r += (float)c[j][0];
        }
    } else {
        const long a = (long)s * 0x0101010101010101L, b = (long)(s ^ 3) * 0x0101010101010101L;
        if constexpr (kKind == kI8_16x16x32) {
            int4_t c[kChains] = {};
            for (int it = 0; it < iters; ++it)
#pragma unroll
                for (int j = 0; j < kChains; ++j) c[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kChains; ++j) r += (float)c[j][0];
        } else {
            int16v_t c[kChains / 2] = {};
            for (int it = 0; it < iters; ++it)
#pragma unroll
                for (int j = 0; j < kChains / 2; ++j) c[j] = __builtin_amdgcn_mfma_i32_32x32x16_i8(a, b, c[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < kChains / 2; ++j) r += (float)c[j][0];
        }
    }
    if (lane == 0) out[blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6)] = r;
}

// Scaled per-block products on register-resident operands: per block, the
// wave forms the products of one 32-wide block for a 32 x 32 output tile and
// adds them, scaled, into fp32 accumulators.
//   kF16: four v_mfma_f32_16x16x32_f16 (A = the weight codes times d, exact
//     in fp16; zero accumulator), then per output one FMA with the token's
//     activation scale: 16 FMAs per lane.
//   kI8: one v_mfma_i32_32x32x32_i8 (zero accumulator), then per output the
//     int32 -> fp32 conversion, the product d_row * s_token and the FMA:
//     16 x 3 VALU per lane.
// The scales change every block (the per-32 format).
template <bool kI8>
__global__ void __launch_bounds__(64 * kWavesPerGroup) scaled_blocks_kernel(int32_t blocks, int32_t seed,
                                                                            float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int s = seed + lane;
    float acc[16] = {};
    float dsc[16];
    for (int i = 0; i < 16; ++i) dsc[i] = 1.0f + (float)((s + i) & 7) * 0x1p-10f;
    float ssc = 1.0f + (float)(s & 15) * 0x1p-12f;
    if constexpr (kI8) {
        int4_t a = {s, s + 1, s + 2, s + 3}, b = {s ^ 5, s ^ 6, s ^ 7, s ^ 8};
#pragma unroll 2
        for (int blk = 0; blk < blocks; ++blk) {
            const int16v_t p = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, (int16v_t){}, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = fmaf((float)p[i], dsc[i] * ssc, acc[i]);
            a += 1;  // the next block's operands
            ssc += 0x1p-20f;
        }
    } else {
        half8_t a[4], b;
        for (int f = 0; f < 4; ++f)
            for (int i = 0; i < 8; ++i) a[f][i] = (_Float16)(float)((s + i + f) & 3);
        for (int i = 0; i < 8; ++i) b[i] = (_Float16)(float)(s - i);
        const half8_t one = {1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll 2
        for (int blk = 0; blk < blocks; ++blk) {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[f], b, (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[4 * f + v] = fmaf(p[v], ssc, acc[4 * f + v]);
            }
            b += one;  // the next block's operands
            ssc += 0x1p-20f;
        }
    }
    float r = 0.f;
    for (int i = 0; i < 16; ++i) r += acc[i];
    if (lane == 0) out[blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6)] = r;
}

// Per block, kTiles output tiles of 32 x 32 (the rows of tile t come from
// its own A operands): kForm 0 forms each with four v_mfma_f32_16x16x32_f16
// (zero accumulator), kForm 1 with two chained v_mfma_f32_32x32x16_f16; then
// one FMA per output with the block's activation scale.  Every tile's A
// operands differ as vectors (no two products are the same expression, so
// the compiler keeps every MFMA).
template <int kForm, int kTiles>
__global__ void __launch_bounds__(64 * kWavesPerGroup, 2) scaled_tiles_kernel(int32_t blocks, int32_t seed,
                                                                             float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int s = seed + lane;
    float acc[kTiles][16] = {};
    float ssc = 1.0f + (float)(s & 15) * 0x1p-12f;
    half8_t a[kTiles][4], b[2];
    for (int t = 0; t < kTiles; ++t)
        for (int f = 0; f < 4; ++f)
            for (int i = 0; i < 8; ++i) a[t][f][i] = (_Float16)(float)(((s * (2 * t + 1) + 5 * f + 3 * i) & 7) - 3);
    for (int j = 0; j < 2; ++j)
        for (int i = 0; i < 8; ++i) b[j][i] = (_Float16)(float)(s - i + j);
    const half8_t one = {1, 1, 1, 1, 1, 1, 1, 1};
    for (int blk = 0; blk < blocks; ++blk) {
#pragma unroll
        for (int t = 0; t < kTiles; ++t) {
            if constexpr (kForm == 0) {
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const float4_t p =
                        __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t][f], b[0], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[t][4 * f + v] = fmaf(p[v], ssc, acc[t][4 * f + v]);
                }
            } else {
                float16_t p = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[t][0], b[0], (float16_t){}, 0, 0, 0);
                p = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[t][1], b[1], p, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[t][v] = fmaf(p[v], ssc, acc[t][v]);
            }
        }
        b[0] += one;  // the next block's operands
        b[1] += one;
        ssc += 0x1p-20f;
    }
    float r = 0.f;
    for (int t = 0; t < kTiles; ++t)
        for (int i = 0; i < 16; ++i) r += acc[t][i];
    if (lane == 0) out[blockIdx.x * kWavesPerGroup + (threadIdx.x >> 6)] = r;
}

// The block step of the 4-wave gate/up kernel, built up (see the file
// header).  kStep 0: 8 weight fragments in registers; 1 and 2: each wave
// makes two of them from a loaded dword and the waves exchange them through
// LDS (buffers kb & 1, or kb & 3 with one barrier per block pair).  Every
// wave: 3 token tiles x 8 fragments of MFMAs and one FMA per output, the next
// block's 3 activation fragments loaded from act (256 fragments of 1 KiB).
template <int kStep>
__global__ void __launch_bounds__(64 * kWavesPerGroup, 2) block_step_kernel(int32_t blocks, int32_t seed,
                                                                           const half8_t* __restrict__ act,
                                                                           const uint32_t* __restrict__ rec,
                                                                           float* __restrict__ out) {
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    __shared__ half8_t a_lds[kStep == 2 ? 4 : 2][8][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, s = seed + lane;
    float4_t acc[8][3] = {};
    float ssc = 1.0f + (float)(s & 15) * 0x1p-12f;
    half8_t a[8], bf[2][3];
    for (int f = 0; f < 8; ++f)
        for (int i = 0; i < 8; ++i) a[f][i] = (_Float16)(float)(((s * (2 * f + 1) + 3 * i) & 7) - 3);
    for (int t = 0; t < 3; ++t)
        for (int i = 0; i < 8; ++i) bf[0][t][i] = bf[1][t][i] = (_Float16)(float)(s - i + t);
    const int base = (blockIdx.x * kWavesPerGroup + wave) % 16;
    // two fp16 fragments from one dword: 8 AND-ORs (a shift for the high codes), 8 packed subtracts and
    // 8 packed multiplies, as the kernel's unpack
    auto unpack = [&](int b, half8_t& r0, half8_t& r1) {
        const uint32_t xw = rec[((base + b) & 255) * 256 + threadIdx.x], hi = xw >> 10;
        const half2_t c = {(_Float16)1025.0f, (_Float16)1025.0f}, d = {(_Float16)0.01f, (_Float16)0.02f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t o0 = ((q < 5 ? xw : hi) & (0x00030003u << (2 * (q % 5)))) | (0x64006400u - (q << 26));
            const uint32_t o1 =
                (((q + 4) < 5 ? xw : hi) & (0x00030003u << (2 * ((q + 4) % 5)))) | (0x64006400u - ((q + 4) << 26));
            const half2_t v0 = (__builtin_bit_cast(half2_t, o0) - c) * d, v1 = (__builtin_bit_cast(half2_t, o1) - c) * d;
            r0[2 * q] = v0[0], r0[2 * q + 1] = v0[1];
            r1[2 * q] = v1[0], r1[2 * q + 1] = v1[1];
        }
    };
    auto products = [&](int b, int h) {
#pragma unroll
        for (int t = 0; t < 3; ++t) bf[h ^ 1][t] = act[((base + 3 * b + t) & 255) * 64 + lane];
#pragma unroll
        for (int f = 0; f < 8; ++f)
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                const float4_t p =
                    __builtin_amdgcn_mfma_f32_16x16x32_f16(a[f], bf[h][t], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[f][t][v] = fmaf(p[v], ssc, acc[f][t][v]);
            }
        ssc += 0x1p-20f;
    };
    for (int blk = 0; blk < blocks; blk += 2) {
        if constexpr (kStep == 2) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                half8_t r0, r1;
                unpack(blk + h, r0, r1);
                a_lds[(blk + h) & 3][2 * wave][lane] = r0;
                a_lds[(blk + h) & 3][2 * wave + 1][lane] = r1;
            }
            __syncthreads();
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int b = blk + h;
            if constexpr (kStep == 1) {
                half8_t r0, r1;
                unpack(b, r0, r1);
                a_lds[b & 1][2 * wave][lane] = r0;
                a_lds[b & 1][2 * wave + 1][lane] = r1;
                __syncthreads();
            }
            if constexpr (kStep > 0) {
#pragma unroll
                for (int f = 0; f < 8; ++f) a[f] = a_lds[b & (kStep == 2 ? 3 : 1)][f][lane];
            }
            products(b, h);
        }
    }
    float r = 0.f;
    for (int f = 0; f < 8; ++f)
        for (int t = 0; t < 3; ++t) r += acc[f][t][0] + acc[f][t][3];
    if (lane == 0) out[blockIdx.x * kWavesPerGroup + wave] = r;
}

// One 16x16x32 fp16 MFMA on row-major operands, one wave.  The lane layout
// of the instruction: A lane l holds row l % 16, k = 8 (l / 16) .. + 7; B
// lane l holds column l % 16, the same k; C/D lane l holds rows
// 4 (l / 16) + v, column l % 16.
__global__ void mfma_f16_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                const float* __restrict__ C, float* __restrict__ D) {
    const int l = threadIdx.x, r = l & 15, g = l >> 4;
    half8_t a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)A[r * 32 + 8 * g + i];
        b[i] = (_Float16)B[(8 * g + i) * 16 + r];
    }
    float4_t c;
    for (int v = 0; v < 4; ++v) c[v] = C[(4 * g + v) * 16 + r];
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    for (int v = 0; v < 4; ++v) D[(4 * g + v) * 16 + r] = c[v];
}

// Streaming read of n16 16-byte words: four independent loads per thread and
// turn, their XOR kept; a store only on a value the fill never makes, so
// the kernel writes nothing and the loads cannot be dropped.
__global__ void __launch_bounds__(256) hbm_read_kernel(const int4_t* __restrict__ src, int64_t n16,
                                                       int4_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int4_t acc = {0, 0, 0, 0};
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const int4_t a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a ^ b ^ c ^ d;
    }
    for (; i < n16; i += stride) acc ^= src[i];
    if (acc[0] == 0x5eed1e55 && acc[1] == 0x5eed1e55) out[blockIdx.x] = acc;
}

int run_timed(void (*launch)(hipStream_t), double* ms) {
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -4;
    launch(nullptr);  // warm
    (void)hipEventRecord(e0, nullptr);
    launch(nullptr);
    (void)hipEventRecord(e1, nullptr);
    int rc = hipEventSynchronize(e1) == hipSuccess ? 0 : -4;
    float t = 0.f;
    if (rc == 0 && hipEventElapsedTime(&t, e0, e1) != hipSuccess) rc = -4;
    *ms = t;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (hipGetLastError() != hipSuccess) rc = -4;
    return rc;
}

float* g_out = nullptr;
int32_t g_iters = 0, g_groups = 0;
const int4_t* g_src = nullptr;
int64_t g_n16 = 0;

void launch_read(hipStream_t st) {
    hipLaunchKernelGGL(hbm_read_kernel, dim3(g_groups), dim3(256), 0, st, g_src, g_n16,
                       reinterpret_cast<int4_t*>(g_out));
}

template <int kKind>
void launch_rate(hipStream_t st) {
    hipLaunchKernelGGL(mfma_rate_kernel<kKind>, dim3(g_groups), dim3(64 * kWavesPerGroup), 0, st, g_iters, 0, g_out);
}
template <bool kI8>
void launch_scaled(hipStream_t st) {
    hipLaunchKernelGGL(scaled_blocks_kernel<kI8>, dim3(g_groups), dim3(64 * kWavesPerGroup), 0, st, g_iters, 0, g_out);
}
const half8_t* g_act = nullptr;
const uint32_t* g_rec = nullptr;
template <int kStep>
void launch_step(hipStream_t st) {
    hipLaunchKernelGGL(block_step_kernel<kStep>, dim3(g_groups), dim3(64 * kWavesPerGroup), 0, st, g_iters, 0, g_act,
                       g_rec, g_out);
}
template <int kForm, int kTiles>
void launch_tiles(hipStream_t st) {
    hipLaunchKernelGGL((scaled_tiles_kernel<kForm, kTiles>), dim3(g_groups), dim3(64 * kWavesPerGroup), 0, st,
                       g_iters, 0, g_out);
}

}  // namespace

extern "C" {

// Kinds: 0 f16 16x16x32, 1 f16 32x32x16, 2 i8 16x16x64, 3 i8 32x32x32,
// 4 i8 16x16x32, 5 i8 32x32x16.  groups workgroups of 4 waves, iters rounds
// of 8 accumulator chains' worth of MFMAs per wave.  Writes the rate in
// ops/s (2 M N K per MFMA) and the kernel time.  Returns 0, -1 (arguments),
// -4 (a HIP call failed).
int strata_probe_mfma_rate(int kind, int32_t groups, int32_t iters, double* ops_per_s, double* ms) {
    if (kind < 0 || kind >= kKinds || groups < 1 || iters < 1 || !ops_per_s || !ms) return -1;
    if (hipMalloc(&g_out, sizeof(float) * groups * kWavesPerGroup) != hipSuccess) return -4;
    g_iters = iters;
    g_groups = groups;
    void (*fns[kKinds])(hipStream_t) = {launch_rate<0>, launch_rate<1>, launch_rate<2>,
                                        launch_rate<3>, launch_rate<4>, launch_rate<5>};
    const int rc = run_timed(fns[kind], ms);
    (void)hipFree(g_out);
    g_out = nullptr;
    // the 32x32 forms run kChains / 2 chains (each instruction is twice as long)
    const bool wide = kind == kF16_32x32x16 || kind == kI8_32x32x32 || kind == kI8_32x32x16;
    const double mfmas = (double)groups * kWavesPerGroup * iters * (wide ? kChains / 2 : kChains);
    *ops_per_s = rc == 0 && *ms > 0 ? mfmas * kind_ops(kind) / (*ms * 1e-3) : 0.0;
    return rc;
}

// i8 = 0: the fp16 formulation, 1: the int8 one.  Writes 32 x 32 x blocks
// output-blocks per wave over the kernel time, per second.
int strata_probe_scaled_blocks(int i8, int32_t groups, int32_t blocks, double* out_blocks_per_s, double* ms) {
    if (groups < 1 || blocks < 1 || !out_blocks_per_s || !ms) return -1;
    if (hipMalloc(&g_out, sizeof(float) * groups * kWavesPerGroup) != hipSuccess) return -4;
    g_iters = blocks;
    g_groups = groups;
    const int rc = run_timed(i8 ? launch_scaled<true> : launch_scaled<false>, ms);
    (void)hipFree(g_out);
    g_out = nullptr;
    const double n = (double)groups * kWavesPerGroup * blocks * 1024.0;
    *out_blocks_per_s = rc == 0 && *ms > 0 ? n / (*ms * 1e-3) : 0.0;
    return rc;
}

// form 0: v_mfma_f32_16x16x32_f16, 1: v_mfma_f32_32x32x16_f16; tiles 1 or 6
// output tiles of 32 x 32 per wave and block.  Writes 32 x 32 x tiles x
// blocks output-blocks per wave over the kernel time, per second.  Returns
// 0, -1 (arguments), -4 (a HIP call failed).
int strata_probe_scaled_tiles(int form, int tiles, int32_t groups, int32_t blocks, double* out_blocks_per_s,
                              double* ms) {
    if ((form != 0 && form != 1) || (tiles != 1 && tiles != 6) || groups < 1 || blocks < 1 || !out_blocks_per_s ||
        !ms)
        return -1;
    if (hipMalloc(&g_out, sizeof(float) * groups * kWavesPerGroup) != hipSuccess) return -4;
    g_iters = blocks;
    g_groups = groups;
    void (*fn)(hipStream_t) = form == 0 ? (tiles == 1 ? launch_tiles<0, 1> : launch_tiles<0, 6>)
                                        : (tiles == 1 ? launch_tiles<1, 1> : launch_tiles<1, 6>);
    const int rc = run_timed(fn, ms);
    (void)hipFree(g_out);
    g_out = nullptr;
    const double n = (double)groups * kWavesPerGroup * blocks * 1024.0 * tiles;
    *out_blocks_per_s = rc == 0 && *ms > 0 ? n / (*ms * 1e-3) : 0.0;
    return rc;
}

// step 0, 1 or 2 (see block_step_kernel); blocks even.  Writes 6 x 32 x 32
// output-blocks per wave and block over the kernel time, per second.
// Returns 0, -1 (arguments), -4 (a HIP call failed).
int strata_probe_block_step(int step, int32_t groups, int32_t blocks, double* out_blocks_per_s, double* ms) {
    if (step < 0 || step > 2 || groups < 1 || blocks < 2 || blocks % 2 || !out_blocks_per_s || !ms) return -1;
    void* act = nullptr;
    void* rec = nullptr;
    if (hipMalloc(&act, sizeof(half8_t) * 64 * 256) != hipSuccess) return -4;
    if (hipMalloc(&rec, sizeof(uint32_t) * 256 * 256) != hipSuccess) {
        (void)hipFree(act);
        return -4;
    }
    int rc = hipMemset(act, 0, sizeof(half8_t) * 64 * 256) == hipSuccess &&
                     hipMemset(rec, 0x5a, sizeof(uint32_t) * 256 * 256) == hipSuccess &&
                     hipMalloc(&g_out, sizeof(float) * groups * kWavesPerGroup) == hipSuccess
                 ? 0
                 : -4;
    if (rc == 0) {
        g_act = static_cast<const half8_t*>(act);
        g_rec = static_cast<const uint32_t*>(rec);
        g_iters = blocks;
        g_groups = groups;
        rc = run_timed(step == 0 ? launch_step<0> : step == 1 ? launch_step<1> : launch_step<2>, ms);
        (void)hipFree(g_out);
        g_out = nullptr;
    }
    (void)hipFree(act);
    (void)hipFree(rec);
    g_act = nullptr;
    g_rec = nullptr;
    const double n = (double)groups * kWavesPerGroup * blocks * 1024.0 * 6;
    *out_blocks_per_s = rc == 0 && *ms > 0 ? n / (*ms * 1e-3) : 0.0;
    return rc;
}

// D = A B + C for one v_mfma_f32_16x16x32_f16; host arrays A [16][32],
// B [32][16] (values rounded to fp16 on the device), C, D [16][16] fp32.
int strata_probe_mfma_f16(const float* A, const float* B, const float* C, float* D) {
    if (!A || !B || !C || !D) return -1;
    float* d = nullptr;
    if (hipMalloc(&d, sizeof(float) * (512 + 512 + 256 + 256)) != hipSuccess) return -4;
    int rc = 0;
    if (hipMemcpy(d, A, 512 * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(d + 512, B, 512 * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(d + 1024, C, 256 * 4, hipMemcpyHostToDevice) != hipSuccess)
        rc = -4;
    if (rc == 0) {
        hipLaunchKernelGGL(mfma_f16_kernel, dim3(1), dim3(64), 0, nullptr, d, d + 512, d + 1024, d + 1280);
        if (hipMemcpy(D, d + 1280, 256 * 4, hipMemcpyDeviceToHost) != hipSuccess) rc = -4;
    }
    (void)hipFree(d);
    return rc;
}

// Reads `bytes` (a multiple of 16, at least 1 MiB) of device memory filled
// with ones, `groups` workgroups of 256 threads; the first pass is untimed.
// With bytes well above the 256 MB Infinity Cache the timed pass streams
// from HBM.  Writes GB/s (1e9 bytes) and the kernel time.  Returns 0, -1
// (arguments), -4 (a HIP call failed).
int strata_probe_hbm_read(int64_t bytes, int32_t groups, double* gbs, double* ms) {
    if (bytes < (1 << 20) || bytes % 16 || groups < 1 || !gbs || !ms) return -1;
    void* buf = nullptr;
    if (hipMalloc(&buf, (size_t)bytes) != hipSuccess) return -4;
    if (hipMalloc(&g_out, sizeof(int4_t) * groups) != hipSuccess) {
        (void)hipFree(buf);
        return -4;
    }
    int rc = hipMemset(buf, 1, (size_t)bytes) == hipSuccess ? 0 : -4;
    g_src = static_cast<const int4_t*>(buf);
    g_n16 = bytes / 16;
    g_groups = groups;
    if (rc == 0) rc = run_timed(launch_read, ms);
    (void)hipFree(buf);
    (void)hipFree(g_out);
    g_out = nullptr;
    g_src = nullptr;
    *gbs = rc == 0 && *ms > 0 ? (double)bytes / (*ms * 1e-3) / 1e9 : 0.0;
    return rc;
}

}  // extern "C"
