// Router projection and route(): each token's K experts and their weights.
//
// Winery-Strata prefill.cpp page, Prefill::run, MoE half: the router
// projection of the layer input (a GEMM over the hidden dimension) followed by
// route(logits, ids, w).  route()'s body is not on the pages; the kernels take
// the K largest logits in rank order (equal logits: lower expert index first)
// and the softmax over those K logits as the weights.
//
// Exactness of the selection.  The logits are computed in fp32; near a tie the
// fp32 order may differ from the real one.  Every token whose K-th/(K+1)-th
// gap, or any gap between consecutive selected logits, is below
// delta = kTieRel * max(1, |l_K|) is re-scored: all experts within delta of
// the K-th value are recomputed as fp64 dot products and re-ranked.  With
// delta above twice the fp32 error, the result equals the ranking of the exact
// logits.
#include "internal.h"

#include <cfloat>
#include <climits>

namespace strata_moe {

namespace {

constexpr float kTieRel = 1.0f / 1024.0f;

// ---------------------------------------------------------------- logits
// logits[T][E] = x[T][H] . wr[H][E] (+ bias), 64x64 tiles, 4x4 per thread.
__global__ void __launch_bounds__(256) router_gemm_kernel(const float* __restrict__ x, const float* __restrict__ wr,
                                                          const float* __restrict__ bias, int64_t T, int32_t H,
                                                          int32_t E, float* __restrict__ out) {
    __shared__ float As[16][64 + 4];
    __shared__ float Bs[16][64 + 4];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;
    const int64_t m0 = (int64_t)blockIdx.y * 64;
    const int n0 = blockIdx.x * 64;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < H; k0 += 16) {
        {
            const int ar = tid >> 2, ac = (tid & 3) * 4;
            float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m0 + ar < T) a = *reinterpret_cast<const float4*>(x + (m0 + ar) * H + k0 + ac);
            As[ac + 0][ar] = a.x;
            As[ac + 1][ar] = a.y;
            As[ac + 2][ar] = a.z;
            As[ac + 3][ar] = a.w;
            const int br = tid >> 4, bc = (tid & 15) * 4;
            const float* wrow = wr + (int64_t)(k0 + br) * E;
#pragma unroll
            for (int i = 0; i < 4; ++i) Bs[br][bc + i] = (n0 + bc + i < E) ? wrow[n0 + bc + i] : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const float4 a = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
            const float4 b = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
            const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + ty * 4 + i;
        if (m >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n < E) out[m * E + n] = acc[i][j] + (bias ? bias[n] : 0.f);
        }
    }
}

// ------------------------------------------------------------------ top-K
// One wave per token; lane l holds experts l, l+64, ... (at most 16).
constexpr int kWaves = 4;
constexpr int kPerLane = kMaxExperts / 64;

__device__ __forceinline__ bool better(float v, int e, float bv, int be) { return v > bv || (v == bv && e < be); }
__device__ __forceinline__ bool better_d(double v, int e, double bv, int be) {
    return v > bv || (v == bv && e < be);
}

__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, const float* __restrict__ x,
                                                   const float* __restrict__ wr, const float* __restrict__ bias,
                                                   int64_t T, int32_t H, int32_t E, int32_t K,
                                                   int32_t* __restrict__ ids, float* __restrict__ p_out) {
    __shared__ int cidx_s[kWaves][kMaxExperts];
    __shared__ double cval_s[kWaves][kMaxExperts];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kWaves + wave;
    if (t >= T) return;  // whole wave; this kernel has no block-level barrier
    const float* l = logits + t * E;
    float v[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int e = lane + 64 * i;
        v[i] = e < E ? l[e] : -FLT_MAX;
    }
    // K + 1 rounds of a wave-wide argmax (larger value, then lower index).
    float selv[kMaxTopK + 1];
    int seli[kMaxTopK + 1];
    uint32_t taken = 0;
    const int rounds = K < E ? K + 1 : K;
#pragma unroll
    for (int k = 0; k <= kMaxTopK; ++k) {
        selv[k] = -FLT_MAX;
        seli[k] = INT_MAX;
        if (k >= rounds) continue;
        float bv = -FLT_MAX;
        int bi = INT_MAX;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, bi)) bv = v[i], bi = e;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            if (better(ov, oi, bv, bi)) bv = ov, bi = oi;
        }
        selv[k] = bv;
        seli[k] = bi;
        if (bi < E && (bi & 63) == lane) taken |= 1u << (bi >> 6);
    }
    float vK = -FLT_MAX;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k == K - 1) vK = selv[k];
    const float delta = kTieRel * fmaxf(1.0f, fabsf(vK));
    bool amb = false;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k + 1 < rounds && selv[k] - selv[k + 1] < delta) amb = true;

    double lv[kMaxTopK];
    int li[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) lv[k] = (double)selv[k], li[k] = seli[k];

    if (amb) {
        // Candidates: every expert within delta below the K-th value.
        int* cidx = cidx_s[wave];
        double* cval = cval_s[wave];
        const float thr = vK - delta;
        int nc = 0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int e = lane + 64 * i;
            const bool cand = e < E && v[i] >= thr;
            const uint64_t m = __ballot(cand);
            if (cand) cidx[nc + __popcll(m & ((1ull << lane) - 1ull))] = e;
            nc += __popcll(m);
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // fp64 re-score of each candidate, the wave splitting the hidden dim.
        const float* xr = x + t * H;
        for (int c = 0; c < nc; ++c) {
            const int e = cidx[c];
            double acc = 0.0;
            for (int h = lane; h < H; h += 64) acc = fma((double)xr[h], (double)wr[(int64_t)h * E + e], acc);
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
            if (bias) acc += (double)bias[e];
            if (lane == 0) cval[c] = acc;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // Re-rank the candidates (larger fp64 value, then lower index).
        double cv[kPerLane];
        int ci[kPerLane];
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int c = lane + 64 * i;
            cv[i] = c < nc ? cval[c] : -DBL_MAX;
            ci[i] = c < nc ? cidx[c] : INT_MAX;
        }
        uint32_t tk = 0;
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            if (k >= K) continue;
            double bv = -DBL_MAX;
            int bi = INT_MAX, bslot = -1;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i)
                if (!((tk >> i) & 1u) && ci[i] != INT_MAX && better_d(cv[i], ci[i], bv, bi))
                    bv = cv[i], bi = ci[i], bslot = i;
            int bl = bslot >= 0 ? lane : 64;
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) {
                const double ov = __shfl_xor(bv, off);
                const int oi = __shfl_xor(bi, off);
                const int os = __shfl_xor(bslot, off);
                const int ol = __shfl_xor(bl, off);
                if (better_d(ov, oi, bv, bi)) bv = ov, bi = oi, bslot = os, bl = ol;
            }
            lv[k] = bv;
            li[k] = bi;
            if (bl == lane && bslot >= 0) tk |= 1u << bslot;
        }
    }
    // Softmax over the K selected logits, in double.
    const double m = lv[0];
    double z = 0.0;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K) z += exp(lv[k] - m);
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K && lane == k) {
            ids[t * K + k] = li[k];
            p_out[t * K + k] = (float)(exp(lv[k] - m) / z);
        }
}

}  // namespace

hipError_t launch_router_logits(const float* x, const float* wr, const float* bias, int64_t T, int32_t H, int32_t E,
                                float* logits, hipStream_t st) {
    if (T > 0)
        hipLaunchKernelGGL(router_gemm_kernel, dim3((E + 63) / 64, (unsigned)((T + 63) / 64)), dim3(256), 0, st, x,
                           wr, bias, T, H, E, logits);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* x, const float* wr, const float* bias, int64_t T, int32_t H,
                       int32_t E, int32_t K, int32_t* ids, float* p, hipStream_t st) {
    if (T > 0)
        hipLaunchKernelGGL(topk_kernel, dim3((unsigned)((T + kWaves - 1) / kWaves)), dim3(64 * kWaves), 0, st,
                           logits, x, wr, bias, T, H, E, K, ids, p);
    return hipGetLastError();
}

}  // namespace strata_moe
