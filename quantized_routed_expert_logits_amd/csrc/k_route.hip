// Router projection and route(): each token's K experts and their weights.
//
// Winery-Strata prefill.cpp page, Prefill::run, MoE half: the router
// projection of the layer input (a GEMM over the hidden dimension) followed by
// route(logits, ids, w).  route()'s body is not on the pages; the kernels take
// the K largest logits in rank order (equal logits: lower expert index first)
// and the softmax over those K logits as the weights.
//
// Exactness of the selection.  The logits carry an error of the order of an
// fp32 dot product's (see the router kernel below); near a tie their order
// may differ from the real one.  For a token where some gap between
// consecutive ranks 0..K (fp32 order) is below delta, the experts whose order
// is in doubt (the ranks next to such a gap, and every expert within delta
// below the K-th value) are recomputed as fp64 dot products and everything
// within delta of the K-th value is re-ranked.  With delta above twice the
// logits' error, the result equals the ranking of the exact logits.
// delta = 2 err_t (1% on top for the fp32 norms), with err_t the token's
// error bound.  Each term of the dot product is carried as three fp16
// products (hi*hi + hi*lo + lo*hi of the two operands' halves: within
// 2^-20 |x w| of x w), each exact in fp32.  v_mfma_f32_16x16x32_f16 sums its
// 32 products in fp32-class arithmetic (at most 31 additions) and then adds
// that sum to the accumulator.  The reduction over H is split into ns equal
// ranges; within a range the fp32 accumulator chains end after kRouterChain
// k blocks (3 MFMAs each) and are added into fp64 sums, which the epilogue
// rounds to fp32 once (with the bias, in range 0); the top-K adds the ns
// range values in order.  So a product passes through at most
// 31 + 3 min(H / (32 ns), kRouterChain) fp32 additions, the fp64 ones (each
// within 2^-52, counted as one more) and ns roundings of a value at most
// sum_h |x_h w_h| + |b_e|; each fp32 addition is taken within 2^-23 of its
// exact result (truncation as well as rounding), and sum_h |x_h w_h| <=
// ||x||_2 ||w_e||_2 (Cauchy-Schwarz).  With 8 additions to spare:
//     err_t = ((3 min(H / (32 ns), 8) + ns + 40) 2^-23 + 2^-20) ||x_t||_2 max_e ||w_e||_2
//             + (ns + 1) 2^-23 max_e |b_e|.
// At the synthetic workloads' scale err_t is about 1.2e-3, and the largest
// deviation from fp64 logits a few 1e-6; inputs with outlier channels raise
// err_t with ||x_t||.
#include "internal.h"

#include <cfloat>
#include <climits>

namespace strata_moe {

namespace {

// The router's fp32 accumulator chains end after this many k blocks (3 MFMAs
// each) and go into fp64 sums.
constexpr int kRouterChain = 8;

// The near-tie window delta = 2 err_t, with 1% on top for the fp32 norms:
// tie_coeff(H, ns) ||x_t|| max_e ||w_e|| + tie_bias_coeff(ns) max_e |b_e|.
__device__ __forceinline__ float tie_coeff(int32_t H, int ns) {
    const int chain = H / 32 / ns < kRouterChain ? H / 32 / ns : kRouterChain;  // blocks per chain
    return 2.02f * ((3.0f * (float)chain + (float)ns + 40.0f) * 0x1p-23f + 0x1p-20f);
}
__device__ __forceinline__ float tie_bias_coeff(int ns) { return 2.02f * (float)(ns + 1) * 0x1p-23f; }

// ---------------------------------------------------------------- logits
// logits[T][E] = x[T][H] . wr[H][E] (+ bias) on the MFMA unit.  Each fp32
// operand is written as hi + lo fp16 (lo = fp16(v - hi), about 22 bits)
// after a power-of-two scaling that puts the row's (token's) or column's
// (expert's) largest magnitude in [2^14, 2^15); the product keeps
// hi*hi + hi*lo + lo*hi (three MFMAs, fp32 accumulation), which leaves an
// error of the order of an fp32 dot product's, and the scalings are undone
// exactly in the epilogue.

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split_hi_lo(float v, _Float16& hi, _Float16& lo) {
    asm volatile("" : "+v"(v));  // v stays the fp32 value (no fused multiply-convert)
    hi = (_Float16)v;
    lo = (_Float16)(v - (float)hi);
}

// 2^(ex - 15) for a row whose largest magnitude is m: m * 2^(15 - ex) lies in
// [2^14, 2^15).  1 for an all-zero row.
__device__ __forceinline__ float row_multiplier(float m) {
    if (!(m > 0.0f)) return 1.0f;
    int ex = 0;
    frexpf(m, &ex);
    ex = ex < -96 ? -96 : ex;
    return ldexpf(1.0f, ex - 15);
}

// xm[t] = row multiplier of x[t], xn[t] = its Euclidean norm (fp32; one
// wave per row).
__global__ void __launch_bounds__(256) row_scale_kernel(const float* __restrict__ x, int64_t T, int32_t H,
                                                        float* __restrict__ xm, float* __restrict__ xn) {
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    float m = 0.0f, q = 0.0f;
    for (int h = lane; h < H; h += 64) {
        const float v = x[t * H + h];
        m = fmaxf(m, fabsf(v));
        q = fmaf(v, v, q);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        m = fmaxf(m, __shfl_xor(m, o));
        q += __shfl_xor(q, o);
    }
    if (lane == 0) {
        xm[t] = row_multiplier(m);
        xn[t] = sqrtf(q);
    }
}

// From wt [E][H] (the transposed router weight) and the column maxima of its
// 32-row tiles pmax [H/32][E]: wb, the hi/lo fp16 form of wt * 2^-ew in MFMA
// fragment order, and wm[e] = 2^ew (one wave per expert; padding experts up
// to a multiple of 16 get zeros and wm = 1).  Fragment order: per 16-expert
// tile and 32-wide k block, the hi fragment then the lo fragment, each 64
// lanes x 8 values with lane r + 16 g holding expert r of the tile, values
// 8g..8g+7 of the block; so a wave reads a fragment as 1 KB in one load.
// Also the largest Euclidean norm of a column, into *wnorm (zeroed before;
// non-negative floats order like their bit patterns, so an integer maximum).
__global__ void __launch_bounds__(256) router_prep_kernel(const float* __restrict__ wt,
                                                          const float* __restrict__ pmax, int32_t H, int32_t E,
                                                          int32_t Ep, _Float16* __restrict__ wb,
                                                          float* __restrict__ wm, float* __restrict__ wnorm) {
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= Ep) return;
    const int lane = threadIdx.x & 63;
    const int nk = H / 32;
    float m = 0.0f;
    if (e < E)
        for (int i = lane; i < H / 32; i += 64) m = fmaxf(m, pmax[(int64_t)i * E + e]);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float mult = row_multiplier(m), inv = 1.0f / mult;  // exact: powers of two
    if (lane == 0) wm[e] = mult;
    const float4* row = reinterpret_cast<const float4*>(wt + (int64_t)(e < E ? e : 0) * H);
    _Float16* tile = wb + (int64_t)(e >> 4) * nk * 1024;
    float q = 0.0f;
    for (int j0 = 0; j0 < H / 8; j0 += 256) {  // 4 groups of 8 values per lane in flight
        float4 v[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + 64 * u + lane;
            v[u][0] = v[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < H / 8 && e < E) {
                v[u][0] = row[2 * j];
                v[u][1] = row[2 * j + 1];
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int j = j0 + 64 * u + lane;  // value group j: block j / 4, group j % 4
            if (j >= H / 8) continue;
            const float f[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w, v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
            half8_t hi, lo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                _Float16 h, l;
                split_hi_lo(f[i] * inv, h, l);
                hi[i] = h;
                lo[i] = l;
                q = fmaf(f[i], f[i], q);
            }
            half8_t* dst = reinterpret_cast<half8_t*>(tile + (int64_t)(j >> 2) * 1024) + (e & 15) + 16 * (j & 3);
            dst[0] = hi;
            dst[64] = lo;
        }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) q += __shfl_xor(q, o);
    if (lane == 0 && e < E) atomicMax(reinterpret_cast<int*>(wnorm), __builtin_bit_cast(int, sqrtf(q)));
}

// 64 tokens x 128 experts per workgroup; wave w takes experts 32w..32w+31 of
// the tile (two 16-wide MFMA columns) against all 64 tokens (four 16-row
// tiles).  Per 32-wide k block: the workgroup converts its 64 x 32 input
// block to hi/lo fp16 into LDS (each thread 8 values), one barrier, then each
// wave reads the 4 x 2 A fragments and runs 4 x 2 x 3 MFMAs.  Input values
// and B fragments (1 KB loads in fragment order) are loaded two k blocks
// ahead.  The fp32 accumulators are added into fp64 sums every kRouterChain
// k blocks (see the error bound above).  Workgroup z of gridDim.z takes the
// z-th of gridDim.z equal ranges of k blocks (each of even length) and writes
// its partial logits to slice z (the bias goes into slice 0).
constexpr int kRtM = 64, kRtN = 128;

struct RouterStage {
    float4 x0, x1;          // this thread's 8 input values of one k block
    half8_t b[2][2];        // [expert tile][hi, lo]
};

__global__ void __launch_bounds__(256, 2) router_mfma_kernel(const float* __restrict__ x,
                                                             const float* __restrict__ xm,
                                                             const _Float16* __restrict__ wb,
                                                             const float* __restrict__ wm,
                                                             const float* __restrict__ bias, int64_t T, int32_t H,
                                                             int32_t E, int32_t Ep, float* __restrict__ out) {
    __shared__ half8_t a_lds[2][4][2][64];  // [buffer][token tile][hi, lo][lane]
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, kg = lane >> 4;
    // XCD-aware order: the dispatcher deals consecutive workgroups to the 8
    // XCDs in turn, so within each run of 8 token tiles the gx expert tiles
    // of one token tile take ids 8 apart and share an XCD: the tile's input
    // rows come from HBM once and from that XCD's L2 after (a last partial
    // run keeps the plain order)
    const int gx = gridDim.x, gy = gridDim.y;
    const int lin = blockIdx.y * gx + blockIdx.x, grp = lin / (8 * gx), rr = lin % (8 * gx);
    const bool full = gy - 8 * grp >= 8;
    const int bx = full ? rr / 8 : rr % gx, by = full ? 8 * grp + rr % 8 : 8 * grp + rr / gx;
    const int n0 = bx * kRtN;
    const int64_t m0 = (int64_t)by * kRtM;
    const int nk = H / 32, kper = nk / gridDim.z, kb0 = blockIdx.z * kper, kb1 = kb0 + kper;

    // staging role: token row sr of the tile, value group sk (8 values) of the k block
    const int sr = tid >> 2, sk = tid & 3;
    const bool srow_ok = m0 + sr < T;
    const float sinv = srow_ok ? 1.0f / xm[m0 + sr] : 0.0f;  // exact: a power of two
    const float* xs = x + (srow_ok ? m0 + sr : 0) * (int64_t)H + 8 * sk;
    const int slane = sk * 16 + (sr & 15), stile = sr >> 4;

    // B role: expert tiles et = 0, 1 of this wave; tiles past the padded
    // experts read the last tile (never stored)
    const half8_t* wbp[2];
#pragma unroll
    for (int et = 0; et < 2; ++et) {
        int te = (n0 >> 4) + 2 * wave + et;
        te = te < Ep / 16 ? te : Ep / 16 - 1;
        wbp[et] = reinterpret_cast<const half8_t*>(wb + (int64_t)te * nk * 1024) + lane;
    }

    auto load = [&](int kb, RouterStage& S) {
        kb = kb < kb1 ? kb : kb1 - 1;
        S.x0 = *reinterpret_cast<const float4*>(xs + 32 * kb);
        S.x1 = *reinterpret_cast<const float4*>(xs + 32 * kb + 4);
#pragma unroll
        for (int et = 0; et < 2; ++et) {
            S.b[et][0] = wbp[et][128 * kb];
            S.b[et][1] = wbp[et][128 * kb + 64];
        }
    };
    auto stage = [&](int kb, const RouterStage& S) {
        const float v[8] = {S.x0.x, S.x0.y, S.x0.z, S.x0.w, S.x1.x, S.x1.y, S.x1.z, S.x1.w};
        half8_t hi, lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            _Float16 h, l;
            split_hi_lo(v[i] * sinv, h, l);
            hi[i] = h;
            lo[i] = l;
        }
        a_lds[kb & 1][stile][0][slane] = hi;
        a_lds[kb & 1][stile][1][slane] = lo;
    };
    // fp32 accumulator chains of at most kRouterChain blocks, each added into
    // an fp64 sum when it ends.  The k loop runs in kRouterChain-block steps
    // of four block pairs; after pair i the accumulators of token tile i end
    // their chains (so each pair adds two of the eight while the others'
    // MFMAs run).  A shorter rest of the range starts fresh chains.
    static_assert(kRouterChain == 8, "four block pairs per step, one token tile's chains ending after each");
    float4_t acc[4][2];
    double dacc[4][2][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int et = 0; et < 2; ++et) {
            acc[mt][et] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int v = 0; v < 4; ++v) dacc[mt][et][v] = 0.0;
        }
    auto end_chain = [&](int mt, int et) {
#pragma unroll
        for (int v = 0; v < 4; ++v) dacc[mt][et][v] += (double)acc[mt][et][v];
        acc[mt][et] = (float4_t){0.f, 0.f, 0.f, 0.f};
    };
    auto products = [&](int kb, const RouterStage& S) {
        half8_t a[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            a[mt][0] = a_lds[kb & 1][mt][0][lane];
            a[mt][1] = a_lds[kb & 1][mt][1][lane];
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int et = 0; et < 2; ++et) {
                acc[mt][et] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][0], S.b[et][0], acc[mt][et], 0, 0, 0);
                acc[mt][et] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][0], S.b[et][1], acc[mt][et], 0, 0, 0);
                acc[mt][et] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[mt][1], S.b[et][0], acc[mt][et], 0, 0, 0);
            }
    };

    RouterStage s0, s1;
    auto pair = [&](int kb) {  // blocks kb and kb + 1
        stage(kb, s0);
        __syncthreads();
        products(kb, s0);
        load(kb + 2, s0);
        stage(kb + 1, s1);
        __syncthreads();
        products(kb + 1, s1);
        load(kb + 3, s1);
    };
    auto end_all = [&]() {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int et = 0; et < 2; ++et) end_chain(mt, et);
    };
    load(kb0, s0);
    load(kb0 + 1, s1);
    int kb = kb0;
    for (; kb + kRouterChain <= kb1; kb += kRouterChain) {
#pragma unroll
        for (int i = 0; i < kRouterChain / 2; ++i) {
            pair(kb + 2 * i);
            end_chain(i, 0);
            end_chain(i, 1);
            // one pair at a time: letting later pairs' loads move up took 244 VGPRs
            // against 186 (2 workgroups per CU either way; 365 vs 340 us at 32768 tokens)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    if (kb < kb1) {  // uniform: the rest of the range, fewer than kRouterChain blocks
        end_all();
        for (; kb < kb1; kb += 2) pair(kb);
    }
    end_all();  // the last chains

    float* part = out + (int64_t)blockIdx.z * T * E;
#pragma unroll
    for (int et = 0; et < 2; ++et) {
        const int e = n0 + 32 * wave + 16 * et + r16;
        if (e >= E) continue;
        const float we = wm[e], be = bias && blockIdx.z == 0 ? bias[e] : 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t t = m0 + 16 * mt + 4 * kg + v;
                // the multipliers are powers of two: one rounding, to fp32
                if (t < T) part[t * E + e] = (float)(dacc[mt][et][v] * (double)xm[t] * (double)we + (double)be);
            }
    }
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int32_t count, int32_t value) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = value;
}

// wt[E][H] = wr[H][E] (the re-score reads one expert's weights as a
// contiguous row), 32x32 tiles through LDS; and pmax[tile row][e] = the
// largest |wr| of expert e in the tile's 32 rows.
__global__ void __launch_bounds__(256) transpose_kernel(const float* __restrict__ in, int32_t R, int32_t C,
                                                        float* __restrict__ out, float* __restrict__ pmax) {
    __shared__ float tile[32][33];
    const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
#pragma unroll
    for (int k = 0; k < 32; k += 8)
        if (r0 + ty + k < R && c0 + tx < C) tile[ty + k][tx] = in[(int64_t)(r0 + ty + k) * C + c0 + tx];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 32; k += 8)
        if (c0 + ty + k < C && r0 + tx < R) out[(int64_t)(c0 + ty + k) * R + r0 + tx] = tile[tx][ty + k];
    if (ty == 0 && c0 + tx < C) {
        float m = 0.0f;
        for (int r = 0; r < 32 && r0 + r < R; ++r) m = fmaxf(m, fabsf(tile[r][tx]));
        pmax[(int64_t)blockIdx.y * C + c0 + tx] = m;
    }
}

// ------------------------------------------------------------------ top-K
constexpr int kPerLane = kMaxExperts / 64;

__device__ __forceinline__ bool better(float v, int e, float bv, int be) { return v > bv || (v == bv && e < be); }
__device__ __forceinline__ bool better_d(double v, int e, double bv, int be) {
    return v > bv || (v == bv && e < be);
}

// Wave-wide best (largest value, then lowest index) in every lane, on the
// vector ALU: quad exchanges (lane ^ 1, lane ^ 2), the mirror within each 8
// and within each 16 lanes (DPP), then the 16-lane and 32-lane row swaps.
// After each step a lane holds the best of twice as many lanes.
template <int kCtrl>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}

template <typename V>
struct Best {
    V v;
    int i;
};

__device__ __forceinline__ void take_better(Best<float>& a, float v, int i) {
    if (better(v, i, a.v, a.i)) a.v = v, a.i = i;
}
__device__ __forceinline__ void take_better(Best<double>& a, double v, int i) {
    if (better_d(v, i, a.v, a.i)) a.v = v, a.i = i;
}

template <int kCtrl>
__device__ __forceinline__ void best_step(Best<float>& a) {
    const float v = __builtin_bit_cast(float, dpp<kCtrl>(__builtin_bit_cast(int, a.v)));
    const int i = dpp<kCtrl>(a.i);
    take_better(a, v, i);
}
template <int kCtrl>
__device__ __forceinline__ void best_step(Best<double>& a) {
    const uint64_t u = __builtin_bit_cast(uint64_t, a.v);
    const uint32_t lo = (uint32_t)dpp<kCtrl>((int)(uint32_t)u), hi = (uint32_t)dpp<kCtrl>((int)(uint32_t)(u >> 32));
    const int i = dpp<kCtrl>(a.i);
    take_better(a, __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo), i);
}

// Each swap returns the row pair's two halves in two registers: lane l holds
// one of them in each, so one comparison combines the pair.
__device__ __forceinline__ uint32_t pair_first(uint32_t a, uint32_t b, bool wide, uint32_t* second) {
    if (wide) {
        const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
        *second = r[1];
        return r[0];
    }
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    *second = r[1];
    return r[0];
}

__device__ __forceinline__ void best_swap(Best<float>& a, bool wide) {
    uint32_t v1, i1;
    const uint32_t v0 = pair_first(__builtin_bit_cast(uint32_t, a.v), __builtin_bit_cast(uint32_t, a.v), wide, &v1);
    const uint32_t i0 = pair_first((uint32_t)a.i, (uint32_t)a.i, wide, &i1);
    a.v = __builtin_bit_cast(float, v0);
    a.i = (int)i0;
    take_better(a, __builtin_bit_cast(float, v1), (int)i1);
}
__device__ __forceinline__ void best_swap(Best<double>& a, bool wide) {
    const uint64_t u = __builtin_bit_cast(uint64_t, a.v);
    uint32_t lo1, hi1, i1;
    const uint32_t lo0 = pair_first((uint32_t)u, (uint32_t)u, wide, &lo1);
    const uint32_t hi0 = pair_first((uint32_t)(u >> 32), (uint32_t)(u >> 32), wide, &hi1);
    const uint32_t i0 = pair_first((uint32_t)a.i, (uint32_t)a.i, wide, &i1);
    a.v = __builtin_bit_cast(double, ((uint64_t)hi0 << 32) | lo0);
    a.i = (int)i0;
    take_better(a, __builtin_bit_cast(double, ((uint64_t)hi1 << 32) | lo1), (int)i1);
}

// Wave-wide fp64 sum in every lane, by the same exchange steps (fp addition
// is commutative, so the lanes of a pair compute the same value and every
// lane ends with the same sum).
template <int kCtrl>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)dpp<kCtrl>((int)(uint32_t)u), hi = (uint32_t)dpp<kCtrl>((int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double swap_add(double v, bool wide) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    uint32_t lo1, hi1;
    const uint32_t lo0 = pair_first((uint32_t)u, (uint32_t)u, wide, &lo1);
    const uint32_t hi0 = pair_first((uint32_t)(u >> 32), (uint32_t)(u >> 32), wide, &hi1);
    return __builtin_bit_cast(double, ((uint64_t)hi0 << 32) | lo0) +
           __builtin_bit_cast(double, ((uint64_t)hi1 << 32) | lo1);
}
__device__ __forceinline__ double wave_sum(double v) {
    v += dpp_d<0xB1>(v);
    v += dpp_d<0x4E>(v);
    v += dpp_d<0x141>(v);
    v += dpp_d<0x140>(v);
    v = swap_add(v, false);
    return swap_add(v, true);
}

template <typename V>
__device__ __forceinline__ Best<V> wave_best(Best<V> a) {
    best_step<0xB1>(a);   // quad_perm [1,0,3,2]: lane ^ 1
    best_step<0x4E>(a);   // quad_perm [2,3,0,1]: lane ^ 2
    best_step<0x141>(a);  // mirror within 8 lanes: the other quad
    best_step<0x140>(a);  // mirror within 16 lanes: the other 8
    best_swap(a, false);  // rows 0/1 and 2/3
    best_swap(a, true);   // halves 0-31 / 32-63
    return a;
}

// The wave-wide selection of one token (every lane ends with the same
// results): lane l holds logits l, l+64, ... in v; selv/seli get ranks
// 0..rounds-1 (K+1 rounds, K when K == E) by larger value, then lower index;
// `loose` has bit k (k < K) set when rank k is within delta of a neighbouring
// rank, i.e. its exact order is in doubt.
template <int kSlots>
struct Selection {
    float v[kSlots];  // lane l: logits of experts l, l + 64, ...
    float selv[kMaxTopK + 1];
    int seli[kMaxTopK + 1];
    int rounds;
    float vK, delta;
    uint32_t loose;
};

// The 19-comparator sorting network for 8 values (descending by value, then
// ascending index), applied to one lane's values.
__device__ __forceinline__ void cas(float (&v)[8], int (&e)[8], int a, int b) {
    if (better(v[b], e[b], v[a], e[a])) {
        const float tv = v[a];
        const int te = e[a];
        v[a] = v[b], e[a] = e[b];
        v[b] = tv, e[b] = te;
    }
}
__device__ __forceinline__ void sort8(float (&v)[8], int (&e)[8]) {
    cas(v, e, 0, 2), cas(v, e, 1, 3), cas(v, e, 4, 6), cas(v, e, 5, 7);
    cas(v, e, 0, 4), cas(v, e, 1, 5), cas(v, e, 2, 6), cas(v, e, 3, 7);
    cas(v, e, 0, 1), cas(v, e, 2, 3), cas(v, e, 4, 5), cas(v, e, 6, 7);
    cas(v, e, 2, 4), cas(v, e, 3, 5);
    cas(v, e, 1, 4), cas(v, e, 3, 6);
    cas(v, e, 1, 2), cas(v, e, 3, 4), cas(v, e, 5, 6);
}

// l: the token's row of the first partial logits slice; nsplit slices
// `sstride` floats apart are added in order.  kSlots = 8 needs E <= 512.
template <int kSlots>
__device__ __forceinline__ void load_logits(const float* __restrict__ l, int nsplit, int64_t sstride, int32_t E,
                                            int lane, Selection<kSlots>& S) {
    // all loads first (the slices are independent), then the sums in slice order
    float part[kMaxRouterSplits][kSlots];
#pragma unroll
    for (int z = 0; z < kMaxRouterSplits; ++z)
        if (z < nsplit)  // uniform
#pragma unroll
            for (int i = 0; i < kSlots; ++i) {
                const int e = lane + 64 * i;
                part[z][i] = e < E ? l[z * sstride + e] : 0.0f;
            }
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        float v = part[0][i];
#pragma unroll
        for (int z = 1; z < kMaxRouterSplits; ++z)
            if (z < nsplit) v += part[z][i];
        S.v[i] = lane + 64 * i < E ? v : -FLT_MAX;
    }
}

template <int kSlots>
__device__ __forceinline__ void select_token(const float* __restrict__ l, int nsplit, int64_t sstride, int32_t E,
                                             int32_t K, float delta, int lane, Selection<kSlots>& S) {
    load_logits(l, nsplit, sstride, E, lane, S);
    S.rounds = K < E ? K + 1 : K;
#pragma unroll
    for (int k = 0; k <= kMaxTopK; ++k) S.selv[k] = -FLT_MAX, S.seli[k] = INT_MAX;
    if constexpr (kSlots == 8) {
        // each lane sorts its 8 values once; a round offers every lane's head,
        // and the winning lane moves its list up by one
        float hv[8];
        int he[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) hv[i] = S.v[i], he[i] = lane + 64 * i < E ? lane + 64 * i : INT_MAX;
        sort8(hv, he);
#pragma unroll
        for (int k = 0; k <= kMaxTopK; ++k) {
            if (k >= S.rounds) continue;
            Best<float> b{hv[0], he[0]};
            b = wave_best(b);
            S.selv[k] = b.v;
            S.seli[k] = b.i;
            const bool win = he[0] == b.i;
#pragma unroll
            for (int i = 0; i < 7; ++i) {
                hv[i] = win ? hv[i + 1] : hv[i];
                he[i] = win ? he[i + 1] : he[i];
            }
            hv[7] = win ? -FLT_MAX : hv[7];
            he[7] = win ? INT_MAX : he[7];
        }
    } else {
        uint32_t taken = 0;
#pragma unroll
        for (int k = 0; k <= kMaxTopK; ++k) {
            if (k >= S.rounds) continue;
            Best<float> b{-FLT_MAX, INT_MAX};
#pragma unroll
            for (int i = 0; i < kSlots; ++i) {
                const int e = lane + 64 * i;
                if (e < E && !((taken >> i) & 1u)) take_better(b, S.v[i], e);
            }
            b = wave_best(b);
            const int bi = b.i;
            S.selv[k] = b.v;
            S.seli[k] = bi;
            if (bi < E && (bi & 63) == lane) taken |= 1u << (bi >> 6);
        }
    }
    S.vK = -FLT_MAX;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k == K - 1) S.vK = S.selv[k];
    S.delta = delta;
    S.loose = 0;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        const bool up = k > 0 && k < S.rounds && S.selv[k - 1] - S.selv[k] < S.delta;
        const bool dn = k + 1 < S.rounds && S.selv[k] - S.selv[k + 1] < S.delta;
        if (k < K && (up || dn)) S.loose |= 1u << k;
    }
}

// Wave-wide fp32 sum in every lane (the exchange steps of wave_best).
__device__ __forceinline__ float wave_sum_f(float v) {
    v += __builtin_bit_cast(float, dpp<0xB1>(__builtin_bit_cast(int, v)));
    v += __builtin_bit_cast(float, dpp<0x4E>(__builtin_bit_cast(int, v)));
    v += __builtin_bit_cast(float, dpp<0x141>(__builtin_bit_cast(int, v)));
    v += __builtin_bit_cast(float, dpp<0x140>(__builtin_bit_cast(int, v)));
    uint32_t b;
    float a = __builtin_bit_cast(float, pair_first(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v),
                                                   false, &b));
    v = a + __builtin_bit_cast(float, b);
    a = __builtin_bit_cast(float, pair_first(__builtin_bit_cast(uint32_t, v), __builtin_bit_cast(uint32_t, v), true,
                                             &b));
    return a + __builtin_bit_cast(float, b);
}

// ids / p of one token from its ranked values: the softmax over the K, in
// fp32 (values relative to the largest, each term in (0, 1]); lane k < K
// takes rank k.
template <typename V>
__device__ __forceinline__ void write_token(const V (&lv)[kMaxTopK], const int (&li)[kMaxTopK], int32_t K, int lane,
                                            int64_t t, int32_t* __restrict__ ids, float* __restrict__ p_out) {
    V mine = lv[0];
    int mi = li[0];
    // a chain of selects; the empty asm keeps the compiler from turning it
    // into a table in scratch memory indexed by the lane
#pragma unroll
    for (int k = 1; k < kMaxTopK; ++k) {
        const bool me = lane == k;
        mine = me ? lv[k] : mine;
        mi = me ? li[k] : mi;
        asm volatile("" : "+v"(mine), "+v"(mi));
    }
    const float ev = lane < K ? expf((float)(mine - lv[0])) : 0.0f;
    const float z = wave_sum_f(ev);
    if (lane < K) {
        ids[t * K + lane] = mi;
        p_out[t * K + lane] = ev / z;
    }
}

// The fp64 dot product x[0..H) . w[0..H) over one wave (every lane ends with
// the same sum).  Lane l takes 4 consecutive elements of every 256, up to
// kDotBatch such groups of loads in flight at once; a tail of H % 256
// elements goes one per lane.
constexpr int kDotBatch = 5;  // 10 measured 48 vs 37 us at 8192 tokens: 187 VGPRs, 2 waves per SIMD
__device__ __forceinline__ double wave_dot_fp64(const float* __restrict__ x, const float* __restrict__ w, int32_t H,
                                                int lane) {
    double acc = 0.0;
    const int n4 = H / 256;
    for (int c0 = 0; c0 < n4; c0 += kDotBatch) {
        float4 xv[kDotBatch], wv[kDotBatch];
#pragma unroll
        for (int j = 0; j < kDotBatch; ++j)
            if (c0 + j < n4) {
                xv[j] = reinterpret_cast<const float4*>(x)[64 * (c0 + j) + lane];
                wv[j] = reinterpret_cast<const float4*>(w)[64 * (c0 + j) + lane];
            }
#pragma unroll
        for (int j = 0; j < kDotBatch; ++j)
            if (c0 + j < n4) {
                acc = fma((double)xv[j].x, (double)wv[j].x, acc);
                acc = fma((double)xv[j].y, (double)wv[j].y, acc);
                acc = fma((double)xv[j].z, (double)wv[j].z, acc);
                acc = fma((double)xv[j].w, (double)wv[j].w, acc);
            }
    }
    for (int h = 256 * n4 + lane; h < H; h += 64) acc = fma((double)x[h], (double)w[h], acc);
    return wave_sum(acc);
}

// Two such dot products, x . w1 and x . w2, with the loads of both in flight
// together; each sum is formed in the same order as wave_dot_fp64's.
__device__ __forceinline__ void wave_dot2_fp64(const float* __restrict__ x, const float* __restrict__ w1,
                                               const float* __restrict__ w2, int32_t H, int lane, double& v1,
                                               double& v2) {
    double a1 = 0.0, a2 = 0.0;
    const int n4 = H / 256;
    for (int c0 = 0; c0 < n4; c0 += kDotBatch) {
        float4 xv[kDotBatch], p[kDotBatch], q[kDotBatch];
#pragma unroll
        for (int j = 0; j < kDotBatch; ++j)
            if (c0 + j < n4) {
                xv[j] = reinterpret_cast<const float4*>(x)[64 * (c0 + j) + lane];
                p[j] = reinterpret_cast<const float4*>(w1)[64 * (c0 + j) + lane];
                q[j] = reinterpret_cast<const float4*>(w2)[64 * (c0 + j) + lane];
            }
#pragma unroll
        for (int j = 0; j < kDotBatch; ++j)
            if (c0 + j < n4) {
                a1 = fma((double)xv[j].x, (double)p[j].x, a1);
                a1 = fma((double)xv[j].y, (double)p[j].y, a1);
                a1 = fma((double)xv[j].z, (double)p[j].z, a1);
                a1 = fma((double)xv[j].w, (double)p[j].w, a1);
                a2 = fma((double)xv[j].x, (double)q[j].x, a2);
                a2 = fma((double)xv[j].y, (double)q[j].y, a2);
                a2 = fma((double)xv[j].z, (double)q[j].z, a2);
                a2 = fma((double)xv[j].w, (double)q[j].w, a2);
            }
    }
    for (int h = 256 * n4 + lane; h < H; h += 64) {
        a1 = fma((double)x[h], (double)w1[h], a1);
        a2 = fma((double)x[h], (double)w2[h], a2);
    }
    v1 = wave_sum(a1);
    v2 = wave_sum(a2);
}

// One top-K pass per token, in fp32 first: the ranking of the token's
// summed logits and the near-tie window.  A token whose ranks are all
// further apart than the window is finished at once.  Otherwise every
// expert within the window below the K-th value (this includes all K
// selected) is a candidate; selected ranks outside every near-tie keep their
// fp32 value (each is at least the window away from any value that is
// re-scored, so the merged order is the exact one), and the others are
// re-scored as wave-wide fp64 dot products of the input row and the
// expert's weight column, two at a time.  Lane l keeps the candidates among
// experts l, l + 64, ... in registers.
// kWide (calls of up to kSelectShort tokens): a workgroup of 4 waves per
// token; every wave ranks the token (the same bits), the waves take every
// fourth pair of the re-score list, the values meet in LDS and wave 0
// re-ranks: a short prompt waits for one token's latency.  Otherwise a wave
// per token, kSelectWaves tokens per workgroup, each wave re-scoring its own
// token's list.  Each value comes from the same dot-product routine
// whichever wave computes it.
constexpr int kWaves = 4;
constexpr int kSelectShort = 1024;  // wide up to here: 29 vs 33 us at 1024 tokens, 102 vs 67 at 8192
// The narrow form held to 5 waves per SIMD (96 VGPRs; the compiler spills a
// few of the re-score's registers): 42 vs 43 us at 8192 tokens, 102 vs 111 at
// 32768 (6 waves: 47 and 107).
template <int kSlots, int kSelectWaves, bool kWide>
__global__ void __launch_bounds__(64 * kSelectWaves, kWide ? 1 : 5) topk_kernel(const float* __restrict__ logits, int nsplit,
                                                                int64_t T, const float* __restrict__ x,
                                                                const float* __restrict__ wt,
                                                                const float* __restrict__ bias, int32_t H, int32_t E,
                                                                int32_t K, const float* __restrict__ xn,
                                                                const float* __restrict__ wnorm,
                                                                int32_t* __restrict__ ids, float* __restrict__ p_out) {
    static_assert(!kWide || kSelectWaves == kWaves, "a workgroup of kWaves waves per token");
    __shared__ double rescored[kWide ? kMaxExperts : 1];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t t = kWide ? (int64_t)blockIdx.x : (int64_t)blockIdx.x * kSelectWaves + wave;
    if (t >= T) return;  // kWide: uniform over the workgroup; otherwise no barrier follows
    Selection<kSlots> S;
    // the largest |b_e| (the bias's share of the error bound)
    float bm = 0.0f;
    if (bias) {
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            if (lane + 64 * i < E) bm = fmaxf(bm, fabsf(bias[lane + 64 * i]));
        for (int o = 1; o < 64; o <<= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
    }
    const float delta = tie_coeff(H, nsplit) * xn[t] * *wnorm + tie_bias_coeff(nsplit) * bm;
    select_token(logits + t * E, nsplit, T * E, E, K, delta, lane, S);
    if (!S.loose) {  // kWide: the same for every wave of the workgroup
        if (!kWide || wave == 0) {
            float lv[kMaxTopK];
            int li[kMaxTopK];
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) lv[k] = S.selv[k], li[k] = S.seli[k];
            write_token(lv, li, K, lane, t, ids, p_out);
        }
        return;
    }
    const float thr = S.vK - S.delta;
    double cv[kSlots];
    uint32_t cand = 0, todo = 0;
#pragma unroll
    for (int i = 0; i < kSlots; ++i) {
        const int e = lane + 64 * i;
        const bool c = e < E && S.v[i] >= thr;
        bool stable = false;
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k)
            if (k < K && !((S.loose >> k) & 1u) && S.seli[k] == e) stable = true;
        cv[i] = (double)S.v[i];
        cand |= (uint32_t)c << i;
        todo |= (uint32_t)(c && !stable) << i;
    }
    const float* xr = x + t * H;
    // the experts to re-score in list order, two per pair; with a workgroup
    // per token this wave takes pairs wave, wave + 4, ...
    uint64_t m[kSlots];
#pragma unroll
    for (int i = 0; i < kSlots; ++i) m[i] = __ballot((todo >> i) & 1u);
    for (int pair = 0;; ++pair) {
        int e1 = -1, e2 = -1;
#pragma unroll
        for (int i = 0; i < kSlots; ++i) {
            if (e1 < 0 && m[i]) {
                e1 = (__ffsll((unsigned long long)m[i]) - 1) + 64 * i;
                m[i] &= m[i] - 1ull;
            }
            if (e1 >= 0 && e2 < 0 && m[i]) {
                e2 = (__ffsll((unsigned long long)m[i]) - 1) + 64 * i;
                m[i] &= m[i] - 1ull;
            }
        }
        if (e1 < 0) break;
        if (kWide && (pair & (kWaves - 1)) != wave) continue;
        double v1, v2 = 0.0;
        if (e2 >= 0)
            wave_dot2_fp64(xr, wt + (int64_t)e1 * H, wt + (int64_t)e2 * H, H, lane, v1, v2);
        else
            v1 = wave_dot_fp64(xr, wt + (int64_t)e1 * H, H, lane);
        if (bias) {
            v1 += (double)bias[e1];
            if (e2 >= 0) v2 += (double)bias[e2];
        }
        if (kWide) {
            if (lane == 0) {
                rescored[e1] = v1;
                if (e2 >= 0) rescored[e2] = v2;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kSlots; ++i) {
                const int e = lane + 64 * i;
                cv[i] = e == e1 ? v1 : e == e2 ? v2 : cv[i];
            }
        }
    }
    if (kWide) {
        __syncthreads();
        if (wave != 0) return;
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            if ((todo >> i) & 1u) cv[i] = rescored[lane + 64 * i];
    }
    double lv[kMaxTopK];
    int li[kMaxTopK];
    uint32_t tk = 0;
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k) {
        lv[k] = -DBL_MAX;
        li[k] = INT_MAX;
        if (k >= K) continue;
        Best<double> b{-DBL_MAX, INT_MAX};
#pragma unroll
        for (int i = 0; i < kSlots; ++i)
            if (((cand & ~tk) >> i) & 1u) take_better(b, cv[i], lane + 64 * i);
        b = wave_best(b);
        const int bi = b.i;
        lv[k] = b.v;
        li[k] = bi;
        if (bi < E && (bi & 63) == lane) tk |= 1u << (bi >> 6);
    }
    write_token(lv, li, K, lane, t, ids, p_out);
}

}  // namespace

hipError_t launch_router_prep(const float* wr, int32_t H, int32_t E, const RouterScratch& rs, hipStream_t st) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, reinterpret_cast<int32_t*>(rs.wnorm), 1, 0);
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((E + 31) / 32), (unsigned)((H + 31) / 32)), dim3(256), 0, st,
                       wr, H, E, rs.wt, rs.pmax);
    const int32_t Ep = (int32_t)router_padded_experts(E);
    hipLaunchKernelGGL(router_prep_kernel, dim3((unsigned)((Ep + 3) / 4)), dim3(256), 0, st, rs.wt, rs.pmax, H, E, Ep,
                       rs.wb, rs.wm, rs.wnorm);
    return hipGetLastError();
}

hipError_t launch_router(const float* x, const float* xm, const float* wr, const float* bias, int64_t T, int32_t H,
                         int32_t E, const RouterScratch& rs, float* logits, hipStream_t st) {
    if (T <= 0) return hipGetLastError();
    if (wr) {
        const hipError_t e = launch_router_prep(wr, H, E, rs, st);
        if (e != hipSuccess) return e;
    }
    const int32_t Ep = (int32_t)router_padded_experts(E);
    if (!xm) {  // the input rows' multipliers and norms
        hipLaunchKernelGGL(row_scale_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, x, T, H, rs.xm, rs.xn);
        xm = rs.xm;
    }
    hipLaunchKernelGGL(router_mfma_kernel,
                       dim3((unsigned)((E + kRtN - 1) / kRtN), (unsigned)((T + kRtM - 1) / kRtM),
                            (unsigned)router_splits(T, H, E)),
                       dim3(256), 0, st, x, xm, rs.wb, rs.wm, bias, T, H, E, Ep, logits);
    return hipGetLastError();
}

hipError_t launch_topk(const float* logits, const float* x, const float* xn, const float* wt, const float* wnorm,
                       const float* bias, int64_t T, int32_t H, int32_t E, int32_t K, int32_t* ids, float* p,
                       hipStream_t st) {
    if (T > 0) {
        const int ns = router_splits(T, H, E);
        if (T <= kSelectShort) {  // a workgroup per token
            auto* k = E <= 512 ? topk_kernel<8, kWaves, true> : topk_kernel<kPerLane, kWaves, true>;
            hipLaunchKernelGGL(k, dim3((unsigned)T), dim3(64 * kWaves), 0, st, logits, ns, T, x, wt, bias, H, E, K,
                               xn, wnorm, ids, p);
        } else {  // a wave per token, 4 per workgroup (16 measured 72 vs 60 us at 8192 tokens)
            constexpr int kw = 4;
            auto* k = E <= 512 ? topk_kernel<8, kw, false> : topk_kernel<kPerLane, kw, false>;
            hipLaunchKernelGGL(k, dim3((unsigned)((T + kw - 1) / kw)), dim3(64 * kw), 0, st, logits, ns, T, x, wt,
                               bias, H, E, K, xn, wnorm, ids, p);
        }
    }
    return hipGetLastError();
}

// ------------------------------------------------------------ shared expert
// The shared expert joins the grouping as expert E, pair slot K of every
// token, its weight the token's scalar gate g = sigmoid(x . wg) (the shared
// expert and its scalar gate, MoE half of Prefill::run, prefill.cpp page).
// One wave per token: the dot in fp32 (lane-strided float4 partial sums, then
// a butterfly), the routed pairs copied to the K + 1 wide arrays beside it.
constexpr int kSharedWaves = 4;

__global__ void __launch_bounds__(64 * kSharedWaves)
    shared_slot_kernel(const float* __restrict__ x, const float* __restrict__ wg, const int32_t* __restrict__ ids,
                       const float* __restrict__ p, int64_t T, int32_t H, int32_t K, int32_t E,
                       int32_t* __restrict__ gids, float* __restrict__ gp) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * kSharedWaves + (threadIdx.x >> 6);
    if (t >= T) return;  // whole waves
    const float4_t* xr = reinterpret_cast<const float4_t*>(x + t * H);
    const float4_t* wr = reinterpret_cast<const float4_t*>(wg);
    float acc = 0.f;
    for (int c = lane; c < H / 4; c += 64) {
        const float4_t a = xr[c], w = wr[c];
        acc = fmaf(a[0], w[0], acc);
        acc = fmaf(a[1], w[1], acc);
        acc = fmaf(a[2], w[2], acc);
        acc = fmaf(a[3], w[3], acc);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    const float g = 1.0f / (1.0f + expf(-acc));
    const int32_t Kg = K + 1;
    if (lane < K) {
        gids[t * Kg + lane] = ids[t * K + lane];
        gp[t * Kg + lane] = p[t * K + lane];
    } else if (lane == K) {
        gids[t * Kg + K] = E;
        gp[t * Kg + K] = g;
    }
}

hipError_t launch_shared_slot(const float* x, const float* wg, const int32_t* ids, const float* p, int64_t T,
                              int32_t H, int32_t K, int32_t E, int32_t* gids, float* gp, hipStream_t st) {
    if (T > 0)
        hipLaunchKernelGGL(shared_slot_kernel, dim3((unsigned)((T + kSharedWaves - 1) / kSharedWaves)),
                           dim3(64 * kSharedWaves), 0, st, x, wg, ids, p, T, H, K, E, gids, gp);
    return hipGetLastError();
}

}  // namespace strata_moe
