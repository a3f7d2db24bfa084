/*
 * strata_oracle.c -- CPU oracle of the routed-expert prompt MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, double-precision reference
 * used by the tests, the smoke check and the benchmark's CPU-baseline leg to
 * check the HIP library.  The product path never links, loads or calls it, and
 * it shares no code, header, table or helper with that library.
 *
 * What it computes, and where the pages say so:
 *   [prefill.cpp]  Winery-Strata, src/prefill/prefill.cpp, Prefill::run, the
 *                  MoE half: the router projection of the layer input, route()
 *                  to ids/weights, and (MMQ path) the host counting sort that
 *                  groups the (token, k) pairs by expert into slot/src.
 *   [moe_fused]    Strata compare v0.1.35...v0.1.37, file
 *                  include/strata/prefill/moe_fused.hpp: activations rounded to
 *                  int8 once per token with one scale per 32 values; gate/up
 *                  on the grouped rows; SwiGLU; H rounded to int8 (per 32) in
 *                  the epilogue; down into per-slot rows; a combine that reads
 *                  those rows.
 * Readings where the pages leave a step open are stated at each step; the
 * 2-bit weight map is the symmetric one, w = d*(q - 1.5)
 * with an fp16 d per 32 codes along the reduction dimension (the pages' own
 * Q2_0 pack uses w = d*(q - 1), moe_fused.hpp header comment).
 *
 * Every function is a direct transcription of the definition; loops run in
 * the obvious order and nothing is blocked, fused or reordered.  OpenMP only
 * splits independent rows across threads.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define QBLOCK 32

/* IEEE binary16 bit pattern -> exact double value (plain decoding of the
 * format: sign, 5-bit biased exponent, 10-bit fraction). */
static double half_bits_to_double(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24); /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    return sign ? -v : v;
}

double oracle_half_to_double(uint16_t h) { return half_bits_to_double(h); }

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- c1 router
 * [prefill.cpp] the router projection: logits[t][e] = x[t] . W_r[:, e].
 * Reading: the logits are the real dot product of the fp32 inputs (the pages
 * run it as a BF16 GEMM); each product of two fp32 values is exact in double,
 * and the sum over h is accumulated with Neumaier's compensated summation, so
 * the result is the exact sum to within a few units of 2^-53.  An optional
 * per-expert bias is added to the logits.
 * x [T][H] fp32, wr [H][E] fp32, bias [E] or NULL, logits [T][E] double. */
void oracle_router_logits(const float* x, const float* wr, const float* bias, int64_t T, int32_t H,
                          int32_t E, double* logits) {
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)E);
        double* c = (double*)malloc(sizeof(double) * (size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            for (int32_t e = 0; e < E; ++e) s[e] = 0.0, c[e] = 0.0;
            for (int32_t h = 0; h < H; ++h) {
                const double xv = (double)x[t * H + h];
                const float* w = wr + (int64_t)h * E;
                for (int32_t e = 0; e < E; ++e) {
                    const double v = xv * (double)w[e];
                    const double sum = s[e] + v;
                    const double big = fabs(s[e]) >= fabs(v) ? s[e] : v;
                    const double small = fabs(s[e]) >= fabs(v) ? v : s[e];
                    c[e] += (big - sum) + small;
                    s[e] = sum;
                }
            }
            for (int32_t e = 0; e < E; ++e)
                logits[t * E + e] = (s[e] + c[e]) + (bias ? (double)bias[e] : 0.0);
        }
        free(s);
        free(c);
    }
}

/* ------------------------------------------------------- c2 top-K, softmax
 * [prefill.cpp] route(logits, ids, w): the K experts of each token and their
 * weights.  The body of route() is not on the pages.  Readings: the ids are
 * the K largest logits in rank order (larger first; equal logits -> lower
 * expert index first); the weights are the softmax over the K selected logits
 * (equal to the softmax over all E renormalised on the K).
 * logits [T][E], ids [T][K], p [T][K] (double). */
void oracle_topk_softmax(const double* logits, int64_t T, int32_t E, int32_t K, int32_t* ids, double* p) {
#pragma omp parallel
    {
        char* taken = (char*)malloc((size_t)E);
#pragma omp for schedule(static)
        for (int64_t t = 0; t < T; ++t) {
            const double* l = logits + t * E;
            memset(taken, 0, (size_t)E);
            for (int32_t k = 0; k < K; ++k) {
                int32_t best = -1;
                for (int32_t e = 0; e < E; ++e) /* strict '>' keeps the lower index on ties */
                    if (!taken[e] && (best < 0 || l[e] > l[best])) best = e;
                taken[best] = 1;
                ids[t * K + k] = best;
            }
            const double m = l[ids[t * K]];
            double z = 0.0;
            for (int32_t k = 0; k < K; ++k) z += exp(l[ids[t * K + k]] - m);
            for (int32_t k = 0; k < K; ++k) p[t * K + k] = exp(l[ids[t * K + k]] - m) / z;
        }
        free(taken);
    }
}

/* -------------------------------------------------------------- c3 grouping
 * [moe_fused] group(): the routed pairs i = t*K + k are laid out expert by
 * expert; slot[i] is the row pair i lands in and src[row] the token (i / K)
 * that row reads.  The pages leave the order inside one expert open; the
 * reading taken is ascending pair index (the order of the MMQ path's host
 * grouping in [prefill.cpp], and ascending token order).  So the rows are the
 * pairs sorted by the key (expert id, pair index), a total order: this
 * function sorts the pair indices by that key and reads every table off the
 * sorted list.  offsets[e] is the first row whose expert is >= e.  Returns -1
 * if an id is outside [0, E), as the pages' "routed id out of range" check.
 * ids [T*K], offsets [E+1], src [T*K], slot [T*K]. */
static int ascending_i64(const void* a, const void* b) {
    const int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return x < y ? -1 : (x > y ? 1 : 0);
}

int oracle_group(const int32_t* ids, int64_t T, int32_t K, int32_t E, int32_t* offsets, int32_t* src,
                 int32_t* slot) {
    const int64_t n = T * K;
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= E) return -1;
    /* the key (expert id, pair index) as one integer: id * 2^32 + i (i < 2^31) */
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i) key[i] = (int64_t)ids[i] * ((int64_t)1 << 32) + i;
    qsort(key, (size_t)n, sizeof(int64_t), ascending_i64);
    int64_t row = 0;
    for (int32_t e = 0; e <= E; ++e) {
        while (row < n && key[row] / ((int64_t)1 << 32) < e) ++row;
        offsets[e] = (int32_t)row;
    }
    for (int64_t r = 0; r < n; ++r) {
        const int64_t i = key[r] % ((int64_t)1 << 32); /* the pair in row r */
        slot[i] = (int32_t)r;
        src[r] = (int32_t)(i / K);
    }
    free(key);
    return 0;
}

/* ------------------------------------------------- c4 / c6 int8 rounding
 * [moe_fused] activations are rounded to int8 with one scale per 32 values.
 * Readings (the pages do not give the rounding): per block of 32, a = max|v|,
 * s = a / 127 rounded to fp32, q = round-half-away-from-zero(v / s) with the
 * quotient rounded to fp32, clamped to [-127, 127]; an all-zero block has
 * s = 0 and q = 0.  The decision is taken in fp32, as the kernels take it:
 * dividing two fp32 values in double and rounding to fp32 gives the correctly
 * rounded fp32 quotient (53 >= 2*24 + 2 bits), so this is exact emulation.
 * v [rows][cols] fp32 (cols a multiple of 32), q [rows][cols], s [rows][cols/32]. */
static void quantize_block(const float* v, int8_t* q, float* s) {
    double a = 0.0;
    for (int i = 0; i < QBLOCK; ++i)
        if (fabs((double)v[i]) > a) a = fabs((double)v[i]);
    const float sc = (float)(a / 127.0);
    *s = sc;
    for (int i = 0; i < QBLOCK; ++i) {
        if (sc == 0.0f) {
            q[i] = 0;
            continue;
        }
        const double t = (double)(float)((double)v[i] / (double)sc); /* RN32(v / s) */
        double r = t >= 0.0 ? floor(t + 0.5) : -floor(-t + 0.5);  /* half away from zero */
        if (r > 127.0) r = 127.0;
        if (r < -127.0) r = -127.0;
        q[i] = (int8_t)r;
    }
}

void oracle_quantize(const float* v, int64_t rows, int32_t cols, int8_t* q, float* s) {
    const int32_t nb = cols / QBLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int32_t b = 0; b < nb; ++b)
            quantize_block(v + r * cols + (int64_t)b * QBLOCK, q + r * cols + (int64_t)b * QBLOCK, s + r * nb + b);
}

/* ----------------------------------------- c5..c7 one expert's routed rows
 * [moe_fused] per routed row (token t of expert e): gate and up from the int8
 * activations of t, SwiGLU, H rounded to int8 per 32 values, then down.
 * With the 2-bit map w = d*(q - z), z = 1.5 (the symmetric map) or z = 1
 * (the pages' Q2_0 packs, moe_fused.hpp header comment):
 *   G[j] = sum_b dg[j][b] * sx[b] * sum_{i in b} (qg[j][i] - z) * qx[i]
 *   U[j] likewise with the up rows (rows I + j of the stacked gate/up matrix)
 *   h[j] = G[j] / (1 + exp(-G[j])) * U[j]            (SwiGLU = silu(gate)*up)
 *   qh, sh = the int8 rounding of RN32(h) per 32 values along I (as c4)
 *   D[o] = sum_b dd[o][b] * sh[b] * sum_{i in b} (qd[o][i] - z) * qh[i]
 * Each per-block term is exact in double (a half-integer below 2^13 times an
 * 11-bit and a 24-bit significand); only the sums over blocks round.
 * Inputs: one expert's canonical arrays cgu [2I][H] (uint8 codes), sgu
 * [2I][H/32] (fp16 bits), cd [H][I], sd [H][I/32]; nrows activation rows
 * qx [nrows][H], sx [nrows][H/32].  Outputs (any may be NULL except D):
 * h [nrows][I] double, qh [nrows][I], sh [nrows][I/32], D [nrows][H] double. */
void oracle_expert_rows(const uint8_t* cgu, const uint16_t* sgu, const uint8_t* cd, const uint16_t* sd,
                        int32_t H, int32_t I, double z, int64_t nrows, const int8_t* qx, const float* sx,
                        double* h_out, int8_t* qh_out, float* sh_out, double* D) {
    const int32_t nbh = H / QBLOCK, nbi = I / QBLOCK;
#pragma omp parallel
    {
        double* h = (double*)malloc(sizeof(double) * (size_t)I);
        float* h32 = (float*)malloc(sizeof(float) * (size_t)I);
        int8_t* qh = (int8_t*)malloc((size_t)I);
        float* sh = (float*)malloc(sizeof(float) * (size_t)nbi);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const int8_t* xr = qx + r * H;
            const float* sxr = sx + r * nbh;
            for (int32_t j = 0; j < I; ++j) {
                double G = 0.0, U = 0.0;
                for (int32_t b = 0; b < nbh; ++b) {
                    double ig = 0.0, iu = 0.0;
                    for (int32_t i = b * QBLOCK; i < (b + 1) * QBLOCK; ++i) {
                        ig += ((double)cgu[(int64_t)j * H + i] - z) * (double)xr[i];
                        iu += ((double)cgu[(int64_t)(I + j) * H + i] - z) * (double)xr[i];
                    }
                    G += half_bits_to_double(sgu[(int64_t)j * nbh + b]) * (double)sxr[b] * ig;
                    U += half_bits_to_double(sgu[(int64_t)(I + j) * nbh + b]) * (double)sxr[b] * iu;
                }
                h[j] = G / (1.0 + exp(-G)) * U;
                h32[j] = (float)h[j];
            }
            for (int32_t b = 0; b < nbi; ++b) quantize_block(h32 + b * QBLOCK, qh + b * QBLOCK, sh + b);
            for (int32_t o = 0; o < H; ++o) {
                double acc = 0.0;
                for (int32_t b = 0; b < nbi; ++b) {
                    double id = 0.0;
                    for (int32_t i = b * QBLOCK; i < (b + 1) * QBLOCK; ++i)
                        id += ((double)cd[(int64_t)o * I + i] - z) * (double)qh[i];
                    acc += half_bits_to_double(sd[(int64_t)o * nbi + b]) * (double)sh[b] * id;
                }
                D[r * H + o] = acc;
            }
            if (h_out) memcpy(h_out + r * I, h, sizeof(double) * (size_t)I);
            if (qh_out) memcpy(qh_out + r * I, qh, (size_t)I);
            if (sh_out) memcpy(sh_out + r * nbi, sh, sizeof(float) * (size_t)nbi);
        }
        free(h);
        free(h32);
        free(qh);
        free(sh);
    }
}

/* Rows of several experts at once: row r uses expert slot which[r] of the
 * pointer tables (the same per-row computation as oracle_expert_rows, with
 * the loop over rows spread across threads). */
void oracle_rows_multi(const uint8_t* const* cgu, const uint16_t* const* sgu, const uint8_t* const* cd,
                       const uint16_t* const* sd, const int32_t* which, int32_t H, int32_t I, double z,
                       int64_t nrows, const int8_t* qx, const float* sx, double* h_out, int8_t* qh_out,
                       float* sh_out, double* D) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int32_t w = which[r];
        oracle_expert_rows(cgu[w], sgu[w], cd[w], sd[w], H, I, z, 1, qx + r * H, sx + r * (H / QBLOCK),
                           h_out ? h_out + r * I : NULL, qh_out ? qh_out + r * I : NULL,
                           sh_out ? sh_out + r * (I / QBLOCK) : NULL, D + r * H);
    }
}

/* ------------------------------------------------------------- c8 combine
 * [moe_fused] the combine reads the per-slot rows: y[t] = sum_k p[t][k] *
 * D[slot[t*K + k]], k ascending, in double.  The shared expert that the pages
 * add in the same MoE half is not part of the routed layer computed here.
 * D [T*K][H] double, p [T][K] double, slot [T*K], y [T][H] double. */
void oracle_combine(const double* D, const double* p, const int32_t* slot, int64_t T, int32_t K, int32_t H,
                    double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int32_t o = 0; o < H; ++o) {
            double acc = 0.0;
            for (int32_t k = 0; k < K; ++k) acc += p[t * K + k] * D[(int64_t)slot[t * K + k] * H + o];
            y[t * H + o] = acc;
        }
}
