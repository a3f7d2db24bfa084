// Grouped expert GEMMs: gate/up with SwiGLU and the int8 rounding of H fused
// in the epilogue (which can also write H straight into down's tiled fp16
// operand, with the block values of down's offset pass); down with the
// routing weight applied in its epilogue, writing each routed row's output to
// its grouped row; and the combine that adds a token's K rows.
//
// Strata compare v0.1.35...v0.1.37 page, include/strata/prefill/moe_fused.hpp,
// experts: per expert, gate/up on the int8 activations of its grouped rows
// (through src), SwiGLU, H rounded to int8 per 32 values in the epilogue, then
// down into the rows the combine reads; each expert is read where it is (no
// gather); the 2-bit codes are unpacked on chip.
//
// Arithmetic.  One weight block is 32 codes q of one row with one fp16 scale
// d, w = d * (q - 1.5); one activation block is 32 int8 codes a with an fp32
// scale s.  Their contribution to an output is
//     d * sum (q - 1.5) * (s a) = s * [sum d (q - 1) * a] + d * u,
//     u = -0.5 * s * sum(a)  (one value per activation block).
// With the pages' Q2_0 map w = d * (q - 1) the same GEMM runs with u = 0
// (the offset pass is then skipped).
// The bracket runs on v_mfma_f32_16x16x32_f16 (K = 32 = one block) with a
// zero accumulator: the A operand d*(q-1) is exact in fp16 (q - 1 in
// {-1, 0, 1, 2}), the B operand is the int8 codes a themselves (exact in
// fp16), and the product is d times an integer below 2^13, at most 24
// significant bits, so the block sum comes out of the MFMA exactly.  One fp32
// FMA per output then adds it times the block's s.  Both GEMMs take this
// form: gate/up on the layer input's codes, down on the int8 SwiGLU codes.
// The d*u terms of all blocks form a small matrix product over the block
// index (K = Kd/32), done after the block loop on the MFMA unit: A = d (exact
// in fp16), B = u of each row scaled by a power of two to [-1, 1] and split
// into a high and a low fp16 part (22 bits).
//
// Work split.  A workgroup (4 waves) takes one chunk of at most 192 grouped
// rows of one expert and one 128-row weight slab (8 fragments of 16 rows).
// Per 32-wide block each thread unpacks one dword of 16 codes into LDS, so the
// slab's block is unpacked once and read by all 4 waves (double-buffered, one
// barrier per block).  The chunk's rows form 16-row tiles; wave w owns tiles
// w, w+4, w+8 and keeps their activation fragments in registers.  Lane l of a
// 16x16 output holds routed row (column) l % 16 and weight rows
// 4*(l/16) + v, v = 0..3, so a row's scale is one value per lane.
//
// Mapping.  Workgroups are dealt round-robin to the 8 XCDs; the id ->
// (chunk, slab) map keeps every slab of a chunk on one XCD, so that chunk's
// activation rows are fetched into one L2 only.
#include "internal.h"

namespace strata_moe {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kFrags = kSlabRows / 16;                               // 8
constexpr int kTilesPerWave = kChunkRows / (16 * kWaves);            // 3
constexpr int kParkStride = kSlabRows + 4;                           // floats per parked output row
constexpr int kSmallTiles = 2;       // 16-row tiles per pass of the small-chunk kernel
constexpr int kDlStride = 40;        // fp16 per row of a small-chunk wave's d buffer (32 blocks + pad)
constexpr int kBufferWord3 = 0x00020000;  // buffer descriptor word 3 for raw dword loads on gfx9 (gfx950)

__device__ __forceinline__ _Float16 lo_half(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ __forceinline__ _Float16 hi_half(uint32_t w) { return __builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

// One packed dword (16 codes) -> two A fragments of 8 fp16 values d*(q-1).
// Pair m (0..7) of the dword fills fragment m/4, elements 2(m%4) and
// 2(m%4)+1; its codes sit at bits [2m, 2m+1] and [16+2m, 17+2m].  A code at
// mantissa bits [2j, 2j+1] of an fp16 whose exponent gives those bits the
// weight 1 (2^10, 2^8, 2^6, 2^4, 2^2 for j = 0..4) reads as 2^(10-2j) + q
// exactly, so one AND-OR per pair places both codes (pairs 5..7 after one
// shift of the dword by 10); subtracting 2^(10-2j) + 1 gives q - 1 and the
// product with d is exact.  The five exponent patterns live in VGPRs (the
// AND-OR takes the mask as its one scalar operand).
struct UnpackMagic {
    uint32_t m[5];
    __device__ __forceinline__ UnpackMagic() {
#pragma unroll
        for (int j = 0; j < 5; ++j) {
            uint32_t v = (uint32_t)(0x6400u - 0x0800u * j) * 0x00010001u;
            asm("" : "+v"(v));  // keep the pattern in a VGPR
            m[j] = v;
        }
    }
};

__device__ __forceinline__ void unpack_dword(uint32_t x, _Float16 d0, _Float16 d1, const UnpackMagic& mg,
                                             half8_t& a0, half8_t& a1) {
#pragma clang fp contract(off)
    const half2_t s0 = {d0, d0}, s1 = {d1, d1};
    const uint32_t y = x >> 10;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
        const int j = m < 5 ? m : m - 5;
        const uint32_t w = ((m < 5 ? x : y) & (0x00030003u << (2 * j))) | mg.m[j];
        const _Float16 c = (_Float16)(float)((1 << (10 - 2 * j)) + 1);
        const half2_t bias = {c, c};
        const half2_t h = (__builtin_bit_cast(half2_t, w) - bias) * (m < 4 ? s0 : s1);
        if (m < 4) {
            a0[2 * (m & 3)] = h[0];
            a0[2 * (m & 3) + 1] = h[1];
        } else {
            a1[2 * (m & 3)] = h[0];
            a1[2 * (m & 3) + 1] = h[1];
        }
    }
}

__device__ __forceinline__ float round_half_away(float t) {
    const float r = floorf(fabsf(t) + 0.5f);
    return copysignf(fminf(r, 127.0f), t);
}

// The 4-wave kernel reads its activations (B operand) in the tiled layout of
// the grouped rows: [tile][block][group g][16 rows][8] fp16 codes, so the
// fragment of one 16-row tile and block is 1 KiB in MFMA lane order (lane
// 16 g + r holds row r, values 8g .. 8g + 7) and one coalesced 16-byte load
// per lane.  The block scales are tiled alike: [tile][block / 4][16 rows][4]
// fp32 (blocks padded with zeros to a multiple of 4).  For a tile's lane:
// activation offset tile * nblk * kTiledBlockBytes + 16 * lane, plus
// blk * kTiledBlockBytes; scale offset tile * tiled_scale_stride(nblk) +
// 16 * r, plus tiled_scale_offset(blk).
constexpr int kTiledBlockBytes = 16 * kBlock * 2;
__device__ __forceinline__ int tiled_scale_offset(int blk) { return (blk >> 2) * 256 + (blk & 3) * 4; }
__host__ __device__ __forceinline__ int tiled_scale_stride(int nblk) { return (nblk + 3) / 4 * 256; }
// The small-chunk kernel reads its block scales as rows [rows][Kd / 32] fp32
// (gate/up: the tokens' scales; down: the grouped rows' scales).  Its
// gate/up codes are read in place too: [tokens][Kd] fp16 (64 bytes per block
// of a row); its down codes come from the tiled layout above.
constexpr int kRowBlockBytes = kBlock * 2;

struct GemmArgs {
    const uint8_t* blobs;  // packed matrices, one per expert
    int64_t stride;        // bytes between experts
    const Tile* chunks;    // this kernel's list of chunks of grouped rows
    const int32_t* nchunks;  // its length
    int32_t nslab;         // 128-row slabs of the packed matrix
    int32_t Kd;            // reduction length (H for gate/up, I for down)
    const int32_t* src;    // token of each grouped row
    const float* prow;     // routing weight of each grouped row (down)
    const _Float16* act;   // activation codes fp16: tiled, or (small-chunk gate/up) [tokens][Kd]
    int64_t act_rows;      // rows of act
    const float* ascale;   // their block scales: tiled [tile][ceil(Kd / 128)][16][4] (4-wave kernel) or
                           // [rows][Kd / 32] (small-chunk kernel)
    int64_t scale_bytes;   // bytes of ascale
    const _Float16* uop;   // offset-pass operand [rows][nch x 32 blocks x 2] (hi, lo), or null (no offset)
    const float* um;       // its row multipliers [rows]
    int32_t I, H;
    int8_t* hq;            // gate/up: H codes [n][I]
    float* hs;             // gate/up: H scales [n][I/32]
    float* y;              // down: weighted routed rows dm [n][H]
    // the launch's chunks: all of the list, or (first != null) entries
    // [first[e0], first[e1]) of it, the chunks of experts [e0, e1)
    const int32_t* first;
    int32_t e0, e1;
    int64_t ring0;         // nring > 0: expert e's blob is in slot (ring0 + e) % nring
    int32_t nring;
    int32_t min_rows;      // small-chunk kernel: chunks with fewer rows are the GEMV kernel's
    // gate/up (optional): the down GEMM's operand written from the epilogue
    // (HTiled); null: only hq / hs
    _Float16* hbt = nullptr;
    float* hbs = nullptr;
    float* hu = nullptr;
    float huoff = 0.f;
};

// Expert e's packed matrix: resident at blobs + e * stride, or in its slot of
// the ring of streamed experts.
__device__ __forceinline__ const uint8_t* expert_blob(const GemmArgs& g, int e) {
    const int64_t slot = g.nring > 0 ? (g.ring0 + e) % g.nring : (int64_t)e;
    return g.blobs + slot * g.stride;
}

// The launch's range of its chunk list: [*lo, *hi).
__device__ __forceinline__ void chunk_range(const GemmArgs& g, int* lo, int* hi) {
    *lo = g.first ? g.first[g.e0] : 0;
    *hi = g.first ? g.first[g.e1] : *g.nchunks;
}

// The K loop over 32-wide blocks.  Per block: every thread unpacks its dword
// of the slab's record into LDS buffer b&1 (and the two scales into the
// offset-pass matrix), one barrier, then the wave's NT tiles x 8 fragments of
// MFMAs, fragment-major.
// Records are prefetched several blocks ahead in a register ring and
// activation fragments one block ahead in two alternating register sets, so
// the loop body has no copies.
struct BlockLoop {
    __amdgpu_buffer_rsrc_t rec;  // this slab's records (nblk x 1280 bytes)
    __amdgpu_buffer_rsrc_t act;  // activation codes fp16, tiled
    __amdgpu_buffer_rsrc_t scl;  // their block scales fp32, tiled
    int32_t Kd, nblk, dstride;
    int tau, lane, r16, kg, p;
    _Float16* d_lds;
    half8_t (*a_lds)[kFrags][64];
    UnpackMagic mg;
    int dw0;  // the first record dword this thread unpacks (a multiple of 64 plus its lane)

    // Buffer loads: per-lane offsets are loop-invariant, the block enters as a
    // scalar offset.  A block beyond the last re-reads the last one.  Dwords
    // dw0 and dw0 + 64 share their scale dword (the lane's).
    template <int KW>
    __device__ __forceinline__ void load_record(int blk, uint32_t& xw, uint32_t& xw2, uint32_t& sw) const {
        blk = blk < nblk ? blk : nblk - 1;
        xw = __builtin_amdgcn_raw_buffer_load_b32(rec, dw0 * 4, blk * kRecordBytes, 0);
        if constexpr (KW == 2) xw2 = __builtin_amdgcn_raw_buffer_load_b32(rec, dw0 * 4 + 256, blk * kRecordBytes, 0);
        sw = __builtin_amdgcn_raw_buffer_load_b32(rec, kRecordCodeBytes + lane * 4, blk * kRecordBytes, 0);
    }

    // Activation fragments of a block (tiled): lvoff[i] is this lane's byte
    // offset in tile i.
    template <int NT>
    __device__ __forceinline__ void load_act(int blk, const int (&lvoff)[kTilesPerWave],
                                             half8_t (&bf)[kTilesPerWave]) const {
        blk = blk < nblk ? blk : nblk - 1;
#pragma unroll
        for (int i = 0; i < NT; ++i)
            bf[i] = __builtin_bit_cast(half8_t,
                                       __builtin_amdgcn_raw_buffer_load_b128(act, lvoff[i], blk * kTiledBlockBytes, 0));
    }

    // The block scale of this lane's MFMA column in each tile; soff[i] is the
    // byte offset of that row's scales (tiled).
    template <int NT>
    __device__ __forceinline__ void load_scales(int blk, const int (&soff)[kTilesPerWave],
                                                float (&sv)[kTilesPerWave]) const {
        blk = blk < nblk ? blk : nblk - 1;
#pragma unroll
        for (int i = 0; i < NT; ++i)
            sv[i] = __builtin_bit_cast(float,
                                       __builtin_amdgcn_raw_buffer_load_b32(scl, soff[i], tiled_scale_offset(blk), 0));
    }

    // The same for blocks blk .. blk + 3 (blk a multiple of 4, 4 | nblk): one
    // 16-byte load per tile and 4 blocks.
    template <int NT>
    __device__ __forceinline__ void load_scales4(int blk, const int (&soff)[kTilesPerWave],
                                                 float4_t (&sq)[kTilesPerWave]) const {
        blk = blk < nblk ? blk : nblk - 4;
#pragma unroll
        for (int i = 0; i < NT; ++i)
            sq[i] = __builtin_bit_cast(float4_t,
                                       __builtin_amdgcn_raw_buffer_load_b128(scl, soff[i], tiled_scale_offset(blk), 0));
    }

    // Record dword dw holds fragments 2p and 2p+1 of MFMA lane dw / 4
    // (p = dw % 4, the thread's lane % 4), stored at lane slot (dw / 4) ^ 2p
    // so that the four pairs of one lane fall in different LDS banks.
    __device__ __forceinline__ void unpack(int blk, int dw, uint32_t xw, uint32_t sw) const {
        half8_t a0, a1;
        const _Float16 d0 = lo_half(sw), d1 = hi_half(sw);
        unpack_dword(xw, d0, d1, mg, a0, a1);
        const int ul = dw >> 2, ur16 = ul & 15;
        a_lds[blk & 1][2 * p][ul ^ (2 * p)] = a0;
        a_lds[blk & 1][2 * p + 1][ul ^ (2 * p)] = a1;
        // every unpacking wave holds the same scales of a row: all write, no
        // branch, so the unpack can interleave with the MFMAs of the previous
        // block
        d_lds[(32 * p + ur16) * dstride + blk] = d0;
        d_lds[(32 * p + 16 + ur16) * dstride + blk] = d1;
    }

    template <int NT>
    __device__ __forceinline__ void products(int blk, const half8_t (&raw)[kTilesPerWave],
                                             const float (&sv)[kTilesPerWave],
                                             float4_t (&acc)[kFrags][kTilesPerWave]) const {
        const half8_t (&bf)[kTilesPerWave] = raw;  // tiled: already in the MFMA layout
        // A fragments in two groups of four (registers are tight: the next
        // block's unpack interleaves with these MFMAs)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            half8_t a[kFrags / 2];
#pragma unroll
            for (int f = 0; f < kFrags / 2; ++f) a[f] = a_lds[blk & 1][4 * g + f][lane ^ ((4 * g + f) & ~1)];
            if constexpr (NT > 0) {
                // the FMAs that scale a product run kLag MFMAs later, beside
                // the MFMAs in between (issued as one MFMA, then four FMAs),
                // so the wave does not wait for each product in turn
                constexpr int kLag = 2, kN = kFrags / 2 * NT;
                float4_t tq[kLag + 1];
#pragma unroll
                for (int k = 0; k < kN + kLag; ++k) {
                    if (k < kN)
                        tq[k % (kLag + 1)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            a[k / NT], bf[k % NT], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    if (k >= kLag) {
                        const int kp = k - kLag, f = kp / NT, i = kp % NT;
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            acc[4 * g + f][i][v] = fmaf(tq[kp % (kLag + 1)][v], sv[i], acc[4 * g + f][i][v]);
                    }
                    if (k < kN) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    if (k >= kLag) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // then its FMAs
                }
            }
        }
    }

    // One step per block: unpack the block's record into LDS, one barrier,
    // issue the loads of later blocks, then the block's MFMAs.  Records (from
    // HBM) run D blocks ahead in a register ring (5 bytes per thread and
    // block), activation fragments (mostly from L2) one block ahead in two
    // register sets.  D divides nblk, so the unrolled body has no exit in the
    // middle and every ring index is a compile-time constant.
    // KW: record dwords this thread unpacks per block (0, 1 or 2).
    template <int NT, int D, int KW>
    __device__ __forceinline__ void run(const int (&lvoff)[kTilesPerWave], const int (&soff)[kTilesPerWave],
                                        float4_t (&acc)[kFrags][kTilesPerWave]) const {
        static_assert(D % 2 == 0, "activation sets alternate per block");
        // 8 | D: block scales in 4-block batches (two sets, batch (blk / 4) & 1
        // = j / 4), the next batch loaded one block ahead
        constexpr bool kBatch = D % 8 == 0;
        uint32_t xw[D], xw2[D], sw[D];
        half8_t bf[2][kTilesPerWave];
        float sv[2][kTilesPerWave] = {};
        float4_t sq[2][kTilesPerWave] = {};
        // Issue order matters: each unpack waits for its record with a vmcnt
        // that counts the loads issued after it, and the loop header merges
        // the entry path with the back edge.  Records first, as in the loop.
#pragma unroll
        for (int j = 0; j < D; ++j)
            if constexpr (KW > 0) load_record<KW>(j, xw[j], xw2[j], sw[j]);
        __builtin_amdgcn_sched_barrier(0);
        load_act<NT>(0, lvoff, bf[0]);
        if constexpr (kBatch)
            load_scales4<NT>(0, soff, sq[0]);
        else
            load_scales<NT>(0, soff, sv[0]);
        __builtin_amdgcn_sched_barrier(0);
        for (int b = 0; b < nblk; b += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const int blk = b + j;
                if constexpr (KW > 0) unpack(blk, dw0, xw[j], sw[j]);
                if constexpr (KW == 2) unpack(blk, dw0 + 64, xw2[j], sw[j]);
                __syncthreads();
                if constexpr (KW > 0) load_record<KW>(blk + D, xw[j], xw2[j], sw[j]);
                load_act<NT>(blk + 1, lvoff, bf[(j + 1) & 1]);
                if constexpr (kBatch) {
                    if ((j & 3) == 3) load_scales4<NT>(blk + 1, soff, sq[((j >> 2) + 1) & 1]);
                } else {
                    load_scales<NT>(blk + 1, soff, sv[(j + 1) & 1]);
                }
                __builtin_amdgcn_sched_barrier(0);  // loads go out before the MFMAs
                if constexpr (kBatch) {
                    float s[kTilesPerWave];
#pragma unroll
                    for (int i = 0; i < kTilesPerWave; ++i) s[i] = sq[(j >> 2) & 1][i][j & 3];
                    products<NT>(blk, bf[j & 1], s, acc);
                } else {
                    products<NT>(blk, bf[j & 1], sv[j & 1], acc);
                }
            }
        }
    }
};


// Gate/up epilogue of one 16-row tile of routed rows (column r16 of this lane,
// grouped row r of the chunk) against one slab: fragments 0..3 are the gate
// rows 64*slab + 16f + 4kg + v, fragments 4..7 the up rows of the same j.
// SwiGLU, then the two 32-wide H blocks of the slab rounded to int8 with their
// scales (the max over a block spans the 4 lanes kg of the row).
__device__ __forceinline__ void gate_up_store(const GemmArgs& g, const Tile& tl, int slab, int r, int kg,
                                              const float4_t (&a)[kFrags]) {
    const int nbi = g.I / kBlock;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
        float h[2][4];
        float amax = 0.f;
#pragma unroll
        for (int ff = 0; ff < 2; ++ff)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float gt = a[2 * hb + ff][v], up = a[4 + 2 * hb + ff][v];
                // silu(gate) * up; hardware exp and reciprocal (about 2 ulp),
                // far inside the rounding-tie tolerance of the int8 H codes
                h[ff][v] = gt * up * __builtin_amdgcn_rcpf(1.0f + __expf(-gt));
                amax = fmaxf(amax, fabsf(h[ff][v]));
            }
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const float sh = amax / 127.0f;
        float q[2][4];
#pragma unroll
        for (int ff = 0; ff < 2; ++ff)
#pragma unroll
            for (int v = 0; v < 4; ++v) q[ff][v] = sh != 0.0f ? round_half_away(h[ff][v] / sh) : 0.0f;
        if (g.hbt) {  // uniform
            // the down GEMM's operand: tile tl.tile0 + r / 16, block 2 slab + hb;
            // this lane's values k = 16 ff + 4 kg + v sit in group 2 ff + kg / 2
            // at positions 4 (kg & 1) + v; padding rows get zeros
            const bool valid = r < tl.nrows;
            const int bb = 2 * slab + hb, nq = (nbi + 3) / 4, rr = r & 15;
            const int64_t t = tl.tile0 + (r >> 4);
            int sum = 0;
#pragma unroll
            for (int ff = 0; ff < 2; ++ff) {
                half4_t h4;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    h4[v] = valid ? (_Float16)q[ff][v] : (_Float16)0.0f;
                    sum += valid ? (int)q[ff][v] : 0;
                }
                *reinterpret_cast<half4_t*>(g.hbt + ((t * nbi + bb) * 64 + 16 * (2 * ff + (kg >> 1)) + rr) * 8 +
                                            4 * (kg & 1)) = h4;
            }
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            if (kg == 0) {
                g.hbs[((t * nq + (bb >> 2)) * 16 + rr) * 4 + (bb & 3)] = valid ? sh : 0.0f;
                if (valid && g.hu) g.hu[(tl.row0 + r) * (int64_t)((nbi + 31) / 32 * 32) + bb] = -g.huoff * sh * (float)sum;
            }
        }
        if (r < tl.nrows) {
            const int64_t row = tl.row0 + r;
            if (g.hq) {  // uniform; null when only the tiled operand is wanted
                int8_t* dst = g.hq + row * g.I + 64 * slab + 32 * hb + 4 * kg;
#pragma unroll
                for (int ff = 0; ff < 2; ++ff) {
                    const uint32_t packed = (uint32_t)(uint8_t)(int8_t)(int)q[ff][0] |
                                            (uint32_t)(uint8_t)(int8_t)(int)q[ff][1] << 8 |
                                            (uint32_t)(uint8_t)(int8_t)(int)q[ff][2] << 16 |
                                            (uint32_t)(uint8_t)(int8_t)(int)q[ff][3] << 24;
                    *reinterpret_cast<uint32_t*>(dst + 16 * ff) = packed;
                }
            }
            if (kg == 0) g.hs[row * nbi + 2 * slab + hb] = sh;
        }
    }
}

// Down epilogue of one 16-row tile (chunk rows 16*tt .. 16*tt + 15) against one
// slab: each routed row's outputs times its routing weight w, written to its
// grouped row of dm [n][H] (the rows the combine reads).  The wave parks the
// 16 rows x 128 outputs in its LDS area `park` and stores them row by row,
// 512 contiguous bytes per row.
__device__ __forceinline__ void down_store(const GemmArgs& g, const Tile& tl, int slab, int tt, int lane, float w,
                                           const float4_t (&a)[kFrags], float* park) {
    const int r16 = lane & 15, kg = lane >> 4;
#pragma unroll
    for (int f = 0; f < kFrags; ++f) {
        const float4 v4 = make_float4(w * a[f][0], w * a[f][1], w * a[f][2], w * a[f][3]);
        *reinterpret_cast<float4*>(park + r16 * kParkStride + 16 * f + 4 * kg) = v4;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // float4 (j*64 + lane): row (j*64 + lane) / 32 of the tile, outputs 4*((j*64 + lane) % 32)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int flat = j * 64 + lane;
        const int rr = flat >> 5, c4 = flat & 31;
        const int r = 16 * tt + rr;
        if (r < tl.nrows) {
            const float4 v4 = *reinterpret_cast<const float4*>(park + rr * kParkStride + 4 * c4);
            *reinterpret_cast<float4*>(g.y + (int64_t)(tl.row0 + r) * g.H + kSlabRows * slab + 4 * c4) = v4;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// The block loop of one wave's shape (wave-uniform): ntw tiles, kw record
// dwords unpacked per thread and block.
template <int D, typename Loop>
__device__ __forceinline__ void run_shape(const Loop& L, int ntw, int kw, const int (&lvoff)[kTilesPerWave],
                                          const int (&soff)[kTilesPerWave], float4_t (&acc)[kFrags][kTilesPerWave]) {
    switch (3 * ntw + kw) {
        case 0: L.template run<0, D, 0>(lvoff, soff, acc); break;
        case 1: L.template run<0, D, 1>(lvoff, soff, acc); break;  // no tiles: still unpack, meet every barrier
        case 2: L.template run<0, D, 2>(lvoff, soff, acc); break;
        case 3: L.template run<1, D, 0>(lvoff, soff, acc); break;
        case 4: L.template run<1, D, 1>(lvoff, soff, acc); break;
        case 5: L.template run<1, D, 2>(lvoff, soff, acc); break;
        case 6: L.template run<2, D, 0>(lvoff, soff, acc); break;
        case 7: L.template run<2, D, 1>(lvoff, soff, acc); break;
        case 8: L.template run<2, D, 2>(lvoff, soff, acc); break;
        case 9: L.template run<3, D, 0>(lvoff, soff, acc); break;
        case 10: L.template run<3, D, 1>(lvoff, soff, acc); break;
        default: L.template run<3, D, 2>(lvoff, soff, acc); break;
    }
}

// kGateUp: activation rows are tokens (through src), epilogue SwiGLU + int8 H.
// Otherwise: activation rows are the grouped rows, epilogue weighted row stores.
// One work item of the 4-wave kernel: chunk tl against slab `slab`.
template <bool kGateUp>
__device__ __forceinline__ void big_chunk_item(const GemmArgs& g, const Tile tl, int slab,
                                               half8_t (*a_lds)[kFrags][64], _Float16* d_lds) {
    const int tau = threadIdx.x, lane = tau & 63, r16 = lane & 15, kg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tau >> 6);
    const int nblk = g.Kd / kBlock;
    const int nch = (nblk + 31) / 32;
    const int dstride = nch * 32 + 8;

    // zero the padding blocks of the offset-pass matrix: two threads per row
    for (int c = nblk + (tau & 1); c < nch * 32; c += 2) d_lds[(tau >> 1) * dstride + c] = (_Float16)0.0f;

    // this wave's tiles: arow = activation row of this lane's MFMA column
    // (gate/up: its token, down: its grouped row), lvoff = byte offset of its
    // loader row and group, soff = byte offset of the column's block scales
    // (padding rows are zeros in the tiled operands and are never stored)
    const int sstride = tiled_scale_stride(nblk);
    int64_t arow[kTilesPerWave];
    int lvoff[kTilesPerWave], soff[kTilesPerWave];
    int ntw = 0;
    const int tw = wave;
#pragma unroll
    for (int i = 0; i < kTilesPerWave; ++i) {
        const int tt = tw + kWaves * i;
        const int r = 16 * tt + r16;
        if (16 * tt < tl.nrows) ntw = i + 1;  // wave-uniform
        arow[i] = -1;
        if (r < tl.nrows) arow[i] = kGateUp ? (int64_t)g.src[tl.row0 + r] : (int64_t)(tl.row0 + r);
        // tile tt of the chunk in the tiled operands (padding rows are zeros, never stored)
        lvoff[i] = (tl.tile0 + tt) * nblk * kTiledBlockBytes + 16 * lane;
        soff[i] = (tl.tile0 + tt) * sstride + 16 * r16;
    }

    const uint8_t* rec = expert_blob(g, tl.e) + (int64_t)slab * nblk * kRecordBytes;
    const int p = tau & 3;  // fragment pair this thread unpacks: fragments 2p, 2p+1 of MFMA lane tau / 4

    float4_t acc[kFrags][kTilesPerWave];
#pragma unroll
    for (int f = 0; f < kFrags; ++f)
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i) acc[f][i] = (float4_t){0.f, 0.f, 0.f, 0.f};
    BlockLoop L{
        __builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, nblk * kRecordBytes, kBufferWord3),
        __builtin_amdgcn_make_buffer_rsrc((void*)g.act, (short)0, (int)(g.act_rows * g.Kd * 2), kBufferWord3),
        __builtin_amdgcn_make_buffer_rsrc((void*)g.ascale, (short)0, (int)g.scale_bytes, kBufferWord3),
        g.Kd, nblk, dstride, tau, lane, r16, kg, p, d_lds, a_lds, UnpackMagic(), 0};
    // The record's 256 dwords are unpacked by the waves with fewer tiles where
    // the chunk's tiles do not split evenly (nt = 4q + r; waves 0..r-1 hold
    // q + 1 tiles): r = 1: dwords per lane (0, 2, 1, 1); r = 2: (0, 0, 2, 2);
    // else one each.  The busiest waves then skip the unpack.
    const int rem = ((tl.nrows + 15) / 16) & 3;
    const int kw = rem == 1 ? (wave == 0 ? 0 : wave == 1 ? 2 : 1) : rem == 2 ? (wave < 2 ? 0 : 2) : 1;
    const int kw_before = rem == 1 ? (wave == 0 ? 0 : wave == 1 ? 0 : wave) : rem == 2 ? (wave < 3 ? 0 : 2) : wave;
    L.dw0 = 64 * kw_before + lane;
    // wave-uniform: the block loop is straight-line code for 1..3 tiles; the
    // record ring is 8 deep when 8 divides the block count (H = 2560, I = 1024)
    if (nblk % 8 == 0)
        run_shape<8>(L, ntw, kw, lvoff, soff, acc);
    else
        run_shape<2>(L, ntw, kw, lvoff, soff, acc);
    __syncthreads();  // every d of the slab is in LDS

    // offset pass: acc += 2^eu * sum_b d[row][b] * u'[row][b], 32 blocks per
    // MFMA, u' = u * 2^-eu as hi and lo fp16 (prepared with the activations,
    // zero-padded to whole chunks of 32 blocks, like the zeroed d padding).
    // Without an offset operand (the Q2_0 map, u = 0) there is none.
#pragma unroll
    for (int i = 0; i < kTilesPerWave; ++i) {
        if (i >= ntw || !g.uop) continue;
        const int64_t ar = arow[i] >= 0 ? arow[i] : 0;
        const half8_t* urow = reinterpret_cast<const half8_t*>(g.uop + ar * nch * 64) + 2 * kg;
        half8_t ub[kMaxOffsetChunks][2];
#pragma unroll
        for (int c = 0; c < kMaxOffsetChunks; ++c)
            if (c < nch) {
                ub[c][0] = urow[8 * c];
                ub[c][1] = urow[8 * c + 1];
            }
        float4_t corr[kFrags];
#pragma unroll
        for (int f = 0; f < kFrags; ++f) corr[f] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < kMaxOffsetChunks; ++c) {
            if (c >= nch) break;
#pragma unroll
            for (int f = 0; f < kFrags; ++f) {
                const half8_t da =
                    *reinterpret_cast<const half8_t*>(&d_lds[(16 * f + r16) * dstride + 32 * c + 8 * kg]);
                corr[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da, ub[c][0], corr[f], 0, 0, 0);
                corr[f] = __builtin_amdgcn_mfma_f32_16x16x32_f16(da, ub[c][1], corr[f], 0, 0, 0);
            }
        }
        const float up = arow[i] >= 0 ? g.um[arow[i]] : 0.f;
#pragma unroll
        for (int f = 0; f < kFrags; ++f)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[f][i][v] = fmaf(corr[f][v], up, acc[f][i][v]);
    }

    if constexpr (kGateUp) {
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i) {
            if (i >= ntw) continue;
            float4_t a[kFrags];
#pragma unroll
            for (int f = 0; f < kFrags; ++f) a[f] = acc[f][i];
            gate_up_store(g, tl, slab, 16 * (tw + kWaves * i) + r16, kg, a);
        }
    } else {
        float* park = reinterpret_cast<float*>(d_lds + kSlabRows * dstride) + wave * 16 * kParkStride;
#pragma unroll
        for (int i = 0; i < kTilesPerWave; ++i) {
            if (i >= ntw) continue;
            float4_t a[kFrags];
#pragma unroll
            for (int f = 0; f < kFrags; ++f) a[f] = acc[f][i];
            down_store(g, tl, slab, tw + kWaves * i, lane, arow[i] >= 0 ? g.prow[arow[i]] : 0.f, a, park);
        }
    }
}


// One workgroup per (chunk, slab); the id -> (chunk, slab) map keeps every
// slab of a chunk on one XCD (workgroups are dealt round-robin to the 8
// XCDs), so that chunk's activation rows are fetched into one L2 only.
template <bool kGateUp>
__global__ void __launch_bounds__(256, 2) expert_gemm_kernel(GemmArgs g) {
    __shared__ half8_t a_lds[2][kFrags][64];
    extern __shared__ _Float16 d_lds[];  // [kSlabRows][dstride]: d of every row and block (offset pass)
    const int id = blockIdx.x;
    const int local = id >> 3;
    int lo, hi;
    chunk_range(g, &lo, &hi);
    const int chunk = lo + (local / g.nslab) * 8 + (id & 7);
    if (chunk >= hi) return;  // uniform over the workgroup, before any barrier
    const Tile tl = g.chunks[chunk];   // a copy: read once, before any store
    big_chunk_item<kGateUp>(g, tl, local % g.nslab, a_lds, d_lds);
}

// Small-chunk kernel (chunks of at most kSmallRows routed rows, the common
// case when a prompt chunk gives each expert only a few rows).  There the
// 4-wave kernel above leaves most of its waves without a tile, and its
// per-block barrier is paid for very few MFMAs.  Here each wave streams one
// slab on its own: per block a lane loads the four dwords of its (r16, kg)
// position (fragments 0..7) and the scales of its rows, unpacks them in
// registers and runs the MFMAs of every tile of the chunk (at most two per
// pass; a three-tile chunk takes two passes).  A workgroup holds four waves on
// four consecutive slabs of one chunk, so the activation fragments they all
// read come from the CU's L1.  No workgroup barrier: each wave keeps the d of
// its rows for the offset pass in its own LDS area, 32 blocks at a time, and
// runs that pass every 32 blocks, adding it with the ratio of the two row
// multipliers (powers of two) before the final multiply.
// The activation fragments are read straight in the MFMA layout: at one
// 16-byte load per tile and block the L1 keeps up with 16 rows per load, and
// the lane exchange of the 4-wave kernel costs more than it saves here.
// kInPlace: the B codes are read from their rows in place (gate/up: the
// tokens' codes [tokens][Kd]); otherwise from the tiled layout (down).
template <int NT, bool kInPlace>
struct SlabPass {
    __amdgpu_buffer_rsrc_t rec, act, scl;
    int32_t Kd, nblk;
    int lane, r16, kg;
    _Float16* dl;  // [kSlabRows][kDlStride]
    UnpackMagic mg;

    // A lane's four code dwords (fragments 0..7 at its position) and the 8
    // scales of its row are 16 contiguous bytes each.
    __device__ __forceinline__ void load_record(int blk, uint32_t (&xw)[4], uint32_t (&sw)[4]) const {
        blk = blk < nblk ? blk : nblk - 1;
        const auto c = __builtin_amdgcn_raw_buffer_load_b128(rec, lane * 16, blk * kRecordBytes, 0);
        const auto d = __builtin_amdgcn_raw_buffer_load_b128(rec, kRecordCodeBytes + r16 * 16, blk * kRecordBytes, 0);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            xw[p] = c[p];
            sw[p] = d[p];
        }
    }

    // Activation fragments of a block (lvoff: this lane's byte offset; gate/up
    // its column's row and group in place, down its place in the tiled
    // operand), and if `scales` the block scale of the lane's column in each
    // tile (soff: byte offset of that row's scales).
    __device__ __forceinline__ void load_act(int blk, const int (&lvoff)[NT], const int (&soff)[NT],
                                             half8_t (&bf)[NT], float (&sv)[NT], bool scales) const {
        blk = blk < nblk ? blk : nblk - 1;
        constexpr int kStride = kInPlace ? kRowBlockBytes : kTiledBlockBytes;
#pragma unroll
        for (int i = 0; i < NT; ++i)
            bf[i] = __builtin_bit_cast(half8_t, __builtin_amdgcn_raw_buffer_load_b128(act, lvoff[i], blk * kStride, 0));
        if (scales)
#pragma unroll
            for (int i = 0; i < NT; ++i)
                sv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(scl, soff[i], blk * 4, 0));
    }

    // The scales of blocks blk .. blk + 3 (blk a multiple of 4, 4 | nblk),
    // one 16-byte load per tile instead of four gathered dwords.
    __device__ __forceinline__ void load_scales4(int blk, const int (&soff)[NT], float4_t (&sq)[NT]) const {
        blk = blk < nblk ? blk : nblk - 4;
#pragma unroll
        for (int i = 0; i < NT; ++i)
            sq[i] = __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(scl, soff[i], blk * 4, 0));
    }

    // Unpack dword p (fragments 2p, 2p+1).
    __device__ __forceinline__ void prepare(int p, const uint32_t (&xw)[4], const uint32_t (&sw)[4],
                                            half8_t (&a)[2]) const {
        unpack_dword(xw[p], lo_half(sw[p]), hi_half(sw[p]), mg, a[0], a[1]);
    }

    // Park the block's scales for the offset pass.  The four lanes kg of a
    // row hold the same 8 scales (fragments 0..7); lane kg writes those of
    // fragments 2kg and 2kg+1 only.
    __device__ __forceinline__ void park_scales(int col, const uint32_t (&sw)[4]) const {
        // a bitwise select: a conditional chain here became a divergent branch
        // that split the block's schedule
        uint32_t s = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) s |= sw[j] & (0u - (uint32_t)(kg == j));
        dl[(32 * kg + r16) * kDlStride + col] = lo_half(s);
        dl[(32 * kg + 16 + r16) * kDlStride + col] = hi_half(s);
    }

    // One block, software-pipelined over the four dwords: the MFMAs of dword
    // p issue interleaved with the unpack of dword p + 1 (one MFMA, then a
    // few VALU instructions), so the matrix unit and the vector ALU of the
    // wave work side by side.  The FMAs that scale dword p's products run one
    // dword later, beside dword p + 1's MFMAs (the products are ready by
    // then).
    __device__ __forceinline__ void block(int blk, const uint32_t (&xw)[4], const uint32_t (&sw)[4],
                                          const half8_t (&bf)[NT], const float (&sv)[NT],
                                          float4_t (&acc)[kFrags][NT]) const {
        constexpr int kMfmas = 2 * NT;                                // per dword
        constexpr int kValu = 26 + 4 * kMfmas;                        // unpack + rescale FMAs per dword
        constexpr int kValuPer = (kValu + kMfmas - 1) / kMfmas;       // VALU instructions per MFMA slot
        const int col = blk & 31;
        half8_t a[2][2];
        float4_t t[2][2][NT];  // products of the last two dwords (fragment pair, tile)
        prepare(0, xw, sw, a[0]);
        park_scales(col, sw);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (p < 3) prepare(p + 1, xw, sw, a[(p + 1) & 1]);
            const float4_t z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                t[p & 1][0][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[p & 1][0], bf[i], z, 0, 0, 0);
                t[p & 1][1][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[p & 1][1], bf[i], z, 0, 0, 0);
            }
            if (p > 0) scale_products(p - 1, t[(p - 1) & 1], sv, acc);
#pragma unroll
            for (int k = 0; k < kMfmas; ++k) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);  // then VALU
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        scale_products(3, t[1], sv, acc);
    }

    // acc of fragments 2p, 2p+1 += block scale * products.
    __device__ __forceinline__ void scale_products(int p, const float4_t (&tp)[2][NT], const float (&sv)[NT],
                                                   float4_t (&acc)[kFrags][NT]) const {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                acc[2 * p][i][v] = fmaf(tp[0][i][v], sv[i], acc[2 * p][i][v]);
                acc[2 * p + 1][i][v] = fmaf(tp[1][i][v], sv[i], acc[2 * p + 1][i][v]);
            }
    }

    // Offset pass of 32-block chunk c: acc += um * sum_b d[row][b] u'[col][b].
    __device__ __forceinline__ void offset(int c, int nch, const _Float16* uop, const int64_t (&arow)[NT],
                                           const float (&ratio)[NT], float4_t (&acc)[kFrags][NT]) const {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        half8_t ub[NT][2];
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int64_t ar = arow[i] >= 0 ? arow[i] : 0;
            const half8_t* urow = reinterpret_cast<const half8_t*>(uop + ar * nch * 64) + 2 * kg + 8 * c;
            ub[i][0] = urow[0];
            ub[i][1] = urow[1];
        }
#pragma unroll
        for (int f = 0; f < kFrags; ++f) {
            const half8_t da = *reinterpret_cast<const half8_t*>(&dl[(16 * f + r16) * kDlStride + 8 * kg]);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                float4_t t = __builtin_amdgcn_mfma_f32_16x16x32_f16(da, ub[i][0], (float4_t){0.f, 0.f, 0.f, 0.f},
                                                                    0, 0, 0);
                t = __builtin_amdgcn_mfma_f32_16x16x32_f16(da, ub[i][1], t, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[f][i][v] = fmaf(t[v], ratio[i], acc[f][i][v]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // Records run D blocks ahead in a register ring (8 dwords per block),
    // activation fragments one block ahead in two alternating sets.  The
    // body is unrolled U blocks (D | U, U | each 32-block chunk's length);
    // with U = 8 the block scales come in 4-block batches (two sets, batch
    // (blk / 4) & 1 = j / 4), the next batch one block ahead.  Without an
    // offset operand (uop null: the Q2_0 map) there is no offset pass.
    template <int D, int U>
    __device__ __forceinline__ void run(int nch, const _Float16* uop, const int64_t (&arow)[NT],
                                        const int (&lvoff)[NT], const int (&soff)[NT], const float (&ratio)[NT],
                                        float4_t (&acc)[kFrags][NT]) const {
        static_assert(U % D == 0 && U % 2 == 0, "ring slots and activation sets are compile-time per body");
        constexpr bool kBatch = U % 8 == 0;
        uint32_t xw[D][4], sw[D][4];
        half8_t bf[2][NT];
        float sv[2][NT] = {};
        float4_t sq[2][NT] = {};
#pragma unroll
        for (int j = 0; j < D; ++j) load_record(j, xw[j], sw[j]);
        __builtin_amdgcn_sched_barrier(0);
        load_act(0, lvoff, soff, bf[0], sv[0], !kBatch);
        if constexpr (kBatch) load_scales4(0, soff, sq[0]);
        __builtin_amdgcn_sched_barrier(0);
        for (int c = 0; c < nch; ++c) {
            const int bend = nblk < 32 * c + 32 ? nblk : 32 * c + 32;
            for (int b = 32 * c; b < bend; b += U) {
#pragma unroll
                for (int j = 0; j < U; ++j) {
                    const int blk = b + j;
                    load_act(blk + 1, lvoff, soff, bf[(j + 1) & 1], sv[(j + 1) & 1], !kBatch);
                    if constexpr (kBatch)
                        if ((j & 3) == 3) load_scales4(blk + 1, soff, sq[((j >> 2) + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (kBatch) {
                        float s[NT];
#pragma unroll
                        for (int i = 0; i < NT; ++i) s[i] = sq[(j >> 2) & 1][i][j & 3];
                        block(blk, xw[j % D], sw[j % D], bf[j & 1], s, acc);
                    } else {
                        block(blk, xw[j % D], sw[j % D], bf[j & 1], sv[j & 1], acc);
                    }
                    load_record(blk + D, xw[j % D], sw[j % D]);
                }
            }
            if (uop) offset(c, nch, uop, arow, ratio, acc);
        }
    }
};

template <bool kGateUp, int NT>
__device__ __forceinline__ void small_chunk_pass(const GemmArgs& g, const Tile& tl, int slab, int t0, int lane,
                                                 _Float16* dl) {
    using Pass = SlabPass<NT, kGateUp>;  // gate/up reads its tokens' codes in place, down the tiled H
    const int r16 = lane & 15, kg = lane >> 4;
    const int nblk = g.Kd / kBlock, nch = (nblk + 31) / 32;

    // zero the d buffer: blocks past the last of a partial chunk meet u = 0
    for (int o = lane; o < kSlabRows * kDlStride / 8; o += 64)
        reinterpret_cast<half8_t*>(dl)[o] = (half8_t){0, 0, 0, 0, 0, 0, 0, 0};

    int64_t arow[NT];
    int lvoff[NT], soff[NT];
    float ratio[NT];  // the offset pass's row multipliers um
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int r = 16 * (t0 + i) + r16;
        arow[i] = -1;
        if (r < tl.nrows) arow[i] = kGateUp ? (int64_t)g.src[tl.row0 + r] : (int64_t)(tl.row0 + r);
        ratio[i] = arow[i] >= 0 && g.uop ? g.um[arow[i]] : 0.f;
        const int64_t ar = arow[i] >= 0 ? arow[i] : 0;  // padding columns read row 0, never stored
        if constexpr (kGateUp)
            lvoff[i] = (int)ar * g.Kd * 2 + 16 * kg;  // MFMA layout: column r16, group kg
        else  // tile t0 + i of the chunk in the tiled operand (padding rows are zeros, never stored)
            lvoff[i] = (tl.tile0 + t0 + i) * nblk * kTiledBlockBytes + 16 * lane;
        soff[i] = (int)ar * nblk * 4;  // scales as rows: gate/up the token's, down the grouped row's
    }
    float4_t acc[kFrags][NT];
#pragma unroll
    for (int f = 0; f < kFrags; ++f)
#pragma unroll
        for (int i = 0; i < NT; ++i) acc[f][i] = (float4_t){0.f, 0.f, 0.f, 0.f};

    const uint8_t* rec = expert_blob(g, tl.e) + (int64_t)slab * nblk * kRecordBytes;
    Pass L{__builtin_amdgcn_make_buffer_rsrc((void*)rec, (short)0, nblk * kRecordBytes, kBufferWord3),
           __builtin_amdgcn_make_buffer_rsrc((void*)g.act, (short)0, (int)(g.act_rows * g.Kd * 2), kBufferWord3),
           __builtin_amdgcn_make_buffer_rsrc((void*)g.ascale, (short)0, (int)g.scale_bytes, kBufferWord3),
           g.Kd, nblk, lane, r16, kg, dl, UnpackMagic()};
    if (nblk % 8 == 0)  // 8 | every chunk's block count: 4-block scale batches
        L.template run<2, 8>(nch, g.uop, arow, lvoff, soff, ratio, acc);
    else
        L.template run<2, 2>(nch, g.uop, arow, lvoff, soff, ratio, acc);

#pragma unroll
    for (int i = 0; i < NT; ++i) {
        float4_t a[kFrags];
#pragma unroll
        for (int f = 0; f < kFrags; ++f) a[f] = acc[f][i];
        if constexpr (kGateUp)
            gate_up_store(g, tl, slab, 16 * (t0 + i) + r16, kg, a);
        else  // the d buffer is free after the last offset pass
            down_store(g, tl, slab, t0 + i, lane, arow[i] >= 0 ? g.prow[arow[i]] : 0.f, a,
                       reinterpret_cast<float*>(dl));
    }
}

template <bool kGateUp>
__global__ void __launch_bounds__(256, 2) expert_gemm_small_kernel(GemmArgs g) {
    __shared__ _Float16 dl_all[kWaves][kSlabRows * kDlStride];
    static_assert(kSlabRows * kDlStride * sizeof(_Float16) >= 16 * kParkStride * sizeof(float),
                  "a wave's d buffer also parks one output tile");
    // workgroup -> (chunk, group of 4 slabs), all groups of a chunk on one XCD
    const int ngroups = (g.nslab + kWaves - 1) / kWaves;
    const int id = blockIdx.x;
    const int local = id >> 3;
    int lo, hi;
    chunk_range(g, &lo, &hi);
    const int chunk = lo + (local / ngroups) * 8 + (id & 7);
    if (chunk >= hi) return;
    const Tile tl = g.chunks[chunk];
    if (tl.nrows < g.min_rows) return;  // uniform: the GEMV kernel takes this chunk
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slab = kWaves * (local % ngroups) + wave;
    if (slab >= g.nslab) return;  // waves are independent: no workgroup barrier follows
    const int lane = threadIdx.x & 63;
    const int nt = (tl.nrows + 15) / 16;
    // a 3-tile chunk in one pass (the weights are unpacked once; 256 VGPRs,
    // still 2 waves per SIMD)
    if (nt == 3) {
        small_chunk_pass<kGateUp, 3>(g, tl, slab, 0, lane, dl_all[wave]);
        return;
    }
    for (int t0 = 0; t0 < nt; t0 += kSmallTiles) {
        if (nt - t0 >= 2)
            small_chunk_pass<kGateUp, 2>(g, tl, slab, t0, lane, dl_all[wave]);
        else
            small_chunk_pass<kGateUp, 1>(g, tl, slab, t0, lane, dl_all[wave]);
    }
}

// The combine: y[t] = sum_k dm[slot[t*K + k]] (rows already weighted), k in
// order, so the result does not depend on scheduling.  A workgroup covers
// kCombineThreads float4 columns of one token row (blockIdx.y picks the
// column range): each thread issues the loads of all K rows at once (the
// row slots are wave-uniform scalar loads), then adds them in k order.  The
// rows are read once, so the loads and the store bypass cache retention.
constexpr int kCombineThreads = 640;  // a 2560-wide row per workgroup (256: 165 vs 160 us at T = 8192)
__global__ void __launch_bounds__(kCombineThreads) combine_kernel(const float* __restrict__ dm,
                                                                  const int32_t* __restrict__ slot, int64_t T,
                                                                  int32_t K, int32_t H, float* __restrict__ y) {
    const int64_t t = blockIdx.x;
    const int c = blockIdx.y * kCombineThreads + threadIdx.x, n4 = H / 4;
    if (c >= n4) return;
    const int32_t* sl = slot + t * K;
    float4_t v[kMaxTopK];
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K) v[k] = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(dm + (int64_t)sl[k] * H) + c);
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kMaxTopK; ++k)
        if (k < K)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += v[k][e];
    __builtin_nontemporal_store(acc, reinterpret_cast<float4_t*>(y + t * H) + c);
}

// Dynamic LDS: the offset-pass matrix d [128][dstride] fp16, then (down only)
// 4 waves x 16 parked output rows.
inline size_t dynamic_lds_bytes(int32_t Kd, bool park) {
    const int nblk = Kd / kBlock, nch = (nblk + 31) / 32;
    size_t b = (size_t)kSlabRows * (nch * 32 + 8) * sizeof(_Float16);
    b = (b + 15) / 16 * 16;
    if (park) b += (size_t)kWaves * 16 * kParkStride * sizeof(float);
    return b;
}

inline unsigned grid_of(int64_t chunks_cap, int32_t per_chunk) {
    return (unsigned)(8 * ((chunks_cap + 7) / 8) * per_chunk);
}

// Both kernels over their own lists.  List bounds known on the host: a big
// chunk holds more than kSmallRows of the n rows; an expert with c rows has
// at most ceil(c / kChunkRows) <= c / kChunkRows + 1 chunks, and at most
// n / (kSmallRows + 1) experts have a big one; an expert has at most one
// small chunk.  Workgroups past the list's length exit at once, so a tight
// bound saves their launches.
// gs: the small-chunk kernel's arguments (its activations may differ).
// rng: a range of experts (then the bounds count its experts only) and the
// ring mapping of the blobs, or all experts resident.
void launch_gemms(GemmArgs g, GemmArgs gs_args, const ChunkLists& cl, int64_t n, int32_t E, size_t big_lds,
                  bool gate_up, hipStream_t st, const ExpertRange& rng) {
    const int32_t ne = rng.first ? rng.e1 - rng.e0 : E;  // experts this launch covers
    const int64_t by_rows = n / (kSmallRows + 1);
    const int64_t by_experts = n / kChunkRows + (ne < by_rows ? ne : by_rows);
    int64_t cap_big = cl.cap < by_rows ? cl.cap : by_rows;
    cap_big = cap_big < by_experts ? cap_big : by_experts;
    if (rng.max_rows <= kSmallRows) cap_big = 0;  // every chunk is a small one
    int64_t cap_small = cl.cap < ne ? cl.cap : ne;
    if (rng.max_rows < rng.small_min_rows) cap_small = 0;  // every chunk is the GEMV's
    for (GemmArgs* a : {&g, &gs_args}) {
        a->e0 = rng.e0;
        a->e1 = rng.e1;
        a->ring0 = rng.ring0;
        a->nring = rng.nring;
        a->min_rows = 0;
    }
    gs_args.min_rows = rng.small_min_rows;
    g.first = rng.first;                                                   // big list: row 0 of the table
    gs_args.first = rng.first ? rng.first + ((int64_t)rng.E + 1) : nullptr;  // small list: row 1
    g.chunks = cl.tiles;
    g.nchunks = cl.sched;
    if (cap_big > 0) {
        const unsigned gb = grid_of(cap_big, g.nslab);
        if (gate_up)
            hipLaunchKernelGGL(expert_gemm_kernel<true>, dim3(gb), dim3(256), big_lds, st, g);
        else
            hipLaunchKernelGGL(expert_gemm_kernel<false>, dim3(gb), dim3(256), big_lds, st, g);
    }
    gs_args.chunks = cl.tiles + cl.cap;
    gs_args.nchunks = cl.sched + 1;
    if (cap_small > 0) {
        const unsigned gs = grid_of(cap_small, (gs_args.nslab + kWaves - 1) / kWaves);
        if (gate_up)
            hipLaunchKernelGGL(expert_gemm_small_kernel<true>, dim3(gs), dim3(256), 0, st, gs_args);
        else
            hipLaunchKernelGGL(expert_gemm_small_kernel<false>, dim3(gs), dim3(256), 0, st, gs_args);
    }
}

}  // namespace

hipError_t launch_gate_up(const uint8_t* blobs, int64_t stride, const ChunkLists& cl, int64_t n, int32_t E,
                          const int32_t* src, const _Float16* xt, const float* xst, int64_t tiled_rows,
                          const _Float16* xa, const float* xs, int64_t T, const _Float16* xuop, const float* xum,
                          int32_t H, int32_t I, int8_t* hq, float* hs, hipStream_t st, const ExpertRange& rng,
                          const HTiled& ht) {
    const int64_t tiled_scale_bytes = tiled_rows / 16 * tiled_scale_stride(H / kBlock);
    GemmArgs g{blobs, stride, nullptr, nullptr, 2 * I / kSlabRows, H, src, nullptr, xt, tiled_rows, xst,
               tiled_scale_bytes, xuop, xum, I, H, hq, hs, nullptr, nullptr, 0, 0, 0, 0, 0};
    g.hbt = ht.hb;
    g.hbs = ht.hst;
    g.hu = ht.hu;
    g.huoff = ht.uoff;
    GemmArgs gs = g;
    gs.act = xa;
    gs.act_rows = T;
    gs.ascale = xs;
    gs.scale_bytes = T * (H / kBlock) * 4;
    launch_gemms(g, gs, cl, n, E, dynamic_lds_bytes(H, false), true, st, rng);
    return hipGetLastError();
}

hipError_t launch_down(const uint8_t* blobs, int64_t stride, const ChunkLists& cl, int64_t n, int32_t E,
                       const int32_t* src, const float* prow, const _Float16* hb, const float* hst,
                       int64_t tiled_rows, const float* hs, const _Float16* huop, const float* hum, int32_t H,
                       int32_t I, float* dm, hipStream_t st, const ExpertRange& rng) {
    const int64_t tiled_scale_bytes = tiled_rows / 16 * tiled_scale_stride(I / kBlock);
    const GemmArgs g{blobs, stride, nullptr, nullptr, H / kSlabRows, I, src, prow, hb, tiled_rows, hst,
                     tiled_scale_bytes, huop, hum, I, H, nullptr, nullptr, dm, nullptr, 0, 0, 0, 0, 0};
    GemmArgs gs = g;  // the small-chunk kernel reads the grouped rows' scales as rows
    gs.ascale = hs;
    gs.scale_bytes = n * (I / kBlock) * 4;
    launch_gemms(g, gs, cl, n, E, dynamic_lds_bytes(I, true), false, st, rng);
    return hipGetLastError();
}

hipError_t launch_combine(const float* dm, const int32_t* slot, int64_t T, int32_t K, int32_t H, float* y,
                          hipStream_t st) {
    if (T > 0)
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T, (unsigned)((H / 4 + kCombineThreads - 1) / kCombineThreads)),
                           dim3(kCombineThreads), 0, st, dm, slot, T, K, H, y);
    return hipGetLastError();
}

}  // namespace strata_moe
