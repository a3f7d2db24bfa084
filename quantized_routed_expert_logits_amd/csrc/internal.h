// Internal declarations shared by the host library and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace strata_moe {

constexpr int kBlock = 32;        // values per quantization block (both activations and weights)
constexpr int kChunkRows = 192;   // grouped rows per GEMM work item (12 tiles of 16 rows)
constexpr int kGroupChunk = 2048; // (token, k) pairs per grouping chunk
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 16;
constexpr int kSlabRows = 128;    // weight rows per GEMM work item (8 MFMA fragments of 16)
constexpr int kRecordCodeBytes = 1024;                    // one slab's codes of one 32-wide block
constexpr int kRecordBytes = kRecordCodeBytes + 256;      // ... plus its 128 fp16 scales
constexpr int kMaxOffsetChunks = 4;                       // reduction length <= 4 * 32 blocks = 4096

// One chunk of grouped rows: rows [row0, row0 + nrows) all belong to expert e.
// tile0: the chunk's first 16-row tile in the tiled row space (each expert's
// rows start on a whole tile there), where the down GEMM's activations live.
struct Tile {
    int32_t e, row0, nrows, tile0;
};

// Packed blob bytes of an M x Kd matrix (2 bits per weight + one fp16 per 32).
inline int64_t packed_matrix_bytes(int64_t M, int64_t Kd) { return M * Kd / 4 + M * Kd / 16; }
inline int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Upper bound of the chunk count of n grouped rows over E experts.
inline int64_t max_tiles(int64_t n, int32_t E) { return n / kChunkRows + E; }

constexpr int kSmallRows = 48;  // chunks of at most this many rows go to the small-chunk GEMM kernel
constexpr int kGemvRows = 2;     // rows per pass of the GEMV kernel
constexpr int kGemvMaxRows = 8;  // the GEMV kernel takes chunks of at most this many rows, where it runs

// The GEMMs' work lists, written on the GPU by the grouping (or from given
// offsets): tiles[0, cap) the chunks of more than kSmallRows rows, tiles[cap,
// 2 cap) the others; sched[0], sched[1] their counts; sched[2] the number of
// 16-row tiles of the tiled row space, trows[t] tile t's grouped rows.
constexpr int kSchedInts = 3;
struct TileRows {
    int32_t row0, nrows;  // grouped rows [row0, row0 + nrows), nrows <= 16
    int32_t big;          // 1 if the tile's chunk has more than kSmallRows rows
};
struct ChunkLists {
    Tile* tiles;      // [2 * cap]
    int32_t* sched;   // [kSchedInts]
    int64_t cap;
    TileRows* trows;  // [tiled_rows_cap / 16]
    // [3][E + 1] or null: per expert e (and e = E: the totals) the index of
    // its first chunk in the big list, in the small list, and its first tile
    // of the tiled row space.  The lists and the tiles run in expert order,
    // so experts [e0, e1) own entries [first[e0], first[e1]) of each.
    int32_t* first;
};
inline int64_t first_table_ints(int32_t E) { return 3 * ((int64_t)E + 1); }

// The experts one GEMM or tile launch covers: all of them (first == null),
// or the range [e0, e1) through the ChunkLists first table of a grouping over
// E experts; and where expert e's blob is: blobs + e * stride, or with
// nring > 0 in slot (ring0 + e) % nring of a ring of streamed experts
// (blobs + slot * stride).
struct ExpertRange {
    const int32_t* first = nullptr;
    int32_t E = 0, e0 = 0, e1 = 0;
    int64_t ring0 = 0;
    int32_t nring = 0;
    int32_t small_min_rows = 0;  // the small-chunk MFMA kernel skips chunks below this (the GEMV's)
    // No expert has more rows than this in the call (the layer: T, since a
    // token picks an expert at most once).  A kernel whose chunks cannot
    // exist under it is not launched.
    int64_t max_rows = INT64_MAX;
};
inline int64_t chunk_list_cap(int64_t n, int32_t E) { return max_tiles(n, E); }

// Rows of the tiled row space: every expert's rows rounded up to whole 16-row
// tiles, so at most n + 15 E (a multiple of 16 after rounding up).
inline int64_t tiled_rows_cap(int64_t n, int32_t E) { return (n + 15 * (int64_t)E + 15) / 16 * 16; }

// Floats of the down GEMM's tiled block scales (launch_tile_h): per 16-row
// tile, ceil(I / 128) groups of 16 rows x 4 blocks.
inline int64_t tiled_h_scale_floats(int64_t n, int32_t E, int32_t I) {
    return tiled_rows_cap(n, E) * ((I / kBlock + 3) / 4) * 4;
}

// fp16 values per row of the offset-pass operand of a reduction length Kd:
// 32-block chunks, hi and lo per block.
inline int64_t offset_operand_halves(int32_t Kd) { return (int64_t)((Kd / kBlock + 31) / 32) * 64; }

// ---- launchers; each returns hipGetLastError() after its launches.
// Up to two int32 words the quantize kernel sets to 0 (a call's flags), or null.
struct ZeroWords {
    int32_t* p[2];
};
hipError_t launch_quantize(const float* v, int64_t rows, int32_t cols, int8_t* q8, float* s, hipStream_t st,
                           ZeroWords z = ZeroWords{{nullptr, nullptr}});
// Per int8 row: the codes q themselves as fp16 (exact), [rows][cols], if out
// is non-null; the row multipliers 2^e_r (127 * the row's largest
// block scale in [2^14, 2^15) after scaling by 2^-e_r) in mult if non-null;
// the offset-pass operand (u = -uoff * s * (block code sum) per block, hi/lo,
// [rows][offset_operand_halves]) and its row multipliers, if uop is non-null.
// uoff = 0.5 for the symmetric weight map w = d (q - 1.5); Q2_0's
// w = d (q - 1) has no offset operand (the GEMMs multiply by d (q - 1), the
// offset pass adds the rest).
hipError_t launch_prescale(const int8_t* q, const float* s, int64_t rows, int32_t cols, float uoff, _Float16* out,
                           float* mult, _Float16* uop, float* umult, hipStream_t st);
// The down GEMM operand of the grouped rows in the tiled layout: tile t of
// the chunk lists' tile table holds grouped rows trows[t]; out = their int8
// codes q as fp16 (exact) in [tile][block][group g of 8 values][row within
// the tile][8] (one MFMA fragment of a tile and block is 1 KiB in MFMA lane
// order; rows past a tile's nrows are zero), sout = their block scales
// [tile][ceil(blocks / 4)][row within the tile][4] (zero padded).  uop, umult
// as launch_prescale, per grouped row (skipped when uop is null).
// tiles_cap bounds the tile count (the grid).
// With rng.first set, only the tiles of experts [rng.e0, rng.e1).
hipError_t launch_tile_h(const int8_t* q, const float* s, const ChunkLists& cl, int64_t tiles_cap, int32_t cols,
                         float uoff, _Float16* out, float* sout, _Float16* uop, float* umult, hipStream_t st,
                         const ExpertRange& rng = ExpertRange());
// The 4-wave gate/up kernel's operand in the tiled layout: tile t of the
// chunk lists' tile table (tiles of chunks of more than kSmallRows rows only)
// holds grouped rows trows[t], each the token src[row] of the int8 rows q
// [tokens][cols] with block scales s; out = [tile][block][group g of 8
// values][row within the tile][8] fp16 codes (exact), sout = [tile][block /
// 4][row within the tile][4] block scales; rows past a tile's nrows are
// zeros.  tiles_cap bounds the tile count.
hipError_t launch_gather_tiles(const int8_t* q, const float* s, const int32_t* src, const ChunkLists& cl,
                               int64_t tiles_cap, int32_t cols, _Float16* out, float* sout, hipStream_t st);
// The layer input in one pass: launch_quantize's outputs (q8, s) and
// launch_prescale's (codes16, mult, uop, umult), bit-identical to
// the two launches, and each row's Euclidean norm xn (fp32); also clears the
// ZeroWords.
hipError_t launch_quantize_prescale(const float* x, int64_t rows, int32_t cols, float uoff, int8_t* q8, float* s,
                                   _Float16* codes16, float* mult, float* xn, _Float16* uop, float* umult,
                                   hipStream_t st, ZeroWords z);
hipError_t launch_fill_zero(float* p, int64_t count, hipStream_t st);

// Router scratch: wt [E][H] fp32 (transposed weight, also read by the top-K
// re-score), wb [Ep][H][2] fp16 (its hi/lo form in MFMA fragment order, Ep =
// router_padded_experts(E)), wm [Ep], wnorm [1] (the largest Euclidean norm
// of a router column), xm [T] and xn [T] (input row multipliers and norms,
// used when the caller passes none), pmax [H/32][E] (column maxima of 32-row
// tiles of the weight).
struct RouterScratch {
    float* wt;
    _Float16* wb;
    float* wm;
    float* wnorm;
    float* xm;
    float* xn;
    float* pmax;
};
// The router GEMM splits the reduction over H into router_splits() ranges
// until the launch has 512 workgroups (2 per CU) or 8 ranges; logits then
// holds that many partial [T][E] arrays, which the top-K adds in order.
constexpr int kMaxRouterSplits = 8;
inline int router_splits(int64_t T, int32_t H, int32_t E) {
    const int64_t nk = H / 32, wgs = ((T + 63) / 64) * ((E + 127) / 128);
    int s = 1;
    while (s < kMaxRouterSplits && wgs * s < 512 && nk % (4 * s) == 0) s *= 2;
    return s;
}
inline int64_t router_logit_floats(int64_t T, int32_t H, int32_t E) { return router_splits(T, H, E) * T * E; }
inline int64_t router_padded_experts(int32_t E) { return round_up(E, 16); }

// logits [splits][T][E]; xm: the input rows' power-of-two multipliers (the
// prescale's row multipliers of the same rows) or nullptr to compute them.
// wr == nullptr: rs.wt / rs.wb / rs.wm already hold wr's prepared forms
// (launch_router_prep); otherwise they are prepared here (rs.pmax: scratch of
// H/32 x E floats).
// When xm is null the rows' multipliers and norms are computed into rs.xm
// and rs.xn.
hipError_t launch_router(const float* x, const float* xm, const float* wr, const float* bias, int64_t T, int32_t H,
                         int32_t E, const RouterScratch& rs, float* logits, hipStream_t st);
// The router matrix's per-call forms: the transposed fp32 copy rs.wt [E][H]
// and the hi/lo fp16 operand rs.wb / rs.wm (rs.pmax: scratch).
hipError_t launch_router_prep(const float* wr, int32_t H, int32_t E, const RouterScratch& rs, hipStream_t st);
// Byte offsets of the prepared router matrix's parts in one buffer.
struct RouterPrepared {
    size_t wt, wb, wm, wnorm, pmax, total;
};
inline RouterPrepared router_prepared_layout(int32_t H, int32_t E) {
    RouterPrepared r;
    const int64_t Ep = router_padded_experts(E);
    auto take = [](size_t& off, size_t bytes) {
        const size_t at = off;
        off += (bytes + 255) / 256 * 256;
        return at;
    };
    size_t off = 0;
    r.wt = take(off, (size_t)E * H * sizeof(float));
    r.wb = take(off, (size_t)Ep * H * 2 * sizeof(_Float16));
    r.wm = take(off, (size_t)Ep * sizeof(float));
    r.wnorm = take(off, sizeof(float));
    r.pmax = take(off, (size_t)((H + 31) / 32) * E * sizeof(float));
    r.total = off;
    return r;
}
// xn: the input rows' Euclidean norms, wnorm: the router columns' largest
// (the near-tie window's error bound); wt from the router scratch (the fp64
// re-score of near-tie tokens reads expert columns as rows of it).
hipError_t launch_topk(const float* logits, const float* x, const float* xn, const float* wt, const float* wnorm,
                       const float* bias, int64_t T, int32_t H, int32_t E, int32_t K, int32_t* ids, float* p,
                       hipStream_t st);

// The shared expert's pair slot: ids / p [T][K] copied to gids / gp [T][K+1]
// with slot K = (E, sigmoid(x[t] . wg)).  x, wg 16-byte aligned; H % 128 == 0.
hipError_t launch_shared_slot(const float* x, const float* wg, const int32_t* ids, const float* p, int64_t T,
                              int32_t H, int32_t K, int32_t E, int32_t* gids, float* gp, hipStream_t st);

hipError_t launch_group(const int32_t* ids, const float* p, int64_t n, int32_t K, int32_t E, int32_t* hist,
                        int32_t* base, int32_t* offsets, const ChunkLists& cl, int32_t* src, int32_t* slot,
                        float* prow, int32_t* err, hipStream_t st);
hipError_t launch_chunks_from_offsets(const int32_t* offsets, int32_t E, int64_t n, const ChunkLists& cl,
                                      hipStream_t st);
hipError_t launch_row_weights(const int32_t* slot, const float* p, int64_t n, float* prow, hipStream_t st);

// gate/up: xt / xst = the tiled codes and scales (launch_gather_tiles,
// tiled_rows rows) for the 4-wave kernel; xa = the input codes as fp16
// (launch_prescale) and xs = their block scales, T rows each, for the small-
// chunk kernel; xuop / xum = offset-pass operand and multipliers (xuop null:
// none); writes int8
// H codes hq and scales hs.
// n = routed rows, E = experts (bounds of the two chunk lists' lengths).
// Optionally the MFMA kernels' epilogue also writes the down GEMM's operand
// for their chunks, as launch_tile_h would from hq / hs: hb and hst (tiled
// codes and scales, padding rows zero) and, if hu is non-null, each block's
// u = -uoff * scale * (code sum) as floats [rows][offset_operand_halves / 2]
// (hu aliases the offset operand uop, which launch_offset_rows then builds
// in place).  With hb set, hq may be null: the MFMA kernels then write no
// int8 H codes (the GEMV's chunks still get theirs from the GEMV launch).
struct HTiled {
    _Float16* hb = nullptr;
    float* hst = nullptr;
    float* hu = nullptr;
    float uoff = 0.f;
};
hipError_t launch_gate_up(const uint8_t* blobs, int64_t stride, const ChunkLists& cl, int64_t n, int32_t E,
                          const int32_t* src, const _Float16* xt, const float* xst, int64_t tiled_rows,
                          const _Float16* xa, const float* xs, int64_t T, const _Float16* xuop, const float* xum,
                          int32_t H, int32_t I, int8_t* hq, float* hs, hipStream_t st,
                          const ExpertRange& rng = ExpertRange(), const HTiled& ht = HTiled());
// The offset operand of rows [0, n) in place: hu holds each row's block
// values u (floats, row stride offset_operand_halves(cols) / 2, as HTiled
// writes them); each row becomes its hi/lo fp16 operand (the layout of
// launch_prescale's uop) with its multiplier in umult, bit-identical to
// launch_tile_h's.  Rows no kernel wrote get meaningless values.
hipError_t launch_offset_rows(float* hu, int64_t n, int32_t cols, float* umult, hipStream_t st);
// down: hb / hst = the tiled H codes and block scales (launch_tile_h) for
// the 4-wave kernel (tiled_rows rows), hs = the grouped rows' block scales
// [n][I/32] for the small-chunk kernel (which reads its codes from hb too),
// huop / hum = offset-pass operand and multipliers (huop null: none); writes
// the weighted rows dm.
hipError_t launch_down(const uint8_t* blobs, int64_t stride, const ChunkLists& cl, int64_t n, int32_t E,
                       const int32_t* src, const float* prow, const _Float16* hb, const float* hst,
                       int64_t tiled_rows, const float* hs, const _Float16* huop, const float* hum, int32_t H,
                       int32_t I, float* dm, hipStream_t st, const ExpertRange& rng = ExpertRange());
// The small-T GEMV over the small-chunk list's chunks of at most max_rows
// (<= kGemvMaxRows) rows, kGemvRows per pass (gate_up: activations act [act_rows][H] int8 by token through src, or
// with asum by grouped row in the per-slot q8_1 form; writes hq / hs.  down:
// act = H codes [n][I] by grouped row; writes the weighted rows y).
struct GemvLaunch {
    bool gate_up;
    const uint8_t* blobs;
    int64_t stride;
    const int32_t* src;
    const int8_t* act;
    int64_t act_rows;
    const float* ascale;
    const int32_t* asum;
    int32_t sym;
    const float* prow;
    int32_t H, I;
    int8_t* hq;
    float* hs;
    float* y;
    int32_t max_rows;
};
hipError_t launch_gemv(const GemvLaunch& l, const ChunkLists& cl, int64_t n, int32_t E, const ExpertRange& rng,
                       hipStream_t st);
// The per-slot q8_1 form of the layer input (the pages' MMQ path quantizes
// each routed slot's row): row r of q8 / s / sum is x[src[r]] rounded as
// launch_quantize rounds it (the same codes), with the block code sums.
hipError_t launch_quantize_slots(const float* x, const int32_t* src, int64_t n, int32_t cols, int8_t* q8, float* s,
                                 int32_t* sum, hipStream_t st);

hipError_t launch_combine(const float* dm, const int32_t* slot, int64_t T, int32_t K, int32_t H, float* y,
                          hipStream_t st);

hipError_t launch_pack(const uint8_t* codes, const uint16_t* scales, int32_t nexp, int32_t M, int32_t Kd,
                       int32_t gate_up_I, uint8_t* dst, int64_t stride, hipStream_t st);
hipError_t launch_unpack(const uint8_t* src, int64_t stride, int32_t nexp, int32_t M, int32_t Kd, int32_t gate_up_I,
                         uint8_t* codes, uint16_t* scales, hipStream_t st);

}  // namespace strata_moe
