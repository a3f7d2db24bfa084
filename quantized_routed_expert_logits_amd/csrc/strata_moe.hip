// Host side of libstrata_moe: argument checks, the device workspace, the
// launch sequence of one layer call, the single-step entry points and the
// per-kernel event timing.  All launches go on the caller's stream; nothing
// here waits for the GPU except strata_moe_group (its id check) and
// strata_moe_timing_read.
//
// The sequence follows the MoE half of Prefill::run (Winery-Strata
// prefill.cpp page) on the fused path of moe_fused.hpp (Strata compare
// v0.1.35...v0.1.37 page): router -> route -> int8 activations once per
// token -> grouping on the GPU -> experts -> combine.  The down GEMM applies
// each routed row's weight and writes the row to its grouped slot; the combine
// then adds every token's K rows in k order (deterministic).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/strata_moe.h"
#include "internal.h"

using namespace strata_moe;

// A ring of device slots through which the experts of layer calls stream
// from pinned host memory (Winery-Strata prefill.cpp page: the streamed
// ring's commentary at the top of the file and the fused batch loop of
// Prefill::run).  Entry k of the stream (a running count over calls) goes to
// slot k % n_slots; copied[s] is recorded on the copy stream after the DMA
// into slot s, used[s] on the compute stream after the last launch that
// reads it, and a DMA into a slot waits for the slot's used event.
struct strata_moe_ring {
    int device = 0;
    int32_t n_slots = 0, hidden = 0, ffn = 0;
    int64_t slot_bytes = 0;  // one expert: gate/up blob, then down blob
    int64_t gate_up_bytes = 0;
    char* slots = nullptr;   // caller-owned device memory
    hipStream_t copy = nullptr;
    std::vector<hipEvent_t> copied, used;
    std::vector<char> used_recorded;
    int64_t next = 0;        // entries streamed by earlier calls
};

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(STRATA_MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                        \
    do {                                           \
        hipError_t e_ = (expr);                    \
        if (e_ != hipSuccess) return hip_fail(e_, what); \
    } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ----------------------------------------------------------------- device
int check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(STRATA_MOE_EUNSUPPORTED, "no HIP device");
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(STRATA_MOE_EUNSUPPORTED, "no HIP device");
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(STRATA_MOE_EUNSUPPORTED, "device %d is %s; this library is built for gfx950 only", dev,
                    prop.gcnArchName);
    return 0;
}

// -------------------------------------------------------------- workspace
struct Workspace {
    void* owned = nullptr;
    size_t owned_bytes = 0;
    void* user = nullptr;
    size_t user_bytes = 0;
};
std::mutex g_ws_mu;
Workspace g_ws[64];

int get_workspace(size_t need, char** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(STRATA_MOE_EINVAL, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_ws_mu);
    Workspace& w = g_ws[dev];
    if (w.user) {
        if (w.user_bytes < need)
            return fail(STRATA_MOE_ENOMEM, "workspace of %zu bytes set, %zu needed", w.user_bytes, need);
        *out = (char*)w.user;
        return 0;
    }
    if (w.owned_bytes < need) {
        if (w.owned) {
            HIP_TRY(hipDeviceSynchronize(), "hipDeviceSynchronize");
            HIP_TRY(hipFree(w.owned), "hipFree");
            w.owned = nullptr;
            w.owned_bytes = 0;
        }
        const size_t bytes = (size_t)round_up((int64_t)need, 1 << 20);
        if (hipMalloc(&w.owned, bytes) != hipSuccess) {
            w.owned = nullptr;
            return fail(STRATA_MOE_ENOMEM, "hipMalloc of %zu workspace bytes failed", bytes);
        }
        w.owned_bytes = bytes;
    }
    *out = (char*)w.owned;
    return 0;
}

// Carves the workspace of one layer call.  Every region is 256-byte aligned.
struct Layout {
    size_t off = 0;
    template <typename T>
    size_t take(int64_t count) {
        const size_t at = off;
        off += (size_t)round_up((int64_t)sizeof(T) * (count > 0 ? count : 1), 256);
        return at;
    }
};

struct Buffers {
    float* logits;
    float* wt;
    _Float16* wb;
    float* wm;
    float* wnorm;
    float* pmax;
    int32_t* ids;   // the routing: [T][K]
    float* p;
    int32_t* gids;  // the grouped pairs: [T][K+1] with a shared expert, else ids / p
    float* gp;
    int8_t* xq;
    float* xs;
    _Float16* xa;  // the input codes as fp16 [T][H] (small-chunk gate/up kernel)
    _Float16* xt;  // tiled gate/up operand of big chunks' rows: fp16 codes
    float* xst;    // and their tiled block scales
    float* xe;
    float* xn;     // the input rows' Euclidean norms (the router's near-tie window)
    _Float16* xuop;
    float* xum;
    int32_t* hist;
    int32_t* base;
    int32_t* offsets;
    Tile* tiles;
    int32_t* ntiles;
    int32_t* first;  // per-expert first chunk / tile table of the grouping
    int32_t* err;
    int32_t* src;
    int32_t* slot;
    float* prow;
    int8_t* hq;
    float* hs;
    TileRows* trows;
    _Float16* hb;   // tiled H codes (fp16) and their tiled block scales: the down GEMM's operand
    float* hst;
    _Float16* huop;
    float* hum;
    float* dm;
    int8_t* sq;    // per-slot q8_1 arm: the layer input per grouped row, its scales and block code sums
    float* ss;
    int32_t* ssum;
    int64_t tiles_cap;
};

struct Offsets {
    size_t logits, wt, wb, wm, wnorm, pmax, ids, p, gids, gp, xq, xs, xa, xt, xst, xe, xn, xuop, xum, hist, base, offsets, tiles, ntiles, first, err, src, slot, prow, hq, hs,
        trows, hb, hst, huop, hum, dm, sq, ss, ssum, total;
    int64_t tiles_cap;
};

// K, E: the routing's; with a shared expert the grouping and the expert GEMMs
// run over K + 1 pairs per token and E + 1 experts.
Offsets plan(int64_t T, int32_t K, int32_t E, int32_t H, int32_t I, bool shared, bool per_slot) {
    const int64_t nr = T * K;
    const int32_t Er = E;
    if (shared) ++K, ++E;
    const int64_t n = T * K;
    const int64_t nchunks = (n + kGroupChunk - 1) / kGroupChunk;
    Layout L;
    Offsets o;
    o.tiles_cap = chunk_list_cap(n, E);
    o.logits = L.take<float>(router_logit_floats(T, H, Er));
    o.wt = L.take<float>((int64_t)Er * H);
    o.wb = L.take<_Float16>(router_padded_experts(Er) * H * 2);
    o.wm = L.take<float>(router_padded_experts(Er));
    o.wnorm = L.take<float>(1);
    o.pmax = L.take<float>((int64_t)((H + 31) / 32) * Er);
    o.ids = L.take<int32_t>(nr);
    o.p = L.take<float>(nr);
    o.gids = shared ? L.take<int32_t>(n) : o.ids;
    o.gp = shared ? L.take<float>(n) : o.p;
    o.xq = L.take<int8_t>(T * H);
    o.xs = L.take<float>(T * (H / kBlock));
    o.xe = L.take<float>(T);
    o.xn = L.take<float>(T);
    o.xuop = L.take<_Float16>(T * offset_operand_halves(H));
    o.xum = L.take<float>(T);
    o.hist = L.take<int32_t>(nchunks * E);
    o.base = L.take<int32_t>(nchunks * E);
    o.offsets = L.take<int32_t>(E + 1);
    o.tiles = L.take<Tile>(2 * o.tiles_cap);
    o.ntiles = L.take<int32_t>(kSchedInts);
    o.first = L.take<int32_t>(first_table_ints(E));
    o.err = L.take<int32_t>(1);
    o.src = L.take<int32_t>(n);
    o.slot = L.take<int32_t>(n);
    o.prow = L.take<float>(n);
    o.hq = L.take<int8_t>(n * I);
    o.hs = L.take<float>(n * (I / kBlock));
    o.trows = L.take<TileRows>(tiled_rows_cap(n, E) / 16);
    o.xa = L.take<_Float16>(T * H);
    o.xt = L.take<_Float16>(tiled_rows_cap(n, E) * H);
    o.xst = L.take<float>(tiled_rows_cap(n, E) * (H / kBlock));
    o.hb = L.take<_Float16>(tiled_rows_cap(n, E) * I);
    o.hst = L.take<float>(tiled_h_scale_floats(n, E, I));
    o.huop = L.take<_Float16>(n * offset_operand_halves(I));
    o.hum = L.take<float>(n);
    o.dm = L.take<float>(n * H);
    o.sq = per_slot ? L.take<int8_t>(n * H) : o.dm;
    o.ss = per_slot ? L.take<float>(n * (H / kBlock)) : o.dm;
    o.ssum = per_slot ? L.take<int32_t>(n * (H / kBlock)) : o.dm;
    o.total = L.off;
    return o;
}

Buffers carve(char* ws, const Offsets& o) {
    Buffers b;
    b.logits = (float*)(ws + o.logits);
    b.wt = (float*)(ws + o.wt);
    b.wb = (_Float16*)(ws + o.wb);
    b.wm = (float*)(ws + o.wm);
    b.wnorm = (float*)(ws + o.wnorm);
    b.pmax = (float*)(ws + o.pmax);
    b.ids = (int32_t*)(ws + o.ids);
    b.p = (float*)(ws + o.p);
    b.gids = (int32_t*)(ws + o.gids);
    b.gp = (float*)(ws + o.gp);
    b.xq = (int8_t*)(ws + o.xq);
    b.xs = (float*)(ws + o.xs);
    b.xa = (_Float16*)(ws + o.xa);
    b.xt = (_Float16*)(ws + o.xt);
    b.xst = (float*)(ws + o.xst);
    b.xe = (float*)(ws + o.xe);
    b.xn = (float*)(ws + o.xn);
    b.xuop = (_Float16*)(ws + o.xuop);
    b.xum = (float*)(ws + o.xum);
    b.hist = (int32_t*)(ws + o.hist);
    b.base = (int32_t*)(ws + o.base);
    b.offsets = (int32_t*)(ws + o.offsets);
    b.tiles = (Tile*)(ws + o.tiles);
    b.ntiles = (int32_t*)(ws + o.ntiles);
    b.first = (int32_t*)(ws + o.first);
    b.err = (int32_t*)(ws + o.err);
    b.src = (int32_t*)(ws + o.src);
    b.slot = (int32_t*)(ws + o.slot);
    b.prow = (float*)(ws + o.prow);
    b.hq = (int8_t*)(ws + o.hq);
    b.hs = (float*)(ws + o.hs);
    b.trows = (TileRows*)(ws + o.trows);
    b.hb = (_Float16*)(ws + o.hb);
    b.hst = (float*)(ws + o.hst);
    b.huop = (_Float16*)(ws + o.huop);
    b.hum = (float*)(ws + o.hum);
    b.dm = (float*)(ws + o.dm);
    b.sq = (int8_t*)(ws + o.sq);
    b.ss = (float*)(ws + o.ss);
    b.ssum = (int32_t*)(ws + o.ssum);
    b.tiles_cap = o.tiles_cap;
    return b;
}

// ----------------------------------------------------------------- timing
enum Kind { kQuantize, kRouter, kTopK, kGroup, kGateUp, kTileH, kDown, kCombine, kStreamed, kNumKinds };
const char* const kKindNames[kNumKinds] = {"quantize", "router_gemm", "topk",    "group",           "gate_up",
                                           "tile_h",   "down",        "combine", "streamed_experts"};

struct Timing {
    bool on = false;
    int max_calls = 0;
    int used = 0;
    std::vector<hipEvent_t> ev;   // [max_calls][kinds][2]
    std::vector<char> recorded;   // [max_calls][kinds]
};
std::mutex g_tm_mu;
Timing g_tm;

struct CallTimer {
    int call = -1;
    hipStream_t st;
    explicit CallTimer(hipStream_t s) : st(s) {
        std::lock_guard<std::mutex> lock(g_tm_mu);
        if (g_tm.on && g_tm.used < g_tm.max_calls) call = g_tm.used++;
    }
    void begin(Kind k) {
        if (call >= 0) hipEventRecord(g_tm.ev[((size_t)call * kNumKinds + k) * 2], st);
    }
    void end(Kind k) {
        if (call >= 0) {
            hipEventRecord(g_tm.ev[((size_t)call * kNumKinds + k) * 2 + 1], st);
            g_tm.recorded[(size_t)call * kNumKinds + k] = 1;
        }
    }
};

// ------------------------------------------------------------- validation
#define TRY(expr)                 \
    do {                          \
        int rc_ = (expr);         \
        if (rc_ != 0) return rc_; \
    } while (0)

// H: 128-row slabs of the down matrix; I: 64-row slabs of gate and of up;
// both <= 4096 (the offset pass covers at most 128 blocks).
int check_dims(int32_t hidden, int32_t ffn) {
    if (hidden < 128 || hidden % 128 || hidden > 4096)
        return fail(STRATA_MOE_EINVAL, "hidden %d is not a multiple of 128 in [128, 4096]", hidden);
    if (ffn < 64 || ffn % 64 || ffn > 4096)
        return fail(STRATA_MOE_EINVAL, "ffn %d is not a multiple of 64 in [64, 4096]", ffn);
    return 0;
}

int check_experts(const strata_moe_experts* ex) {
    if (!ex) return fail(STRATA_MOE_EINVAL, "experts is NULL");
    if (ex->format != STRATA_MOE_Q2_SYM && ex->format != STRATA_MOE_Q2_0)
        return fail(STRATA_MOE_EUNSUPPORTED, "unknown weight format %d", ex->format);
    if (ex->n_expert < 1 || ex->n_expert > kMaxExperts)
        return fail(STRATA_MOE_EINVAL, "n_expert %d outside [1, %d]", ex->n_expert, kMaxExperts);
    TRY(check_dims(ex->hidden, ex->ffn));
    if (!ex->gate_up || !ex->down) return fail(STRATA_MOE_EINVAL, "expert blob pointer is NULL");
    const int64_t gu = round_up(packed_matrix_bytes(2LL * ex->ffn, ex->hidden), 256);
    const int64_t dn = round_up(packed_matrix_bytes(ex->hidden, ex->ffn), 256);
    if (ex->gate_up_stride < gu || ex->down_stride < dn)
        return fail(STRATA_MOE_EINVAL, "expert strides (%lld, %lld) below the packed sizes (%lld, %lld)",
                    (long long)ex->gate_up_stride, (long long)ex->down_stride, (long long)gu, (long long)dn);
    if (ex->gate_up_stride % 256 || ex->down_stride % 256 || !aligned(ex->gate_up, 256) || !aligned(ex->down, 256))
        return fail(STRATA_MOE_EINVAL, "expert blobs and strides must be 256-byte aligned");
    if (ex->router_prepared && !aligned(ex->router_prepared, 256))
        return fail(STRATA_MOE_EINVAL, "router_prepared must be 256-byte aligned");
    if (ex->shared_gate && !aligned(ex->shared_gate, 16))
        return fail(STRATA_MOE_EINVAL, "shared_gate must be 16-byte aligned");
    if (ex->flags & ~(STRATA_MOE_FLAG_NO_GEMV | STRATA_MOE_FLAG_PER_SLOT_Q8 | STRATA_MOE_FLAG_GEMV_ALWAYS))
        return fail(STRATA_MOE_EINVAL, "unknown flags 0x%x", ex->flags);
    if (ex->shared_gate && ex->n_expert + 1 > kMaxExperts)
        return fail(STRATA_MOE_EINVAL, "n_expert %d leaves no room for the shared expert (at most %d)", ex->n_expert,
                    kMaxExperts - 1);
    return 0;
}

// The GEMMs multiply by d (q - 1); the offset pass adds -uoff * d * s * (block
// code sum) for the rest of the weight map's offset: 0.5 for w = d (q - 1.5),
// 0 for Q2_0's w = d (q - 1), which has no offset pass.
float code_offset(const strata_moe_experts* ex) { return ex->format == STRATA_MOE_Q2_0 ? 0.0f : 0.5f; }
bool has_offset(const strata_moe_experts* ex) { return code_offset(ex) != 0.0f; }

// The GEMMs address activations with 32-bit buffer offsets: their tiled
// operands (T*K rows and up to 15 padding rows per expert, [.][H] and [.][I]
// fp16) must each stay below 2 GiB; so must x.
int check_buffers(int64_t T, int32_t K, int32_t E, int32_t H, int32_t I) {
    const int64_t rows = tiled_rows_cap(T * K, E), lim = (int64_t)1 << 31;
    if (T * (int64_t)H * 4 >= lim || rows * H * 2 >= lim || rows * I * 2 >= lim)
        return fail(STRATA_MOE_EINVAL, "T = %lld too large for one call at H = %d, I = %d, K = %d", (long long)T, H, I,
                    K);
    return 0;
}

int check_tk(int64_t T, int32_t K, int32_t E) {
    if (T < 0) return fail(STRATA_MOE_EINVAL, "T = %lld is negative", (long long)T);
    if (K < 1 || K > kMaxTopK) return fail(STRATA_MOE_EINVAL, "K = %d outside [1, %d]", K, kMaxTopK);
    if (K > E) return fail(STRATA_MOE_EINVAL, "K = %d exceeds the %d experts", K, E);
    if (T * (int64_t)K >= (int64_t)1 << 31) return fail(STRATA_MOE_EINVAL, "T*K = %lld too large", (long long)(T * K));
    return 0;
}

// A layer call's sizes: the routing's K of E, then the grouped pairs (K + 1 of
// E + 1 with a shared expert).
int check_layer(int64_t T, int32_t K, const strata_moe_experts* ex) {
    TRY(check_experts(ex));
    TRY(check_tk(T, K, ex->n_expert));
    const int32_t sh = ex->shared_gate ? 1 : 0;
    if (K + sh > kMaxTopK)
        return fail(STRATA_MOE_EINVAL, "K = %d leaves no pair slot for the shared expert (at most %d)", K,
                    kMaxTopK - 1);
    if (T * (int64_t)(K + sh) >= (int64_t)1 << 31)
        return fail(STRATA_MOE_EINVAL, "T*(K+1) = %lld too large", (long long)(T * (K + sh)));
    return check_buffers(T, K + sh, ex->n_expert + sh, ex->hidden, ex->ffn);
}

// The layer zeroes `out` before its router reads `x`: the two must not overlap.
int check_no_overlap(const void* a, const void* b, int64_t bytes) {
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    if (pa < pb + (uintptr_t)bytes && pb < pa + (uintptr_t)bytes)
        return fail(STRATA_MOE_EINVAL, "out overlaps x");
    return 0;
}

// The GEMV takes the small-chunk list's chunks of at most this many rows (0:
// none).  It runs where the experts get at most two rows each on average
// (n <= 2 E): there nearly every chunk is that short, and the MFMA kernel
// left with the few longer ones costs one slab's pass in time however few
// they are.  At larger averages the MFMA kernels take everything: there the
// GEMV's passes (two rows each) cost more than the MFMA's one.
int32_t gemv_rows(const strata_moe_experts* ex, int64_t n, int32_t Eg) {
    if (ex->flags & STRATA_MOE_FLAG_NO_GEMV) return 0;
    if ((ex->flags & STRATA_MOE_FLAG_GEMV_ALWAYS) || n <= 2 * (int64_t)Eg) return kGemvMaxRows;
    return 0;
}
bool per_slot_q8(const strata_moe_experts* ex, int64_t n, int32_t Eg) {
    return gemv_rows(ex, n, Eg) > 0 && (ex->flags & STRATA_MOE_FLAG_PER_SLOT_Q8);
}
// The small-chunk MFMA kernel's lower row bound beside the GEMV.
int32_t small_min_rows(const strata_moe_experts* ex, int64_t n, int32_t Eg) {
    const int32_t g = gemv_rows(ex, n, Eg);
    return g > 0 ? g + 1 : 0;
}

// The GEMV launches of the experts in rng (gate/up, or down), beside the MFMA
// kernels of the same range: the small-chunk list's chunks of at most
// gemv_rows() rows.
int launch_gemv_step(const strata_moe_experts* ex, bool gate_up, const uint8_t* blobs, int64_t stride,
                     const Buffers& b, const ChunkLists& cl, int64_t T, int64_t n, int32_t Eg, const ExpertRange& rng,
                     hipStream_t st) {
    const int32_t rows = gemv_rows(ex, n, Eg);
    if (rows == 0) return 0;
    GemvLaunch l{};
    l.max_rows = rows;
    l.gate_up = gate_up;
    l.blobs = blobs;
    l.stride = stride;
    l.sym = ex->format == STRATA_MOE_Q2_SYM ? 1 : 0;
    l.H = ex->hidden;
    l.I = ex->ffn;
    if (gate_up) {
        const bool ps = per_slot_q8(ex, n, Eg);
        l.src = b.src;
        l.act = ps ? b.sq : b.xq;
        l.act_rows = ps ? n : T;
        l.ascale = ps ? b.ss : b.xs;
        l.asum = ps ? b.ssum : nullptr;
        l.hq = b.hq;
        l.hs = b.hs;
    } else {
        l.act = b.hq;
        l.act_rows = n;
        l.ascale = b.hs;
        l.prow = b.prow;
        l.y = b.dm;
    }
    HIP_TRY(launch_gemv(l, cl, n, Eg, rng, st), "GEMV launch");
    return 0;
}

// The expert phase with every expert streamed through the ring: batches of
// at most a third of the ring in expert id order; each batch waits for its
// last DMA, runs gate/up, the tiled H and down on its experts' rows, and
// gives its slots back (used events), which lets the next DMAs into them go.
// All copies are on the ring's one copy stream, in order, so a batch's last
// copied event covers the others.  Entry k of this call is expert k - G0.
int run_streamed_experts(const strata_moe_experts* ex, strata_moe_ring* ring, const Buffers& b,
                         const ChunkLists& cl, int64_t T, int64_t n, int32_t Eg, const _Float16* xuop,
                         _Float16* huop, hipStream_t st) {
    const int32_t H = ex->hidden, I = ex->ffn, R = ring->n_slots;
    const int32_t per = R / 3 > 0 ? R / 3 : 1;
    const int64_t G0 = ring->next, end = G0 + Eg;
    int64_t issued = G0, consumed = G0;
    const char* host = (const char*)ex->gate_up;
    // Enqueue the DMAs of entries [issued, upto).  Consecutive entries of one
    // batch go in one copy as far as the ring does not wrap (host blobs and
    // slots are both one slot apart): slot-sized copies measured ~37 GB/s on
    // the host link, copies of many slots ~56 GB/s.  A run first waits for
    // its slots' last use: the used events are recorded on the compute stream
    // in entry order, so the run's last slot (the latest earlier entry among
    // them) covers the others.  Each slot gets its copied event after the run,
    // and a run never spans two batches, so a batch's last event still covers
    // the batch.
    auto issue = [&](int64_t upto) -> int {
        while (issued < upto) {
            const int64_t batch_end = G0 + ((issued - G0) / per + 1) * per;
            const int s0 = (int)(issued % R);
            int64_t run_end = upto < batch_end ? upto : batch_end;
            if (run_end > issued + (R - s0)) run_end = issued + (R - s0);  // no wrap inside a copy
            for (int64_t k = run_end - 1; k >= issued; --k) {  // the latest recorded use among the run's slots
                const int s = (int)(k % R);
                if (ring->used_recorded[s]) {
                    HIP_TRY(hipStreamWaitEvent(ring->copy, ring->used[s], 0), "hipStreamWaitEvent");
                    break;
                }
            }
            HIP_TRY(hipMemcpyAsync(ring->slots + (int64_t)s0 * ring->slot_bytes, host + (issued - G0) * ring->slot_bytes,
                                   (size_t)(run_end - issued) * ring->slot_bytes, hipMemcpyHostToDevice, ring->copy),
                    "hipMemcpyAsync (expert DMA)");
            for (int64_t k = issued; k < run_end; ++k)
                HIP_TRY(hipEventRecord(ring->copied[k % R], ring->copy), "hipEventRecord");
            issued = run_end;
        }
        return 0;
    };
    TRY(issue(end < consumed + R ? end : consumed + R));
    for (int32_t e0 = 0; e0 < Eg;) {
        const int32_t e1 = Eg - e0 < per ? Eg : e0 + per;
        // every copy of the batch is enqueued: e1 - e0 <= per < R entries past `consumed`
        HIP_TRY(hipStreamWaitEvent(st, ring->copied[(G0 + e1 - 1) % R], 0), "hipStreamWaitEvent");
        ExpertRange rng;
        rng.first = cl.first;
        rng.E = Eg;
        rng.e0 = e0;
        rng.e1 = e1;
        rng.ring0 = G0 % R;
        rng.nring = R;
        rng.small_min_rows = small_min_rows(ex, n, Eg);
        rng.max_rows = T;
        HIP_TRY(launch_gate_up((const uint8_t*)ring->slots, ring->slot_bytes, cl, n, Eg, b.src, b.xt, b.xst,
                               tiled_rows_cap(n, Eg), b.xa, b.xs, T, xuop, b.xum, H, I, b.hq, b.hs, st, rng),
                "gate/up launch");
        TRY(launch_gemv_step(ex, true, (const uint8_t*)ring->slots, ring->slot_bytes, b, cl, T, n, Eg, rng, st));
        HIP_TRY(launch_tile_h(b.hq, b.hs, cl, tiled_rows_cap(n, Eg) / 16, I, code_offset(ex), b.hb, b.hst, huop, b.hum,
                              st, rng),
                "tile launch");
        HIP_TRY(launch_down((const uint8_t*)ring->slots + ring->gate_up_bytes, ring->slot_bytes, cl, n, Eg, b.src,
                            b.prow, b.hb, b.hst, tiled_rows_cap(n, Eg), b.hs, huop, b.hum, H, I, b.dm, st, rng),
                "down launch");
        TRY(launch_gemv_step(ex, false, (const uint8_t*)ring->slots + ring->gate_up_bytes, ring->slot_bytes, b, cl, T,
                             n, Eg, rng, st));
        for (int64_t k = G0 + e0; k < G0 + e1; ++k) {
            const int s = (int)(k % R);
            HIP_TRY(hipEventRecord(ring->used[s], st), "hipEventRecord");
            ring->used_recorded[s] = 1;
        }
        consumed = G0 + e1;
        TRY(issue(end < consumed + R ? end : consumed + R));
        e0 = e1;
    }
    ring->next = end;
    return 0;
}

// fixed_ws: a caller-provided workspace of fixed_bytes (then nothing is
// allocated), or null for the library's workspace.
int run_layer(const float* x, const float* wr, const strata_moe_experts* ex, int64_t T, int32_t K, float* out,
              hipStream_t st, Buffers* keep, strata_moe_ring* ring = nullptr, char* fixed_ws = nullptr,
              size_t fixed_bytes = 0) {
    const bool shared = ex->shared_gate != nullptr;
    const int32_t E = ex->n_expert, H = ex->hidden, I = ex->ffn;
    const int32_t Kg = K + shared, Eg = E + shared;  // the grouped pairs per token, the experts they go to
    const int64_t n = T * Kg;
    const Offsets o = plan(T, K, E, H, I, shared, per_slot_q8(ex, n, Eg));
    char* ws = fixed_ws;
    if (fixed_ws) {
        if (o.total > fixed_bytes)
            return fail(STRATA_MOE_EINVAL,
                        "this call needs %zu bytes of scratch; the fixed scratch holds %zu (fewer tokens per call)",
                        o.total, fixed_bytes);
    } else {
        TRY(get_workspace(o.total, &ws));
    }
    Buffers b = carve(ws, o);
    CallTimer tm(st);
    tm.begin(kQuantize);
    // one pass over x: int8 codes and scales, their fp16 copy, row multipliers and
    // offset operand; it also clears the id error flag
    _Float16* xuop = has_offset(ex) ? b.xuop : nullptr;
    _Float16* huop = has_offset(ex) ? b.huop : nullptr;
    HIP_TRY(launch_quantize_prescale(x, T, H, code_offset(ex), b.xq, b.xs, b.xa, b.xe, b.xn, xuop, b.xum, st,
                                     ZeroWords{{b.err, nullptr}}),
            "quantize launch");
    tm.end(kQuantize);
    tm.begin(kRouter);
    // the router matrix's MFMA operand and transposed copy: prepared once by the
    // caller (experts->router_prepared) or here on every call
    RouterScratch rs{b.wt, b.wb, b.wm, b.wnorm, nullptr, nullptr, b.pmax};
    if (ex->router_prepared) {
        const RouterPrepared rp = router_prepared_layout(H, E);
        char* base = (char*)ex->router_prepared;
        rs = RouterScratch{(float*)(base + rp.wt), (_Float16*)(base + rp.wb), (float*)(base + rp.wm),
                           (float*)(base + rp.wnorm), nullptr, nullptr, nullptr};
    }
    HIP_TRY(launch_router(x, b.xe, ex->router_prepared ? nullptr : wr, ex->router_bias, T, H, E, rs, b.logits, st),
            "router launch");
    tm.end(kRouter);
    tm.begin(kTopK);
    HIP_TRY(launch_topk(b.logits, x, b.xn, rs.wt, rs.wnorm, ex->router_bias, T, H, E, K, b.ids, b.p, st),
            "top-K launch");
    if (shared)
        HIP_TRY(launch_shared_slot(x, ex->shared_gate, b.ids, b.p, T, H, K, E, b.gids, b.gp, st), "shared gate launch");
    tm.end(kTopK);
    tm.begin(kGroup);
    const ChunkLists cl{b.tiles, b.ntiles, b.tiles_cap, b.trows, b.first};
    HIP_TRY(launch_group(b.gids, b.gp, n, Kg, Eg, b.hist, b.base, b.offsets, cl, b.src, b.slot, b.prow, b.err, st),
            "group launch");
    // the big chunks' input codes and scales, gathered into the tiled layout
    // (none where no expert can have more than kSmallRows rows: T <= kSmallRows)
    if (T > kSmallRows)
        HIP_TRY(launch_gather_tiles(b.xq, b.xs, b.src, cl, tiled_rows_cap(n, Eg) / 16, H, b.xt, b.xst, st),
                "gather launch");
    // the per-slot q8_1 arm: every routed slot's input row rounded again, with block code sums
    if (per_slot_q8(ex, n, Eg)) HIP_TRY(launch_quantize_slots(x, b.src, n, H, b.sq, b.ss, b.ssum, st), "quantize launch");
    tm.end(kGroup);
    if (ring) {
        tm.begin(kStreamed);
        TRY(run_streamed_experts(ex, ring, b, cl, T, n, Eg, xuop, huop, st));
        tm.end(kStreamed);
        tm.begin(kCombine);
        HIP_TRY(launch_combine(b.dm, b.slot, T, Kg, H, out, st), "combine launch");
        tm.end(kCombine);
        if (keep) *keep = b;
        return 0;
    }
    ExpertRange all;  // every expert, resident
    all.small_min_rows = small_min_rows(ex, n, Eg);
    all.max_rows = T;
    // the MFMA down kernels' tiled H: not needed where every chunk is the GEMV's
    const bool mfma_down = all.small_min_rows == 0 || T >= all.small_min_rows;
    // the MFMA gate/up kernels' epilogue writes the down GEMM's tiled operand
    // and the offset pass's block values of their chunks' rows
    HTiled ht;
    if (mfma_down) ht = HTiled{b.hb, b.hst, huop ? reinterpret_cast<float*>(huop) : nullptr, code_offset(ex)};
    tm.begin(kGateUp);
    // (their int8 H codes only where the caller keeps the intermediates)
    HIP_TRY(launch_gate_up((const uint8_t*)ex->gate_up, ex->gate_up_stride, cl, n, Eg, b.src, b.xt, b.xst,
                           tiled_rows_cap(n, Eg), b.xa, b.xs, T, xuop, b.xum, H, I, mfma_down && !keep ? nullptr : b.hq,
                           b.hs, st, all, ht),
            "gate/up launch");
    TRY(launch_gemv_step(ex, true, (const uint8_t*)ex->gate_up, ex->gate_up_stride, b, cl, T, n, Eg, all, st));
    tm.end(kGateUp);
    tm.begin(kTileH);
    if (mfma_down && huop)
        HIP_TRY(launch_offset_rows(reinterpret_cast<float*>(huop), n, I, b.hum, st), "offset operand launch");
    tm.end(kTileH);
    tm.begin(kDown);
    HIP_TRY(launch_down((const uint8_t*)ex->down, ex->down_stride, cl, n, Eg, b.src, b.prow, b.hb, b.hst,
                        tiled_rows_cap(n, Eg), b.hs, huop, b.hum, H, I, b.dm, st, all),
            "down launch");
    TRY(launch_gemv_step(ex, false, (const uint8_t*)ex->down, ex->down_stride, b, cl, T, n, Eg, all, st));
    tm.end(kDown);
    tm.begin(kCombine);
    HIP_TRY(launch_combine(b.dm, b.slot, T, Kg, H, out, st), "combine launch");
    tm.end(kCombine);
    if (keep) *keep = b;
    return 0;
}

// The scratch of strata_moe_prefill_noalloc: one array per GPU the library
// runs on, loaded with the code object and held until the process ends.  Its
// device address comes from hipGetSymbolAddress once per device (the array's
// name in host code is not a device address).
static __device__ __align__(256) unsigned char scratch[STRATA_MOE_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
char* g_scratch_ptr[64] = {};

int noalloc_scratch(char** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(STRATA_MOE_EINVAL, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (!p || !aligned(p, 256)) return fail(STRATA_MOE_EHIP, "the scratch array has no usable device address");
        g_scratch_ptr[dev] = (char*)p;
    }
    *out = g_scratch_ptr[dev];
    return 0;
}

}  // namespace

// ===================================================================== C ABI
extern "C" {

int strata_moe_device_supported(void) {
    const std::string saved = g_err;
    const int rc = check_device();
    g_err = saved;
    return rc == 0 ? 1 : 0;
}

const char* strata_moe_last_error(void) { return g_err.c_str(); }

int strata_moe_packed_bytes(int32_t hidden, int32_t ffn, int64_t* gate_up_bytes, int64_t* down_bytes) {
    g_err.clear();
    if (!gate_up_bytes || !down_bytes) return fail(STRATA_MOE_EINVAL, "null output pointer");
    TRY(check_dims(hidden, ffn));
    *gate_up_bytes = round_up(packed_matrix_bytes(2LL * ffn, hidden), 256);
    *down_bytes = round_up(packed_matrix_bytes(hidden, ffn), 256);
    return 0;
}

int strata_moe_router_prepared_bytes(int32_t hidden, int32_t n_expert, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(STRATA_MOE_EINVAL, "bytes is NULL");
    if (hidden < 128 || hidden % 128 || hidden > 4096)
        return fail(STRATA_MOE_EINVAL, "hidden %d is not a multiple of 128 in [128, 4096]", hidden);
    if (n_expert < 1 || n_expert > kMaxExperts)
        return fail(STRATA_MOE_EINVAL, "n_expert %d outside [1, %d]", n_expert, kMaxExperts);
    *bytes = router_prepared_layout(hidden, n_expert).total;
    return 0;
}

int strata_moe_prepare_router(const float* router_w, int32_t hidden, int32_t n_expert, void* prepared, void* stream) {
    size_t bytes = 0;
    TRY(strata_moe_router_prepared_bytes(hidden, n_expert, &bytes));
    if (!router_w || !prepared) return fail(STRATA_MOE_EINVAL, "null pointer");
    if (!aligned(prepared, 256)) return fail(STRATA_MOE_EINVAL, "prepared must be 256-byte aligned");
    TRY(check_device());
    const RouterPrepared rp = router_prepared_layout(hidden, n_expert);
    char* base = (char*)prepared;
    const RouterScratch rs{(float*)(base + rp.wt), (_Float16*)(base + rp.wb), (float*)(base + rp.wm),
                           (float*)(base + rp.wnorm), nullptr, nullptr, (float*)(base + rp.pmax)};
    HIP_TRY(launch_router_prep(router_w, hidden, n_expert, rs, (hipStream_t)stream), "router prep launch");
    return 0;
}

int strata_moe_workspace_bytes(int64_t T, int32_t K, const strata_moe_experts* experts, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(STRATA_MOE_EINVAL, "bytes is NULL");
    TRY(check_layer(T, K, experts));
    const int32_t sh = experts->shared_gate != nullptr;
    *bytes = plan(T, K, experts->n_expert, experts->hidden, experts->ffn, sh,
                  per_slot_q8(experts, T * (K + sh), experts->n_expert + sh))
                 .total;
    return 0;
}

int strata_moe_set_workspace(void* dev_ptr, size_t bytes) {
    g_err.clear();
    if (dev_ptr && !aligned(dev_ptr, 256)) return fail(STRATA_MOE_EINVAL, "workspace must be 256-byte aligned");
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(STRATA_MOE_EINVAL, "device index %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_ws_mu);
    g_ws[dev].user = dev_ptr;
    g_ws[dev].user_bytes = dev_ptr ? bytes : 0;
    return 0;
}

int strata_moe_pack(const uint8_t* codes_gu, const uint16_t* scales_gu, const uint8_t* codes_d,
                    const uint16_t* scales_d, int32_t e0, int32_t e1, int32_t hidden, int32_t ffn, void* gate_up,
                    int64_t gate_up_stride, void* down, int64_t down_stride, void* stream) {
    g_err.clear();
    int64_t gu = 0, dn = 0;
    TRY(strata_moe_packed_bytes(hidden, ffn, &gu, &dn));
    if (!codes_gu || !scales_gu || !codes_d || !scales_d || !gate_up || !down)
        return fail(STRATA_MOE_EINVAL, "null pointer");
    if (e0 < 0 || e1 < e0) return fail(STRATA_MOE_EINVAL, "bad expert range [%d, %d)", e0, e1);
    if (gate_up_stride < gu || down_stride < dn || gate_up_stride % 256 || down_stride % 256 ||
        !aligned(gate_up, 256) || !aligned(down, 256))
        return fail(STRATA_MOE_EINVAL, "blob strides/pointers must be 256-byte aligned and >= the packed sizes");
    TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    const int32_t ne = e1 - e0;
    HIP_TRY(launch_pack(codes_gu, scales_gu, ne, 2 * ffn, hidden, ffn, (uint8_t*)gate_up + (int64_t)e0 * gate_up_stride,
                        gate_up_stride, st),
            "pack launch");
    HIP_TRY(launch_pack(codes_d, scales_d, ne, hidden, ffn, 0, (uint8_t*)down + (int64_t)e0 * down_stride, down_stride,
                        st),
            "pack launch");
    return 0;
}

int strata_moe_unpack(const void* gate_up, int64_t gate_up_stride, const void* down, int64_t down_stride, int32_t e0,
                      int32_t e1, int32_t hidden, int32_t ffn, uint8_t* codes_gu, uint16_t* scales_gu,
                      uint8_t* codes_d, uint16_t* scales_d, void* stream) {
    g_err.clear();
    int64_t gu = 0, dn = 0;
    TRY(strata_moe_packed_bytes(hidden, ffn, &gu, &dn));
    if (!codes_gu || !scales_gu || !codes_d || !scales_d || !gate_up || !down)
        return fail(STRATA_MOE_EINVAL, "null pointer");
    if (e0 < 0 || e1 < e0) return fail(STRATA_MOE_EINVAL, "bad expert range [%d, %d)", e0, e1);
    if (gate_up_stride < gu || down_stride < dn) return fail(STRATA_MOE_EINVAL, "strides below the packed sizes");
    TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    const int32_t ne = e1 - e0;
    HIP_TRY(launch_unpack((const uint8_t*)gate_up + (int64_t)e0 * gate_up_stride, gate_up_stride, ne, 2 * ffn, hidden,
                          ffn, codes_gu, scales_gu, st),
            "unpack launch");
    HIP_TRY(launch_unpack((const uint8_t*)down + (int64_t)e0 * down_stride, down_stride, ne, hidden, ffn, 0, codes_d,
                          scales_d, st),
            "unpack launch");
    return 0;
}

int strata_moe_prefill(const float* x, const float* router_w, const strata_moe_experts* experts, int64_t T,
                       int32_t K, float* out, void* stream) {
    g_err.clear();
    TRY(check_layer(T, K, experts));
    if (T == 0) return 0;
    if (!x || !router_w || !out) return fail(STRATA_MOE_EINVAL, "null x / router_w / out");
    if (!aligned(x, 16) || !aligned(out, 16)) return fail(STRATA_MOE_EINVAL, "x and out must be 16-byte aligned");
    TRY(check_no_overlap(x, out, T * experts->hidden * 4));
    TRY(check_device());
    return run_layer(x, router_w, experts, T, K, out, (hipStream_t)stream, nullptr);
}

int strata_moe_prefill_noalloc(const float* x, const float* router_w, const strata_moe_experts* experts, int64_t T,
                               int32_t K, float* out, void* stream) {
    g_err.clear();
    TRY(check_layer(T, K, experts));
    if (T == 0) return 0;
    if (!x || !router_w || !out) return fail(STRATA_MOE_EINVAL, "null x / router_w / out");
    if (!aligned(x, 16) || !aligned(out, 16)) return fail(STRATA_MOE_EINVAL, "x and out must be 16-byte aligned");
    TRY(check_no_overlap(x, out, T * experts->hidden * 4));
    TRY(check_device());
    char* ws = nullptr;
    TRY(noalloc_scratch(&ws));
    return run_layer(x, router_w, experts, T, K, out, (hipStream_t)stream, nullptr, nullptr, ws,
                     STRATA_MOE_NOALLOC_SCRATCH_BYTES);
}

int strata_moe_prefill_debug(const float* x, const float* router_w, const strata_moe_experts* experts, int64_t T,
                             int32_t K, float* out, const strata_moe_debug* dbg, void* stream) {
    g_err.clear();
    TRY(check_layer(T, K, experts));
    if (T == 0) return 0;
    if (!x || !router_w || !out || !dbg) return fail(STRATA_MOE_EINVAL, "null x / router_w / out / dbg");
    if (!aligned(x, 16) || !aligned(out, 16)) return fail(STRATA_MOE_EINVAL, "x and out must be 16-byte aligned");
    TRY(check_no_overlap(x, out, T * experts->hidden * 4));
    TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    Buffers b;
    TRY(run_layer(x, router_w, experts, T, K, out, st, &b));
    const int32_t sh = experts->shared_gate ? 1 : 0;
    const int32_t E = experts->n_expert + sh, H = experts->hidden, I = experts->ffn;
    const int64_t n = T * (K + sh);
    auto cp = [&](void* dst, const void* src, size_t bytes) -> int {
        if (dst) HIP_TRY(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st), "hipMemcpyAsync");
        return 0;
    };
    TRY(cp(dbg->ids, b.gids, n * 4));
    TRY(cp(dbg->p, b.gp, n * 4));
    TRY(cp(dbg->offsets, b.offsets, (E + 1) * 4));
    TRY(cp(dbg->src, b.src, n * 4));
    TRY(cp(dbg->slot, b.slot, n * 4));
    TRY(cp(dbg->sx, b.xs, T * (H / kBlock) * 4));
    TRY(cp(dbg->sh, b.hs, n * (I / kBlock) * 4));
    TRY(cp(dbg->qx, b.xq, T * H));
    TRY(cp(dbg->qh, b.hq, n * I));
    return 0;
}

int strata_moe_ring_bytes(int32_t n_slots, int32_t hidden, int32_t ffn, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(STRATA_MOE_EINVAL, "bytes is NULL");
    if (n_slots < 1 || n_slots > 65536) return fail(STRATA_MOE_EINVAL, "n_slots %d outside [1, 65536]", n_slots);
    int64_t gu = 0, dn = 0;
    TRY(strata_moe_packed_bytes(hidden, ffn, &gu, &dn));
    *bytes = (size_t)n_slots * (size_t)(gu + dn);
    return 0;
}

int strata_moe_ring_create(int32_t n_slots, int32_t hidden, int32_t ffn, void* slots, size_t slot_memory_bytes,
                           void* copy_stream, strata_moe_ring** ring) {
    g_err.clear();
    if (!ring) return fail(STRATA_MOE_EINVAL, "ring is NULL");
    *ring = nullptr;
    size_t need = 0;
    TRY(strata_moe_ring_bytes(n_slots, hidden, ffn, &need));
    if (!slots || !aligned(slots, 256)) return fail(STRATA_MOE_EINVAL, "slot memory must be 256-byte aligned device memory");
    if (slot_memory_bytes < need)
        return fail(STRATA_MOE_EINVAL, "slot memory of %zu bytes, %zu needed", slot_memory_bytes, need);
    if (!copy_stream) return fail(STRATA_MOE_EINVAL, "the ring needs a copy stream of its own");
    TRY(check_device());
    int64_t gu = 0, dn = 0;
    TRY(strata_moe_packed_bytes(hidden, ffn, &gu, &dn));
    strata_moe_ring* r = new strata_moe_ring();
    HIP_TRY(hipGetDevice(&r->device), "hipGetDevice");
    r->n_slots = n_slots;
    r->hidden = hidden;
    r->ffn = ffn;
    r->gate_up_bytes = gu;
    r->slot_bytes = gu + dn;
    r->slots = (char*)slots;
    r->copy = (hipStream_t)copy_stream;
    r->copied.assign(n_slots, nullptr);
    r->used.assign(n_slots, nullptr);
    r->used_recorded.assign(n_slots, 0);
    for (int i = 0; i < n_slots; ++i)
        if (hipEventCreateWithFlags(&r->copied[i], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&r->used[i], hipEventDisableTiming) != hipSuccess) {
            strata_moe_ring_destroy(r);
            return fail(STRATA_MOE_EHIP, "hipEventCreate failed");
        }
    *ring = r;
    return 0;
}

int strata_moe_ring_destroy(strata_moe_ring* ring) {
    g_err.clear();
    if (!ring) return 0;
    // the events may still be pending: wait for the ring's last DMA and use
    for (size_t i = 0; i < ring->copied.size(); ++i) {
        if (ring->copied[i]) (void)hipEventSynchronize(ring->copied[i]);
        if (ring->used[i] && ring->used_recorded[i]) (void)hipEventSynchronize(ring->used[i]);
    }
    for (hipEvent_t e : ring->copied)
        if (e) (void)hipEventDestroy(e);
    for (hipEvent_t e : ring->used)
        if (e) (void)hipEventDestroy(e);
    delete ring;
    return 0;
}

int strata_moe_prefill_streamed(const float* x, const float* router_w, const strata_moe_experts* experts,
                                strata_moe_ring* ring, int64_t T, int32_t K, float* out, void* stream) {
    g_err.clear();
    if (!ring) return fail(STRATA_MOE_EINVAL, "ring is NULL");
    if (!experts) return fail(STRATA_MOE_EINVAL, "experts is NULL");
    // the host blobs: expert e's gate/up blob then its down blob, one slot's
    // bytes per expert (so one DMA moves an expert)
    if (experts->hidden != ring->hidden || experts->ffn != ring->ffn)
        return fail(STRATA_MOE_EINVAL, "the ring was made for H = %d, I = %d", ring->hidden, ring->ffn);
    if (experts->gate_up_stride != ring->slot_bytes || experts->down_stride != ring->slot_bytes ||
        (const char*)experts->down != (const char*)experts->gate_up + ring->gate_up_bytes)
        return fail(STRATA_MOE_EINVAL,
                    "streamed experts must be interleaved: expert e at gate_up + e * %lld, its down blob %lld bytes "
                    "after its gate/up blob",
                    (long long)ring->slot_bytes, (long long)ring->gate_up_bytes);
    TRY(check_layer(T, K, experts));
    if (T == 0) return 0;
    if (!x || !router_w || !out) return fail(STRATA_MOE_EINVAL, "null x / router_w / out");
    if (!aligned(x, 16) || !aligned(out, 16)) return fail(STRATA_MOE_EINVAL, "x and out must be 16-byte aligned");
    TRY(check_no_overlap(x, out, T * experts->hidden * 4));
    TRY(check_device());
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev), "hipGetDevice");
    if (dev != ring->device) return fail(STRATA_MOE_EINVAL, "the ring belongs to device %d", ring->device);
    if ((hipStream_t)stream == ring->copy) return fail(STRATA_MOE_EINVAL, "the compute stream is the ring's copy stream");
    hipPointerAttribute_t pa;
    if (hipPointerGetAttributes(&pa, experts->gate_up) != hipSuccess || pa.type != hipMemoryTypeHost) {
        (void)hipGetLastError();
        return fail(STRATA_MOE_EINVAL, "streamed expert blobs must be pinned host memory (hipHostMalloc)");
    }
    return run_layer(x, router_w, experts, T, K, out, (hipStream_t)stream, nullptr, ring);
}

int strata_moe_route(const float* x, const float* router_w, const float* bias, int64_t T, int32_t H, int32_t E,
                     int32_t K, int32_t* ids, float* p, void* stream) {
    g_err.clear();
    if (E < 1 || E > kMaxExperts) return fail(STRATA_MOE_EINVAL, "E = %d outside [1, %d]", E, kMaxExperts);
    if (H < 64 || H % 64) return fail(STRATA_MOE_EINVAL, "H = %d is not a positive multiple of 64", H);  // top-K rescore
    TRY(check_tk(T, K, E));
    if (T == 0) return 0;
    if (!x || !router_w || !ids || !p) return fail(STRATA_MOE_EINVAL, "null pointer");
    if (!aligned(x, 16)) return fail(STRATA_MOE_EINVAL, "x must be 16-byte aligned");
    TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    Layout L;
    const size_t lo = L.take<float>(router_logit_floats(T, H, E)), o_wt = L.take<float>((int64_t)E * H);
    const size_t o_wb = L.take<_Float16>(router_padded_experts(E) * H * 2);
    const size_t o_wm = L.take<float>(router_padded_experts(E)), o_xm = L.take<float>(T);
    const size_t o_wn = L.take<float>(1), o_xn = L.take<float>(T);
    const size_t o_pm = L.take<float>((int64_t)((H + 31) / 32) * E);
    char* ws = nullptr;
    TRY(get_workspace(L.off, &ws));
    float* logits = (float*)(ws + lo);
    float* wt = (float*)(ws + o_wt);
    const RouterScratch rs{wt, (_Float16*)(ws + o_wb), (float*)(ws + o_wm), (float*)(ws + o_wn), (float*)(ws + o_xm),
                           (float*)(ws + o_xn), (float*)(ws + o_pm)};
    HIP_TRY(launch_router(x, nullptr, router_w, bias, T, H, E, rs, logits, st), "router launch");
    HIP_TRY(launch_topk(logits, x, rs.xn, wt, rs.wnorm, bias, T, H, E, K, ids, p, st), "top-K launch");
    return 0;
}

int strata_moe_group(const int32_t* ids, int64_t T, int32_t K, int32_t E, int32_t* offsets, int32_t* src,
                     int32_t* slot, void* stream) {
    g_err.clear();
    if (E < 1 || E > kMaxExperts) return fail(STRATA_MOE_EINVAL, "E = %d outside [1, %d]", E, kMaxExperts);
    TRY(check_tk(T, K, E));
    if (!ids || !offsets || !src || !slot) return fail(STRATA_MOE_EINVAL, "null pointer");
    TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    const int64_t n = T * K;
    const int64_t nchunks = (n + kGroupChunk - 1) / kGroupChunk;
    Layout L;
    const size_t o_hist = L.take<int32_t>(nchunks * E), o_base = L.take<int32_t>(nchunks * E);
    const int64_t cap = chunk_list_cap(n, E);
    const size_t o_tiles = L.take<Tile>(2 * cap), o_nt = L.take<int32_t>(kSchedInts), o_err = L.take<int32_t>(1);
    const size_t o_trows = L.take<TileRows>(tiled_rows_cap(n, E) / 16);
    char* ws = nullptr;
    TRY(get_workspace(L.off, &ws));
    int32_t* err = (int32_t*)(ws + o_err);
    HIP_TRY(launch_fill_zero((float*)err, 1, st), "fill launch");
    HIP_TRY(launch_group(ids, nullptr, n, K, E, (int32_t*)(ws + o_hist), (int32_t*)(ws + o_base), offsets,
                         ChunkLists{(Tile*)(ws + o_tiles), (int32_t*)(ws + o_nt), cap, (TileRows*)(ws + o_trows)}, src,
                         slot, nullptr, err, st),
            "group launch");
    int32_t herr = 0;
    HIP_TRY(hipMemcpyAsync(&herr, err, 4, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
    HIP_TRY(hipStreamSynchronize(st), "hipStreamSynchronize");
    if (herr) return fail(STRATA_MOE_EDATA, "routed expert id out of range [0, %d)", E);
    return 0;
}

int strata_moe_quantize(const float* v, int64_t rows, int32_t cols, int8_t* codes, float* scales, void* stream) {
    g_err.clear();
    if (rows < 0 || cols < 32 || cols % 32) return fail(STRATA_MOE_EINVAL, "rows %lld / cols %d", (long long)rows, cols);
    if (rows == 0) return 0;
    if (!v || !codes || !scales) return fail(STRATA_MOE_EINVAL, "null pointer");
    if (!aligned(v, 16) || !aligned(codes, 4)) return fail(STRATA_MOE_EINVAL, "v must be 16-, codes 4-byte aligned");
    TRY(check_device());
    HIP_TRY(launch_quantize(v, rows, cols, codes, scales, (hipStream_t)stream), "quantize launch");
    return 0;
}

int strata_moe_gate_up(const int8_t* qx, const float* sx, const int32_t* offsets, const int32_t* src, int64_t T,
                       int32_t K, const strata_moe_experts* experts, int8_t* qh, float* sh, void* stream) {
    g_err.clear();
    TRY(check_experts(experts));
    TRY(check_tk(T, K, experts->n_expert));
    TRY(check_buffers(T, K, experts->n_expert, experts->hidden, experts->ffn));
    if (T == 0) return 0;
    if (!qx || !sx || !offsets || !src || !qh || !sh) return fail(STRATA_MOE_EINVAL, "null pointer");
    TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    const int32_t E = experts->n_expert, H = experts->hidden, I = experts->ffn;
    const int64_t n = T * K;
    Layout L;
    const size_t o_xa = L.take<_Float16>(T * H), o_xt = L.take<_Float16>(tiled_rows_cap(n, E) * H);
    const size_t o_xst = L.take<float>(tiled_rows_cap(n, E) * (H / kBlock));
    const size_t o_xuop = L.take<_Float16>(T * offset_operand_halves(H)), o_xum = L.take<float>(T);
    const int64_t cap = chunk_list_cap(n, E);
    const size_t o_tiles = L.take<Tile>(2 * cap), o_nt = L.take<int32_t>(kSchedInts),
                 o_trows = L.take<TileRows>(tiled_rows_cap(n, E) / 16);
    char* ws = nullptr;
    TRY(get_workspace(L.off, &ws));
    const ChunkLists cl{(Tile*)(ws + o_tiles), (int32_t*)(ws + o_nt), cap, (TileRows*)(ws + o_trows)};
    _Float16* xa = (_Float16*)(ws + o_xa);
    _Float16* xt = (_Float16*)(ws + o_xt);
    float* xst = (float*)(ws + o_xst);
    _Float16* xuop = (_Float16*)(ws + o_xuop);
    float* xum = (float*)(ws + o_xum);
    if (!has_offset(experts)) xuop = nullptr;
    HIP_TRY(launch_prescale(qx, sx, T, H, code_offset(experts), xa, nullptr, xuop, xum, st), "prescale launch");
    HIP_TRY(launch_chunks_from_offsets(offsets, E, n, cl, st), "chunk list launch");  // and the tile table
    HIP_TRY(launch_gather_tiles(qx, sx, src, cl, tiled_rows_cap(n, E) / 16, H, xt, xst, st), "gather launch");
    // the layer's kernel choice for short chunks (the GEMV by token: the
    // per-slot arm needs the fp32 input, which this entry has not)
    ExpertRange all;
    all.small_min_rows = small_min_rows(experts, n, E);
    HIP_TRY(launch_gate_up((const uint8_t*)experts->gate_up, experts->gate_up_stride, cl, n, E, src, xt, xst,
                           tiled_rows_cap(n, E), xa, sx, T, xuop, xum, H, I, qh, sh, st, all),
            "gate/up launch");
    if (gemv_rows(experts, n, E) > 0) {
        GemvLaunch l{};
        l.max_rows = gemv_rows(experts, n, E);
        l.gate_up = true;
        l.blobs = (const uint8_t*)experts->gate_up;
        l.stride = experts->gate_up_stride;
        l.src = src;
        l.act = qx;
        l.act_rows = T;
        l.ascale = sx;
        l.sym = experts->format == STRATA_MOE_Q2_SYM ? 1 : 0;
        l.H = H;
        l.I = I;
        l.hq = qh;
        l.hs = sh;
        HIP_TRY(launch_gemv(l, cl, n, E, all, st), "GEMV launch");
    }
    return 0;
}

int strata_moe_down(const int8_t* qh, const float* sh, const int32_t* offsets, const int32_t* src,
                    const int32_t* slot, const float* p, int64_t T, int32_t K, const strata_moe_experts* experts,
                    float* out, void* stream) {
    g_err.clear();
    TRY(check_experts(experts));
    TRY(check_tk(T, K, experts->n_expert));
    TRY(check_buffers(T, K, experts->n_expert, experts->hidden, experts->ffn));
    if (T == 0) return 0;
    if (!qh || !sh || !offsets || !src || !slot || !p || !out) return fail(STRATA_MOE_EINVAL, "null pointer");
    TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    const int32_t E = experts->n_expert, H = experts->hidden, I = experts->ffn;
    const int64_t n = T * K;
    Layout L;
    const size_t o_hb = L.take<_Float16>(tiled_rows_cap(n, E) * I), o_hst = L.take<float>(tiled_h_scale_floats(n, E, I));
    const size_t o_huop = L.take<_Float16>(n * offset_operand_halves(I)), o_hum = L.take<float>(n);
    const int64_t cap = chunk_list_cap(n, E);
    const size_t o_tiles = L.take<Tile>(2 * cap), o_nt = L.take<int32_t>(kSchedInts), o_prow = L.take<float>(n);
    const size_t o_dm = L.take<float>(n * H), o_trows = L.take<TileRows>(tiled_rows_cap(n, E) / 16);
    char* ws = nullptr;
    TRY(get_workspace(L.off, &ws));
    const ChunkLists cl{(Tile*)(ws + o_tiles), (int32_t*)(ws + o_nt), cap, (TileRows*)(ws + o_trows)};
    _Float16* hb = (_Float16*)(ws + o_hb);
    float* hst = (float*)(ws + o_hst);
    _Float16* huop = (_Float16*)(ws + o_huop);
    float* hum = (float*)(ws + o_hum);
    float* prow = (float*)(ws + o_prow);
    float* dm = (float*)(ws + o_dm);
    HIP_TRY(launch_chunks_from_offsets(offsets, E, n, cl, st), "chunk list launch");  // and the tile table
    if (!has_offset(experts)) huop = nullptr;
    HIP_TRY(launch_tile_h(qh, sh, cl, tiled_rows_cap(n, E) / 16, I, code_offset(experts), hb, hst, huop, hum, st),
            "tile launch");
    HIP_TRY(launch_row_weights(slot, p, n, prow, st), "weights launch");
    ExpertRange all;  // the layer's kernel choice, as strata_moe_gate_up
    all.small_min_rows = small_min_rows(experts, n, E);
    HIP_TRY(launch_down((const uint8_t*)experts->down, experts->down_stride, cl, n, E, src, prow, hb, hst,
                        tiled_rows_cap(n, E), sh, huop, hum, H, I, dm, st, all),
            "down launch");
    if (gemv_rows(experts, n, E) > 0) {
        GemvLaunch l{};
        l.max_rows = gemv_rows(experts, n, E);
        l.gate_up = false;
        l.blobs = (const uint8_t*)experts->down;
        l.stride = experts->down_stride;
        l.act = qh;
        l.act_rows = n;
        l.ascale = sh;
        l.sym = experts->format == STRATA_MOE_Q2_SYM ? 1 : 0;
        l.prow = prow;
        l.H = H;
        l.I = I;
        l.y = dm;
        HIP_TRY(launch_gemv(l, cl, n, E, all, st), "GEMV launch");
    }
    HIP_TRY(launch_combine(dm, slot, T, K, H, out, st), "combine launch");
    return 0;
}

int strata_moe_timing(int enable, int32_t max_calls) {
    g_err.clear();
    std::lock_guard<std::mutex> lock(g_tm_mu);
    for (hipEvent_t e : g_tm.ev) hipEventDestroy(e);
    g_tm = Timing();
    if (!enable) return 0;
    if (max_calls < 1 || max_calls > 100000) return fail(STRATA_MOE_EINVAL, "max_calls %d", max_calls);
    g_tm.ev.resize((size_t)max_calls * kNumKinds * 2);
    for (auto& e : g_tm.ev) HIP_TRY(hipEventCreate(&e), "hipEventCreate");
    g_tm.recorded.assign((size_t)max_calls * kNumKinds, 0);
    g_tm.max_calls = max_calls;
    g_tm.on = true;
    return 0;
}

int strata_moe_timing_kinds(void) { return kNumKinds; }

const char* strata_moe_timing_name(int id) { return id >= 0 && id < kNumKinds ? kKindNames[id] : ""; }

int strata_moe_timing_read(double* total_ms, int32_t* launches, int n) {
    g_err.clear();
    if (!total_ms || !launches || n < kNumKinds) return fail(STRATA_MOE_EINVAL, "need arrays of %d", kNumKinds);
    std::lock_guard<std::mutex> lock(g_tm_mu);
    for (int k = 0; k < kNumKinds; ++k) total_ms[k] = 0.0, launches[k] = 0;
    for (int c = 0; c < g_tm.used; ++c)
        for (int k = 0; k < kNumKinds; ++k) {
            if (!g_tm.recorded[(size_t)c * kNumKinds + k]) continue;
            hipEvent_t a = g_tm.ev[((size_t)c * kNumKinds + k) * 2], b = g_tm.ev[((size_t)c * kNumKinds + k) * 2 + 1];
            HIP_TRY(hipEventSynchronize(b), "hipEventSynchronize");
            float ms = 0.f;
            HIP_TRY(hipEventElapsedTime(&ms, a, b), "hipEventElapsedTime");
            total_ms[k] += ms;
            launches[k] += 1;
        }
    return 0;
}

}  // extern "C"
