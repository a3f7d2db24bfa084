/*
 * strata_moe.h -- C ABI of the MI355X (gfx950) routed-expert prompt MoE layer.
 *
 * One call runs the prompt-prefill mixture-of-experts layer that the Strata
 * pages describe as the "fused int8 experts" (Strata compare
 * v0.1.35...v0.1.37 page, include/strata/prefill/moe_fused.hpp; called from
 * the MoE half of Prefill::run on the Winery-Strata prefill.cpp page):
 *
 *   1. router projection of the layer input and route() to K experts/token
 *      with their weights (prefill.cpp, MoE half);
 *   2. the input rounded to int8 once per token, one scale per 32 values
 *      (moe_fused.hpp, quantize_act);
 *   3. the (token, k) pairs grouped by expert on the GPU, no host wait
 *      (moe_fused.hpp, group: slot[i] = row of pair i, src[row] = token);
 *   4. per expert: gate/up on the grouped int8 rows, SwiGLU, H rounded to
 *      int8 per 32 values, then down (moe_fused.hpp, experts);
 *   5. the combine of each token's K rows with its routing weights.
 *
 * The experts are either resident in device memory (strata_moe_prefill) or
 * streamed from pinned host memory through a ring of device slots while the
 * layer runs (strata_moe_prefill_streamed).
 *
 * Conventions for every entry point:
 *   - Pointers named in the argument lists are DEVICE pointers owned by the
 *     caller unless stated otherwise; the library keeps no reference to them
 *     after the call returns.  `stream` is a hipStream_t (NULL = the default
 *     stream); all work is enqueued on it in order and the call returns
 *     without waiting for the GPU unless stated.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     non-zero return means nothing (or, for STRATA_MOE_EHIP, not all) of the
 *     work was enqueued; strata_moe_last_error() then describes why.
 *   - Sizes: H a multiple of 128 and I a multiple of 64, both at most 4096;
 *     1 <= K <= 16, K <= E <= 1024, T * K < 2^31.  T = 0 is a no-op.  (The
 *     single-step route entry point only needs H a multiple of 64.)  One call
 *     also keeps its tiled fp16 GEMM operands below 2 GiB each:
 *     (T * K + 15 * E) * max(H, I) * 2 bytes < 2^31 (and x below 2 GiB), which
 *     at H = 2560, K = 10, E = 512 allows up to about 41,000 tokens; longer
 *     prompts run as several chunks (the pages' prompt path is chunked too).
 *   - Thread safety: calls may come from several host threads; calls that
 *     share the library-owned workspace of one device (the default when no
 *     workspace was set) must not overlap on different streams.
 */
#ifndef STRATA_MOE_H
#define STRATA_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define STRATA_MOE_OK 0
#define STRATA_MOE_EINVAL (-1)       /* bad argument: null pointer, size, alignment */
#define STRATA_MOE_EUNSUPPORTED (-2) /* no gfx950 device, or an unknown weight format */
#define STRATA_MOE_ENOMEM (-3)       /* workspace allocation failed or was too small */
#define STRATA_MOE_EHIP (-4)         /* a HIP runtime call or launch failed */
#define STRATA_MOE_EDATA (-5)        /* a routed expert id out of range (strata_moe_group) */

/* Weight formats: 2-bit codes q in {0,1,2,3} with one fp16 scale d per 32
 * consecutive codes along the reduction dimension.
 *   STRATA_MOE_Q2_SYM: w = d * (q - 1.5), the symmetric map.
 *   STRATA_MOE_Q2_0:   w = d * (q - 1), the map of the pages' own Q2_0 packs
 *                      (Strata compare page, moe_fused.hpp header comment).
 * Both use the same packed layout (strata_moe_pack); the format only changes
 * the arithmetic of the layer. */
#define STRATA_MOE_Q2_SYM 1
#define STRATA_MOE_Q2_0 2

/* A layer's experts, resident in device memory.  The blobs are written by
 * strata_moe_pack() in the kernels' own layout (not a GGUF layout).
 *   gate_up: E blobs of gate_up_stride bytes, expert e at gate_up + e*stride,
 *            holding the stacked [gate; up] matrix (2I rows x H, reduction
 *            over H), from which expert e's SwiGLU input is computed.
 *   down:    E blobs of down_stride bytes (H rows x I, reduction over I).
 *   router_bias: [E] fp32 added to the router logits before the top-K and
 *            the softmax, or NULL.
 *   router_prepared: strata_moe_prepare_router()'s output for the router_w
 *            that the layer calls pass, or NULL (then the layer prepares
 *            router_w on every call).  Added after the fields above; code
 *            that zero-initialises the struct keeps the per-call path.
 *   shared_gate: [H] fp32, or NULL for no shared expert.  When set, the
 *            blobs hold E + 1 experts and the last one (index E) is the
 *            layer's shared expert: every token also goes through it, and
 *            its output is added with the token's scalar gate
 *            g = sigmoid(x . shared_gate), computed in fp32 (the shared expert
 *            and its scalar gate in the MoE half of Prefill::run, prefill.cpp
 *            page; the pages do not print how the two outputs are combined,
 *            and this is the sigmoid-gated sum).  The shared expert takes the
 *            routed experts' path: int8 input, gate/up, SwiGLU, int8 H, down.
 *            It is pair slot K of every token, so with it K <= 15 and
 *            E <= 1023.  Code that zero-initialises the struct has none.
 *   flags:   0 (the default), or a sum of the STRATA_MOE_FLAG_ values below;
 *            they pick among kernels that compute the same layer (A/B
 *            measurements).  Added last; zero-initialised code keeps 0. */
typedef struct strata_moe_experts {
    int32_t n_expert; /* E */
    int32_t hidden;   /* H */
    int32_t ffn;      /* I */
    int32_t format;   /* STRATA_MOE_Q2_SYM or STRATA_MOE_Q2_0 */
    const void* gate_up;
    int64_t gate_up_stride;
    const void* down;
    int64_t down_stride;
    const float* router_bias;
    const void* router_prepared;
    const float* shared_gate;
    int32_t flags;
} strata_moe_experts;

/* Kernel choice for short chunks.  Where the call gives the experts at most
 * two routed rows each on average (n = T * K pairs over E experts, n <= 2 E:
 * decode-window sizes), chunks of at most 8 rows go to a GEMV kernel on int8
 * dot products (two rows per pass over the weights) and the rest to the
 * small-chunk MFMA kernel; otherwise every chunk takes an MFMA kernel.
 * STRATA_MOE_FLAG_NO_GEMV keeps every chunk on the MFMA kernels;
 * STRATA_MOE_FLAG_GEMV_ALWAYS gives the GEMV its chunks at any average. */
#define STRATA_MOE_FLAG_NO_GEMV 1
/* The per-slot q8_1 arm (the pages' MMQ form, Strata compare page,
 * moe_fused.hpp header comment): for the GEMV's chunks the layer input is
 * rounded to int8 again per routed slot, with each block's code sum, and the
 * weight offset comes from those sums.  The same codes as the per-token
 * rounding; only the data flow differs.  No effect where the GEMV does not
 * run. */
#define STRATA_MOE_FLAG_PER_SLOT_Q8 2
#define STRATA_MOE_FLAG_GEMV_ALWAYS 4

/* Optional intermediate outputs of strata_moe_prefill_debug (each may be
 * NULL; all device pointers, sized for T tokens).  The library's own buffers
 * are copied into them after the layer has run.  With a shared expert every
 * K below reads K + 1 and E reads E + 1: pair slot K of token t is the shared
 * expert (id E, p = its gate). */
typedef struct strata_moe_debug {
    int32_t* ids;     /* [T][K] routed experts, rank order */
    float* p;         /* [T][K] routing weights */
    int32_t* offsets; /* [E+1] first grouped row of each expert */
    int32_t* src;     /* [T*K] token of each grouped row */
    int32_t* slot;    /* [T*K] grouped row of pair i = t*K + k */
    int8_t* qx;       /* [T][H] int8 codes of the layer input */
    float* sx;        /* [T][H/32] their scales */
    int8_t* qh;       /* [T*K][I] int8 codes of the SwiGLU output, grouped rows */
    float* sh;        /* [T*K][I/32] their scales */
} strata_moe_debug;

/* ---------------------------------------------------------------- queries */

/* 1 if the current HIP device is gfx950 (this library's only target), else 0. */
int strata_moe_device_supported(void);

/* Message for the last non-zero return on this host thread ("" if none). */
const char* strata_moe_last_error(void);

/* Bytes of one expert's packed gate/up blob and down blob for (H, I); the
 * caller allocates E times each (the strides passed in strata_moe_experts
 * must be at least these, multiples of 256). */
int strata_moe_packed_bytes(int32_t hidden, int32_t ffn, int64_t* gate_up_bytes, int64_t* down_bytes);

/* Device workspace a strata_moe_prefill call of T tokens needs. */
int strata_moe_workspace_bytes(int64_t T, int32_t K, const strata_moe_experts* experts, size_t* bytes);

/* Hand the library a caller-owned device workspace for the current device
 * (NULL/0 returns to library-owned, lazily grown workspace).  Calls whose need
 * exceeds it fail with STRATA_MOE_ENOMEM. */
int strata_moe_set_workspace(void* dev_ptr, size_t bytes);

/* ---------------------------------------------------------------- packing */

/* Pack experts [e0, e1) from canonical device arrays into the kernels' blobs.
 *   codes_gu  uint8 [e1-e0][2I][H]     gate rows 0..I-1 then up rows, codes 0..3
 *   scales_gu uint16 [e1-e0][2I][H/32] fp16 bit patterns
 *   codes_d   uint8 [e1-e0][H][I]
 *   scales_d  uint16 [e1-e0][H][I/32]
 * Expert e is written at gate_up + e*gate_up_stride and down + e*down_stride.
 * Codes above 3 are masked to their low 2 bits.  Asynchronous on `stream`. */
int strata_moe_pack(const uint8_t* codes_gu, const uint16_t* scales_gu, const uint8_t* codes_d,
                    const uint16_t* scales_d, int32_t e0, int32_t e1, int32_t hidden, int32_t ffn, void* gate_up,
                    int64_t gate_up_stride, void* down, int64_t down_stride, void* stream);

/* The inverse of strata_moe_pack for experts [e0, e1) (round-trip checks). */
int strata_moe_unpack(const void* gate_up, int64_t gate_up_stride, const void* down, int64_t down_stride, int32_t e0,
                      int32_t e1, int32_t hidden, int32_t ffn, uint8_t* codes_gu, uint16_t* scales_gu,
                      uint8_t* codes_d, uint16_t* scales_d, void* stream);

/* Device bytes of a prepared router matrix of H x E.  Errors: EINVAL for H
 * not a multiple of 128 in [128, 4096] or E outside [1, 1024]. */
int strata_moe_router_prepared_bytes(int32_t hidden, int32_t n_expert, size_t* bytes);

/* The router matrix's per-call forms, computed once (Winery-Strata
 * prefill.cpp page, the router step: the logits are x . W_r; the layer builds
 * from W_r a transposed fp32 copy for the fp64 re-score of near-ties and the
 * hi/lo fp16 MFMA operand).  router_w [H][E] fp32 (device); prepared:
 * caller-owned device memory of strata_moe_router_prepared_bytes() bytes,
 * 256-byte aligned.  Point experts->router_prepared at it and pass the same
 * router_w to the layer calls; prepare again whenever router_w changes (the
 * layer does not check).  Asynchronous on `stream`. */
int strata_moe_prepare_router(const float* router_w, int32_t hidden, int32_t n_expert, void* prepared, void* stream);

/* ------------------------------------------------------------- the layer */

/* The whole routed-expert layer for T tokens.
 *   x        [T][H] fp32 layer input (row-major)
 *   router_w [H][E] fp32 router matrix (column e is expert e's router vector)
 *   out      [T][H] fp32, overwritten with y[t] = sum_k p[t][k] * down_e(...)
 * The down GEMM writes each routed row's weighted output to its grouped row;
 * the combine adds a token's K rows in k order, so results are bitwise
 * reproducible from run to run. */
int strata_moe_prefill(const float* x, const float* router_w, const strata_moe_experts* experts, int64_t T,
                       int32_t K, float* out, void* stream);

/* strata_moe_prefill for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same launches as strata_moe_prefill, but the workspace is
 * a fixed device array of STRATA_MOE_NOALLOC_SCRATCH_BYTES inside the
 * library (one per GPU, held until the process ends), so the call allocates
 * and frees nothing.  A call whose workspace (strata_moe_workspace_bytes)
 * exceeds it fails with EINVAL and enqueues nothing: at H = 2560, I = 1024,
 * E = 512, K = 10 that is above 2,246 tokens.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams,
 * other host threads) race and must not be made.  Nothing in the array needs
 * to start at zero; the flags a call relies on are cleared by its own first
 * kernel. */
#define STRATA_MOE_NOALLOC_SCRATCH_BYTES ((size_t)512 << 20)
int strata_moe_prefill_noalloc(const float* x, const float* router_w, const strata_moe_experts* experts, int64_t T,
                               int32_t K, float* out, void* stream);

/* strata_moe_prefill, then the intermediates copied into `dbg` (host struct
 * of device pointers). */
int strata_moe_prefill_debug(const float* x, const float* router_w, const strata_moe_experts* experts, int64_t T,
                             int32_t K, float* out, const strata_moe_debug* dbg, void* stream);

/* ------------------------------------------- single steps (parity checks) */

/* Router logits and route() (Winery-Strata prefill.cpp page, Prefill::run,
 * MoE half: the router projection, then route(logits, ids, w); the body of
 * route() is not printed, and the reading is the K largest logits with a
 * softmax over them): ids [T][K] int32 in rank order (ties -> lower expert
 * index), p [T][K] fp32 = softmax over the K selected logits.  x [T][H] fp32,
 * router_w [H][E] fp32, bias [E] or NULL.  Near-ties are settled in fp64, so
 * the ids are those of the exact logits.  Errors: EINVAL for sizes or NULL
 * pointers, EHIP for a failed launch. */
int strata_moe_route(const float* x, const float* router_w, const float* bias, int64_t T, int32_t H, int32_t E,
                     int32_t K, int32_t* ids, float* p, void* stream);

/* Grouping of the (token, k) pairs by expert (Strata compare page,
 * moe_fused.hpp, group(): slot[i] = the row of pair i, src[row] = its token,
 * the rows of each expert contiguous; the order inside an expert, left open
 * there, is ascending pair index here).  ids [T][K] int32 (device); offsets
 * [E+1], src [T*K], slot [T*K] (device, written).  Synchronises `stream` to
 * check the ids; returns STRATA_MOE_EDATA if any id is outside [0, E). */
int strata_moe_group(const int32_t* ids, int64_t T, int32_t K, int32_t E, int32_t* offsets, int32_t* src,
                     int32_t* slot, void* stream);

/* Per-32 int8 rounding of fp32 rows (Strata compare page, moe_fused.hpp,
 * quantize_act: int8 codes with one scale per 32 values; the rounding rule,
 * not printed there, is the reading below): v [rows][cols] fp32 (cols a
 * multiple of 32, 16-byte aligned), codes [rows][cols] int8, scales
 * [rows][cols/32] fp32; s = max|v|/127 (fp32), q = round-half-away(v/s),
 * both divisions IEEE fp32.  Errors: EINVAL for sizes, alignment or NULL. */
int strata_moe_quantize(const float* v, int64_t rows, int32_t cols, int8_t* codes, float* scales, void* stream);

/* Gate/up + SwiGLU + int8 H for grouped rows (Strata compare page,
 * moe_fused.hpp, experts(): gate/up on the int8 input rows of each expert
 * through src, SwiGLU, H rounded to int8 per 32 values in the epilogue): qx
 * [T][H] int8 / sx [T][H/32] fp32 from strata_moe_quantize of the layer
 * input, offsets [E+1] / src [T*K] from strata_moe_group (all device); writes
 * qh [T*K][I] int8 and sh [T*K][I/32] fp32 by grouped row.  Errors: those of
 * strata_moe_prefill's size checks. */
int strata_moe_gate_up(const int8_t* qx, const float* sx, const int32_t* offsets, const int32_t* src, int64_t T,
                       int32_t K, const strata_moe_experts* experts, int8_t* qh, float* sh, void* stream);

/* Down + combine from given H codes (Strata compare page, moe_fused.hpp,
 * experts(): down into the per-slot rows that the combine reads): qh
 * [T*K][I] int8 / sh [T*K][I/32] fp32 by grouped row, offsets / src / slot
 * from strata_moe_group, p [T][K] fp32 (all device); out [T][H] fp32 is
 * overwritten with sum_k p[t][k] * down(qh[slot[t*K+k]]), k ascending.
 * Errors: those of strata_moe_prefill's size checks. */
int strata_moe_down(const int8_t* qh, const float* sh, const int32_t* offsets, const int32_t* src,
                    const int32_t* slot, const float* p, int64_t T, int32_t K, const strata_moe_experts* experts,
                    float* out, void* stream);

/* ------------------------------------------------------ streamed experts */

/* A ring of device slots through which a layer's experts stream from pinned
 * host memory while the layer runs (Winery-Strata prefill.cpp page: the
 * streamed ring described in the comments at the top of the file, and the
 * fused batch loop in the MoE half of Prefill::run).  Entry k of the stream
 * (counted across calls) lands in slot k % n_slots by a host-to-device copy
 * on the ring's copy stream; a per-slot "copied" event gates the launches
 * that read the slot, and a per-slot "used" event, recorded on the compute
 * stream after them, gates the next copy into it.  Opaque; one ring serves
 * one compute stream at a time (calls on it must not overlap). */
typedef struct strata_moe_ring strata_moe_ring;

/* Device bytes of a ring of n_slots expert slots for (H, I): n_slots times
 * one expert's gate/up plus down blob (strata_moe_packed_bytes).  Errors:
 * EINVAL for n_slots outside [1, 65536] or H, I as strata_moe_packed_bytes. */
int strata_moe_ring_bytes(int32_t n_slots, int32_t hidden, int32_t ffn, size_t* bytes);

/* A ring over caller-owned device memory `slots` (at least
 * strata_moe_ring_bytes, 256-byte aligned; the caller frees it after
 * strata_moe_ring_destroy).  copy_stream: a hipStream_t of its own (not
 * NULL, not the compute stream; default priority), on which every expert DMA
 * is enqueued.  The library owns the ring object and its 2 x n_slots events.
 * Errors: EINVAL for bad sizes, pointers or a NULL stream; EHIP if an event
 * cannot be created. */
int strata_moe_ring_create(int32_t n_slots, int32_t hidden, int32_t ffn, void* slots, size_t slot_memory_bytes,
                           void* copy_stream, strata_moe_ring** ring);

/* Waits for the ring's last copy and use, then frees the ring object (not the
 * slot memory).  NULL is a no-op. */
int strata_moe_ring_destroy(strata_moe_ring* ring);

/* The layer of strata_moe_prefill with every expert streamed through `ring`:
 * experts->gate_up is pinned host memory (hipHostMalloc) holding expert e's
 * gate/up blob at gate_up + e * S and its down blob right after it, at
 * experts->down + e * S, with S = gate_up_stride = down_stride = one ring
 * slot (gate/up bytes + down bytes of strata_moe_packed_bytes): the layout
 * strata_moe_pack writes with those pointers and strides.  With a shared
 * expert it is entry E.  The experts are walked in id order in batches of at
 * most n_slots / 3 (at least 1): each batch's launches wait for its last
 * copy, and up to n_slots later experts are in flight meanwhile.  The output
 * is bitwise the resident layer's (the same kernels over the same chunks).
 * Asynchronous on `stream` and the ring's copy stream; the host blobs must
 * stay unchanged until the copies are done.  Errors: those of
 * strata_moe_prefill, plus EINVAL for a ring of another device or shape, a
 * host layout other than the one above, or blobs that are not pinned. */
int strata_moe_prefill_streamed(const float* x, const float* router_w, const strata_moe_experts* experts,
                                strata_moe_ring* ring, int64_t T, int32_t K, float* out, void* stream);

/* ----------------------------------------------------------------- timing */

/* Per-kernel GPU timing with HIP events on the launch stream.  enable=1
 * starts a session of at most `max_calls` layer calls (events are recorded
 * around each kernel of each call); enable=0 ends it and frees the events. */
int strata_moe_timing(int enable, int32_t max_calls);
/* Number of kernel kinds the timing reports and the name of kind `id`. */
int strata_moe_timing_kinds(void);
const char* strata_moe_timing_name(int id);
/* Waits for the recorded events, then writes for each kind the total
 * milliseconds and the number of launches timed so far in the session. */
int strata_moe_timing_read(double* total_ms, int32_t* launches, int n);

#ifdef __cplusplus
}
#endif

#endif /* STRATA_MOE_H */
