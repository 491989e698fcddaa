/*
 * moe_q4.h -- C ABI of libmoe_q4.so: the routed int4 MoE expert layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (web pages on the Fish Audio Drama 3 4-bit builds):
 *   - 256 routed experts per layer hold most of the model's parameters and set
 *     its speed (drama-rs page, "Experts: where they run");
 *   - each expert has gate, up and down projections (NVFP4 routed experts card,
 *     "Quantization");
 *   - expert weights are int4, asymmetric, group 64 along the input dimension,
 *     with an f16 scale and an f16 min per group (drama-q4 card, "What's
 *     quantized"), an affine map w = scale * q + min (drama-rs page,
 *     "Apple Silicon (MLX)"), or int4 symmetric with one f16 scale per 128
 *     input weights (drama-3-w4a16 card, "At a glance", "How it was made");
 *   - the router is bf16 (drama-q4 card, "What's quantized");
 *   - rows are grouped by routed expert before the expert products (drama-rs
 *     page, "Apple Silicon (MLX)" and "Layout": grouped MoE prefill).
 * The pages leave the routing function, the activation and the combine open;
 * this library computes: bf16 logits, the k largest (ties to the lower expert
 * index), gates = softmax over the k selected logits, SwiGLU experts
 * h = silu(Wg x) * (Wu x), o = Wd h, and y[t] = sum_i gate[t][i] * o(t, i).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library keeps none of them after the call returns.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream).  Nothing is synchronised, no device memory is allocated and no
 *     value is read back to the host.  Inputs must stay valid, and the
 *     workspace untouched, until the stream has passed the call.  Calls that
 *     share a workspace must be ordered on one stream.
 *   - Arguments are checked on the host before anything is launched; a
 *     negative status is returned and nothing is enqueued on failure.  A
 *     launch failure reported by the HIP runtime returns MOE_Q4_ERR_HIP.
 *     Faults inside kernels surface at the caller's next synchronisation.
 *   - T = 0 returns MOE_Q4_OK without launching anything.
 *   - bf16 and f16 tensors are passed as raw 16-bit patterns.
 *   - x, y, x_out, residual_y and the packed code arrays must be 16-byte
 *     aligned, the scale arrays 4-byte aligned; otherwise the call returns
 *     MOE_Q4_ERR_INVALID_ARG.
 *   - Expert indices read from device memory are clamped into [0, E) by every
 *     kernel, so malformed indices give undefined numbers but stay in bounds.
 *
 * Supported shapes: 1 <= E <= 1024, 1 <= k <= min(E, 32), T * k < 2^31;
 * hidden H and inter I are powers of two in [64, 2048] and multiples of the
 * group (64 asym, 128 sym); moe_q4_prefill additionally needs I % 128 == 0
 * and H % 256 == 0, T * H, T * k * I and T * k * H below 2^31 (so are the calls of
 * moe_q4_forward that take the prefill path).  Other shapes return
 * MOE_Q4_ERR_UNSUPPORTED.
 */
#ifndef MOE_Q4_H
#define MOE_Q4_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MOE_Q4_API __attribute__((visibility("default")))
#else
#define MOE_Q4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
struct ihipStream_t;
typedef struct ihipStream_t *moe_q4_stream;

typedef enum {
    MOE_Q4_ASYM_G64 = 0,   /* w = scale * q + min, q in 0..15, group 64 along K  */
    MOE_Q4_SYM_G128 = 1,   /* w = scale * (q - 8), q in 0..15, group 128 along K */
    MOE_Q4_FP8_B128 = 2,   /* w = e4m3(q) * scale, one float scale per 128 x 128 block */
    MOE_Q4_NVFP4 = 3       /* w = e2m1(q) * e4m3(scale) * global, scale per 16 along K */
} moe_q4_format;

typedef enum {
    MOE_Q4_OK = 0,
    MOE_Q4_ERR_INVALID_ARG = -1,   /* NULL pointer, negative size, k > E, ...   */
    MOE_Q4_ERR_UNSUPPORTED = -2,   /* valid but outside the supported shapes  */
    MOE_Q4_ERR_WORKSPACE = -3,     /* ws NULL or smaller than moe_q4_workspace_size */
    MOE_Q4_ERR_HIP = -4            /* the HIP runtime refused a launch          */
} moe_q4_status;

typedef enum {
    MOE_Q4_WS_ROUTE = 0,
    MOE_Q4_WS_DECODE = 1,
    MOE_Q4_WS_PREFILL = 2,
    MOE_Q4_WS_GROUP = 3,
    MOE_Q4_WS_FORWARD = 4,
    MOE_Q4_WS_SHARED = 5,   /* moe_q4_shared: pass the shared expert's H and I */
    MOE_Q4_WS_FORWARD_DET = 6  /* moe_q4_forward_det */
} moe_q4_ws_kind;

/*
 * One MoE layer's routed experts, canonical layout (all device pointers):
 *   gate_q, up_q   uint8 [E][I][H/2]   packed codes, row n = output n, input k
 *                                      at byte k/2, low nibble for even k
 *   down_q         uint8 [E][H][I/2]   same packing, row d = output d
 *   *_sm           f16 bit patterns:
 *                    asym g64:  [E][N][K/64][2] = {scale, min}
 *                    sym g128:  [E][N][K/128]   = scale
 *                  (N, K) = (I, H) for gate and up, (H, I) for down.
 * Block FP8 (MOE_Q4_FP8_B128; the released experts' format: drama-3-w4a16
 * card, "At a glance", each matrix dequantised with its 128 x 128 block
 * scales, "How it was made"):
 *   *_q            uint8 [E][N][K], one OCP E4M3 code per weight
 *   *_sm           point to float32 [E][N/128][K/128] block scales (cast to
 *                  the field's type)
 * Block FP8 needs H and I of at least 128.  Its codes are converted to
 * 16-bit floats exactly; the decode GEMVs use exact products with fp32 sums
 * (block scale on each 32-code partial sum), the prefill GEMMs run bf16 (x
 * as given) and f16 (h) matrix cores with the block scales applied by
 * rescaling the fp32 accumulators at each 128-input block.
 * NVFP4 (MOE_Q4_NVFP4; drama-3-nvfp4 card, "Quantization": packed E2M1
 * values, one E4M3 scale per 16 input weights, a float32 global scale per
 * matrix, gate and up sharing theirs within an expert):
 *   *_q            uint8 [E][N][K/2], E2M1 codes packed as the int4 formats
 *   *_sm           point to uint8 [E][N][K/16] E4M3 block scales
 *   global_scale   float [E][2] = {gate and up, down} (required; NULL for the
 *                  other formats); 4-byte aligned
 * Codes times block scales are exact in bf16 and f16; the decode GEMVs take
 * exact products with fp32 sums, the prefill GEMMs run f16 matrix cores on
 * the exact weights; the global scale multiplies each output.
 */
typedef struct moe_q4_layer {
    int32_t num_experts;   /* E */
    int32_t hidden;        /* H */
    int32_t inter;         /* I */
    int32_t format;        /* moe_q4_format */
    const uint8_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_sm, *up_sm, *down_sm;
    const float *global_scale;   /* NVFP4 only (see below), else NULL */
    const void *prefill_pack;    /* NULL, or the prefill copy (see moe_q4_prefill_pack) */
} moe_q4_layer;

/*
 * A layer's shared expert: a SwiGLU MLP every token passes through, beside
 * the routed experts.  Its linears are int8, symmetric, with one f16 scale per
 * 128 input weights (drama-q4 card, "What's quantized"), w = scale * q with q
 * the signed byte.  All device pointers:
 *   gate_q, up_q   int8 [I][H]   row n = output n, input k contiguous
 *   down_q         int8 [H][I]   row d = output d
 *   gate_s, up_s   f16 bit patterns [I][H/128]; down_s [H][I/128]
 * hidden H and inter I: powers of two in [128, 2048].  Code arrays 16-byte
 * aligned, scale arrays 2-byte aligned.
 */
typedef struct moe_q4_shared_expert {
    int32_t hidden;   /* H */
    int32_t inter;    /* I */
    const int8_t *gate_q, *up_q, *down_q;
    const uint16_t *gate_s, *up_s, *down_s;
} moe_q4_shared_expert;

/*
 * Prefill copy of a layer's routed weights.  The prefill GEMMs read, per
 * K-step of 64 inputs, 32 bytes of codes (64 for block FP8) from each of a
 * tile's 256 weight rows; in the canonical layout those are 256 separate
 * cache lines per step.  The copy stores each (expert, column block, K-step)
 * tile contiguously, so one step of a tile is 8 KB of consecutive codes plus
 * 1 KB of consecutive scale words (block FP8: 16 KB of codes).  It is made once per set of weights (a
 * reordering, bit for bit: the results of the prefill path are the same with
 * or without it) and then set in the layer's `prefill_pack` field; the
 * decode path reads the canonical arrays either way.
 *
 * Layout of the copy (bytes from its start; E, H, I as the layer):
 *   gate|up codes  [E][I/128][H/64][256][32] at 0: column block c holds gate
 *                  rows 128c .. 128c+127 (slots 0-127) and the same up rows
 *                  (slots 128-255); a slot's two 16-byte halves are swapped
 *                  when bit 3 of the slot index is set.
 *   gate|up scales [E][I/128][H/64][256] uint32 at E*I*H: for K-step j and
 *                  slot r, the 4-byte-aligned word of the row's canonical
 *                  scale array that holds its group 64j/G entry, both f16
 *                  halves multiplied by 2^L of the slot's row (one rounding;
 *                  int4 formats, see the lifts below).
 *   down codes     [E][H/256][I/64][256][32] at 9*E*I*H/8: block c holds
 *                  down rows 256c .. 256c+255, halves swapped as above.
 *   down scales    [E][H/256][I/64][256] uint32 at 13*E*I*H/8, as above.
 *   gate|up lifts  [E][I/128][256] int8 at 27*E*I*H/16 (int4 formats only):
 *                  L = 10 - floor(log2 A) of each slot's row, A the largest
 *                  magnitude among the row's f16 scales and mins (0 if A is
 *                  0); the GEMM multiplies the row's outputs by 2^-L.
 *   down lifts     [E][H/256][256] int8 after them (int4 formats only).
 * Total 27*E*I*H/16 bytes, plus 2*E*I + E*H for the int4 formats
 * (moe_q4_prefill_pack_size); dst 256-byte aligned.
 * Block FP8: codes only (its block scales are read from the canonical array):
 *   gate|up codes  [E][I/128][H/64][256][64] at 0, down codes
 *                  [E][H/256][I/64][256][64] at 2*E*I*H; a slot's four
 *                  16-byte quarters q are stored at q ^ ((slot >> 2) & 3).
 *   Total 3*E*I*H bytes.
 */
MOE_Q4_API size_t moe_q4_prefill_pack_size(const moe_q4_layer *w);

/* Writes the prefill copy of w's weights (w->prefill_pack is ignored) to
 * dst on `stream`.  MOE_Q4_ERR_UNSUPPORTED for shapes the prefill path does
 * not take; MOE_Q4_ERR_INVALID_ARG when dst is NULL,
 * misaligned or smaller than moe_q4_prefill_pack_size(w).  The copy stays
 * valid while the canonical weights are unchanged. */
MOE_Q4_API int moe_q4_prefill_pack(const moe_q4_layer *w, void *dst, size_t dst_bytes, moe_q4_stream stream);

/* Bytes of workspace the call of kind `which` needs for these sizes (0 if
 * none).  The value covers both weight formats. */
MOE_Q4_API size_t moe_q4_workspace_size(int which, int64_t T, int32_t E, int32_t k, int32_t H, int32_t I);

/*
 * Router and top-k.
 *   x         bf16 [T][H] or NULL.  When x != NULL the logits
 *             logits[t][e] = bf16(float(sum_h x[t][h] * Wr[e][h] + bias[e]))
 *             are computed with a double-precision sum and WRITTEN to
 *             `logits`; when x == NULL, `logits` is READ as given.
 *   router_w  bf16 [E][H] (required when x != NULL)
 *   bias      float [E] or NULL (added before rounding; the pages describe no
 *             router bias, it exists to shape synthetic expert popularity)
 *   logits    bf16 [T][E], output or input as above
 *   topk_idx  int32 [T][k] out: the k largest logits, descending, equal
 *             logits ordered by lower expert index
 *   topk_gate float [T][k] out: exp(l_i - l_0) / sum_j exp(l_j - l_0) over
 *             the selected, computed in double and rounded once
 *   ws        unused (may be NULL)
 */
MOE_Q4_API int moe_q4_route(const void *x, const void *router_w, const float *bias, void *logits,
                 int64_t T, int32_t H, int32_t E, int32_t k,
                 int32_t *topk_idx, float *topk_gate,
                 void *ws, size_t ws_bytes, moe_q4_stream stream);

/*
 * Grouping of the T*k (token, slot) pairs by routed expert (a stable
 * counting sort; drama-rs page "Apple Silicon (MLX)": prefill groups rows by
 * routed expert).  Outputs (int32, device):
 *   cnt[E]       pairs routed to each expert
 *   off[E+1]     exclusive prefix sum of cnt, off[E] = T*k
 *   perm[T*k]    pair index t*k+i at sorted position r, pairs of one expert in
 *                (t, i) order
 *   inv[T*k]     sorted position of pair t*k+i
 * ws: at least moe_q4_workspace_size(MOE_Q4_WS_GROUP, ...) bytes.
 */
MOE_Q4_API int moe_q4_group(const int32_t *topk_idx, int64_t T, int32_t k, int32_t E,
                 int32_t *cnt, int32_t *off, int32_t *perm, int32_t *inv,
                 void *ws, size_t ws_bytes, moe_q4_stream stream);

/*
 * Expert layer for few tokens (tuned for T <= 64): grouping (which also
 * clears y), then two kernels of fused-dequant GEMVs that stream the active
 * experts' packed nibbles once: gate and up with SwiGLU in fp32 into h
 * (workspace, fp32), then the down GEMV over full rows with each row of h
 * scaled by a power of two (its largest magnitude into [2^14, 2^15)) and
 * rounded to f16, so f16's range does not limit h; the outputs are
 * multiplied by the gate and the inverse power of two and added into y with
 * float atomics (y may differ between runs in the last bits).  The group
 * scale and min are applied exactly in fp32 (drama-q4 card, "What's
 * quantized": scale and min per group of 64; drama-3-w4a16 card: scale per
 * 128).
 *   x          bf16 [T][H]
 *   topk_idx   int32 [T][k], topk_gate float [T][k] (as from moe_q4_route)
 *   w          the layer (host struct holding device pointers)
 *   y          float [T][H] out
 *   ws         >= moe_q4_workspace_size(MOE_Q4_WS_DECODE, T, E, k, H, I) bytes
 */
MOE_Q4_API int moe_q4_decode(const void *x, const int32_t *topk_idx, const float *topk_gate,
                  int64_t T, int32_t k, const moe_q4_layer *w, float *y,
                  void *ws, size_t ws_bytes, moe_q4_stream stream);

/*
 * Expert layer for many tokens (tuned for T >= 64): grouping, then grouped
 * GEMMs on the f16 matrix cores with fp32 accumulation.  Each x row is scaled
 * by a power of two and converted to f16 exactly (elements more than 2^31
 * below the row's largest magnitude may round); int4 weights are
 * dequantised to f16 in registers with one rounding each (s q + m, or
 * s (q - 8)), each weight row lifted by the power of two that puts it below
 * 2^15 and keeps its groups' scale / 16 normal (groups more than 2^24 below
 * the row's largest scale lose precision; FP8 and NVFP4 codes enter
 * exactly); h between the two products and each routed row's gate-weighted
 * down output are rounded to f16 after scaling by a power of two chosen per
 * block, after each row's 2^-2e with 2^e the power of two of its token's x
 * (h: 128 columns of I, one exponent for all rows of a work tile; the
 * down output: 32 rows by 64 columns of H) that puts the block's largest
 * magnitude into [2^14, 2^15), so f16's range limits none of them, and a
 * token's k rows are summed in fp32 into y (float
 * [T][H], written whole; deterministic).  Same arguments
 * as moe_q4_decode; ws >= moe_q4_workspace_size(MOE_Q4_WS_PREFILL, ...).
 */
/* With w->prefill_pack set the GEMMs read that copy instead of the
 * canonical codes and scale words; the results are identical. */
MOE_Q4_API int moe_q4_prefill(const void *x, const int32_t *topk_idx, const float *topk_gate,
                   int64_t T, int32_t k, const moe_q4_layer *w, float *y,
                   void *ws, size_t ws_bytes, moe_q4_stream stream);

/*
 * Whole layer in one call: routing (router GEMV when router_w != NULL, else
 * the given logits), top-k gates, grouping and the experts, y float [T][H].
 * For T <= 64 (and T*k <= 1024) this is three kernel launches: routing, the
 * gate/up GEMV and the down GEMV.  With at most 64 (token, slot) pairs and
 * E <= 256 every gate/up workgroup takes the top-k and grouping itself from
 * the logits; otherwise the routing launch does them in its last workgroup
 * to finish.  Larger T takes the prefill path.
 *   residual_y  float [T][H] or NULL.  When given, the layer input is the
 *               residual step bf16(float(x) + residual_y) of a chain of layers
 *               (as moe_q4_residual_bf16), written to x_out (bf16 [T][H],
 *               required then); y must not alias residual_y.
 *   logits      bf16 [T][E]: written when router_w != NULL, read otherwise.
 *   topk_idx, topk_gate: as moe_q4_route (outputs).
 *   ws          >= moe_q4_workspace_size(MOE_Q4_WS_FORWARD, ...) bytes; its
 *               control block must be cleared once by moe_q4_workspace_init
 *               before the first call (it is left cleared by every call).
 * Results equal moe_q4_route followed by moe_q4_decode (T <= 64) or
 * moe_q4_prefill.
 */
MOE_Q4_API int moe_q4_forward(const void *x, const float *residual_y, void *x_out,
                              const void *router_w, const float *bias, void *logits,
                              int64_t T, int32_t k, const moe_q4_layer *w,
                              int32_t *topk_idx, float *topk_gate, float *y,
                              void *ws, size_t ws_bytes, moe_q4_stream stream);

/*
 * moe_q4_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The workspace is a device array of
 * MOE_Q4_NOALLOC_SCRATCH_BYTES that the library holds for the life of the
 * process, one per GPU (its address is looked up on the first call on each
 * device; the stream must belong to the current device).  No allocation
 * routine is called.  Shapes whose forward workspace
 * (moe_q4_workspace_size(MOE_Q4_WS_FORWARD, T, E, k, H, I)) exceeds
 * MOE_Q4_NOALLOC_SCRATCH_BYTES return MOE_Q4_ERR_WORKSPACE; that covers the
 * decode path (T <= 64) at H, I <= 2048 and E <= 1024.  Every call clears the
 * routing counters with a small kernel on the stream before its launches.
 * All calls on one GPU share the array: calls that overlap on one GPU (two
 * streams, two host threads) race and give wrong results; serialise them.
 * Arguments and results otherwise as moe_q4_forward.
 */
#define MOE_Q4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
MOE_Q4_API int moe_q4_forward_noalloc(const void *x, const float *residual_y, void *x_out,
                                      const void *router_w, const float *bias, void *logits,
                                      int64_t T, int32_t k, const moe_q4_layer *w,
                                      int32_t *topk_idx, float *topk_gate, float *y,
                                      moe_q4_stream stream);

/*
 * moe_q4_forward with the caller's MOE_Q4_STAGE_EVENTS HIP events recorded at
 * the start and end of its two main kernels (extended launch): decode path
 * events[0..1] the gate/up GEMV, events[2..3] the routing launch (grouping
 * launch when the router runs separately); prefill path as
 * moe_q4_prefill_timed.  events must not be NULL.
 */
MOE_Q4_API int moe_q4_forward_timed(const void *x, const float *residual_y, void *x_out,
                                    const void *router_w, const float *bias, void *logits, int64_t T,
                                    int32_t k, const moe_q4_layer *w, int32_t *topk_idx, float *topk_gate,
                                    float *y, void *ws, size_t ws_bytes, moe_q4_stream stream,
                                    void *const *events);

/*
 * moe_q4_forward of a layer with a shared expert (drama-q4 card, "What's
 * quantized": the layer's shared expert, int8 symmetric group 128, beside
 * the routed experts): y[t] = sum_i gate[t][i] * o(t, i) + shared(x_t), the
 * shared output added as is.  shared == NULL is moe_q4_forward; events ==
 * NULL or as moe_q4_forward_timed.  shared->hidden must equal w->hidden.
 * On the decode path the shared expert's work items run inside the two
 * expert launches when shared->inter == w->inter (its down outputs added
 * with float atomics), otherwise in moe_q4_shared's two launches after them;
 * on the prefill path moe_q4_shared's launches follow the combine.
 *   ws  >= moe_q4_workspace_size(MOE_Q4_WS_FORWARD, T, E, k, H, I)
 *          + moe_q4_workspace_size(MOE_Q4_WS_SHARED, T, 1, 1, H, shared->inter)
 */
MOE_Q4_API int moe_q4_forward_ex(const void *x, const float *residual_y, void *x_out, const void *router_w,
                                 const float *bias, void *logits, int64_t T, int32_t k, const moe_q4_layer *w,
                                 const moe_q4_shared_expert *shared, int32_t *topk_idx, float *topk_gate, float *y,
                                 void *ws, size_t ws_bytes, moe_q4_stream stream, void *const *events);

/*
 * moe_q4_forward_ex with a run-to-run bit-identical y on the decode path
 * (drama-rs page, "Tests": every kernel checked against a plain reference;
 * the same input must give the same output).  moe_q4_forward_ex's decode
 * path adds each routed row into y with float atomics, whose order, and so
 * whose last bits, vary between runs.  Here the down launch stores each
 * routed (token, slot) row, gate applied, in the workspace ([T*k][H] fp32),
 * and one more launch sums a token's rows in slot order 0, 1, ..., k-1
 * into y; the shared expert (if any) then runs in moe_q4_shared's own
 * launches and is added last.  The prefill path is the same as
 * moe_q4_forward_ex's (already slot-ordered).  Arguments, layouts and
 * errors as moe_q4_forward_ex, except the workspace:
 *   ws  >= moe_q4_workspace_size(MOE_Q4_WS_FORWARD_DET, T, E, k, H, I)
 *          (+ moe_q4_workspace_size(MOE_Q4_WS_SHARED, ...) with a shared
 *          expert),
 * its control block cleared once by moe_q4_workspace_init.
 */
MOE_Q4_API int moe_q4_forward_det(const void *x, const float *residual_y, void *x_out, const void *router_w,
                                  const float *bias, void *logits, int64_t T, int32_t k, const moe_q4_layer *w,
                                  const moe_q4_shared_expert *shared, int32_t *topk_idx, float *topk_gate, float *y,
                                  void *ws, size_t ws_bytes, moe_q4_stream stream, void *const *events);

/*
 * A decode frame: n_layers MoE layers in sequence over T tokens, the
 * residual chain of the backbone (drama-rs page, "Experts: where they run":
 * the experts of every layer set the speed of a frame), run as `lanes`
 * token lanes side by side.  Every step of the chain works token by token
 * (routing, experts, combine, the residual step), so lane i takes token rows
 * [T*i/lanes, T*(i+1)/lanes) through all n_layers layers on streams[i], and
 * layer j of one lane overlaps layers j - 1 and j + 1 of another: one lane's
 * routing and kernel ramps run beside the other's weight streaming (the
 * pages' engine hides the gaps between its weight-streaming launches by
 * prefetching the next kernel's weights into L2; drama-rs page, "Footprint
 * and speed").  Each lane's expert GEMVs take 1/lanes of the GPU's resident
 * grid.  Measured on MI355X at 16 tokens x 40 layers of 256 experts: two
 * lanes 2.21 ms per frame against 2.30 ms for one; four lanes, or
 * two with whole-GPU grids, were slower.
 *   x          bf16 [T][H]: layer 0's input.
 *   layers     [n_layers]: one shape (E, H, I) for every layer; router_w
 *              [n_layers] bf16 [E][H] router weights (required); shared:
 *              NULL or [n_layers] shared experts of one inner size.
 *   x_chain    bf16 [n_layers - 1][T][H] (out; NULL when n_layers == 1):
 *              entry j - 1 is layer j's input bf16(x_{j-1} + y_{j-1}).
 *   y_chain    float [n_layers][T][H] (out): entry j is layer j's y.
 *   logits     bf16 [n_layers][T][E], topk_idx int32 [n_layers][T][k],
 *   topk_gate  float [n_layers][T][k] (out): each layer's routing.
 *   lanes      1 .. MOE_Q4_FRAME_MAX_LANES, at most T; lanes == 1 is
 *              n_layers moe_q4_forward_ex calls on streams[0].
 *   streams    [lanes] streams.  Inputs must be complete before any of
 *              them reaches the call, and the outputs are complete when all
 *              of them have passed it (the caller orders the streams, e.g.
 *              with events); the lanes share no memory.
 *   ws         >= moe_q4_frame_workspace_size(T, E, k, H, I, shared inter
 *              size or 0, lanes) bytes, untouched until every stream has
 *              passed the call; the call clears its routing counters itself
 *              (no moe_q4_workspace_init needed).
 *   events     NULL, or n_layers * lanes * MOE_Q4_STAGE_EVENTS events:
 *              entries [(j * lanes + i) * MOE_Q4_STAGE_EVENTS, +4) are
 *              recorded as moe_q4_forward_ex's for layer j of lane i.
 * Results equal moe_q4_forward_ex applied layer by layer to each lane's
 * rows.  Every argument of every layer and lane is checked before the first
 * launch; a launch failure after some launches returns MOE_Q4_ERR_HIP with
 * the earlier work enqueued.
 */
#define MOE_Q4_FRAME_MAX_LANES 4
MOE_Q4_API size_t moe_q4_frame_workspace_size(int64_t T, int32_t E, int32_t k, int32_t H, int32_t I,
                                              int32_t shared_inter, int32_t lanes);
MOE_Q4_API int moe_q4_frame(const void *x, int64_t T, int32_t k, int32_t n_layers, const moe_q4_layer *layers,
                            const void *const *router_w, const moe_q4_shared_expert *shared, void *x_chain,
                            float *y_chain, void *logits, int32_t *topk_idx, float *topk_gate, int32_t lanes,
                            const moe_q4_stream *streams, void *ws, size_t ws_bytes, void *const *events);

/* Clears the control block of a workspace used with moe_q4_forward (once,
 * after allocation).  Enqueued on stream. */
MOE_Q4_API int moe_q4_workspace_init(void *ws, size_t ws_bytes, moe_q4_stream stream);

/*
 * Same as moe_q4_decode / moe_q4_prefill; additionally the caller's HIP
 * events (hipEvent_t handles created by the caller) are recorded by the
 * runtime at the start and end of the two main kernels (extended launch), so
 * that hipEventElapsedTime gives exactly those kernels' durations:
 *   decode:  events[0..1] the gate/up GEMV + SwiGLU kernel,
 *            events[2..3] the grouping kernel
 *   prefill: events[0..1] the gate/up grouped GEMM + SwiGLU,
 *            events[2..3] the down grouped GEMM (the combine into y
 *            follows it)
 * events must point to MOE_Q4_STAGE_EVENTS valid events.
 */
#define MOE_Q4_STAGE_EVENTS 4
MOE_Q4_API int moe_q4_decode_timed(const void *x, const int32_t *topk_idx, const float *topk_gate,
                        int64_t T, int32_t k, const moe_q4_layer *w, float *y,
                        void *ws, size_t ws_bytes, moe_q4_stream stream, void *const *events);
MOE_Q4_API int moe_q4_prefill_timed(const void *x, const int32_t *topk_idx, const float *topk_gate,
                         int64_t T, int32_t k, const moe_q4_layer *w, float *y,
                         void *ws, size_t ws_bytes, moe_q4_stream stream, void *const *events);

/*
 * Shared expert for T tokens (the pages name no gate for it, so its output
 * is added as is):
 *   y[t] = (accumulate ? y[t] : 0) + Wd (silu(Wg x_t) * (Wu x_t)).
 * Up to 64 tokens (or H not a multiple of 256): two GEMV launches that
 * stream the int8 codes: gate and up with SwiGLU (products of codes and x
 * exact in fp32, fp32 sums, each 128-group's scale applied to its partial
 * sum) into fp32 h, then the down GEMV, which scales each token's h row by
 * the power of two that puts its largest magnitude in [2^14, 2^15) before
 * rounding it to f16 (exact products of codes and f16 h, fp32 sums, the
 * power of two taken off the result).  From 65 tokens: x scaled per token by
 * a power of two 2^-e into f16 (as moe_q4_prefill), then two dense f16
 * matrix-core GEMMs whose weights are s * q rounded once to f16; h is
 * rounded to f16 between them after scaling each token's row by 2^-2e and
 * each block of 128 h columns of a tile of tokens by a power of two (both
 * taken off in the down GEMM).  So f16's range limits neither x nor h on
 * either path.  y is written by one thread per output (deterministic).
 *   x   bf16 [T][H];  y  float [T][H], read when accumulate != 0
 *   ws  >= moe_q4_workspace_size(MOE_Q4_WS_SHARED, T, 1, 1, H, I) bytes
 * Same conventions as the other entry points; T * H and T * I below 2^31.
 */
MOE_Q4_API int moe_q4_shared(const void *x, int64_t T, const moe_q4_shared_expert *sx, float *y,
                             int32_t accumulate, void *ws, size_t ws_bytes, moe_q4_stream stream);

/* moe_q4_shared with the caller's MOE_Q4_STAGE_EVENTS HIP events recorded at
 * the start and end of its gate/up launch (events[0..1]) and its down launch
 * (events[2..3]) by the runtime (extended launch).  events must not be NULL. */
MOE_Q4_API int moe_q4_shared_timed(const void *x, int64_t T, const moe_q4_shared_expert *sx, float *y,
                                   int32_t accumulate, void *ws, size_t ws_bytes, moe_q4_stream stream,
                                   void *const *events);

/*
 * Test hook: dequantise projection `proj` (0 gate [I][H], 1 up [I][H],
 * 2 down [H][I]) of a shared expert to float [N][K] = float(q) * scale (exact)
 * through the kernels' own code decoding.
 */
MOE_Q4_API int moe_q4_dequant_int8(const moe_q4_shared_expert *sx, int32_t proj, float *out,
                                   moe_q4_stream stream);

/*
 * Test hook: dequantise projection `proj` (0 gate [I][H], 1 up [I][H],
 * 2 down [H][I]) of `expert` to float [N][K] through the kernels' own nibble
 * unpacking and scale indexing: out = float(scale * q + min) (asym) or
 * float(scale * (q - 8)) (sym), one rounding.
 */
MOE_Q4_API int moe_q4_dequant(const moe_q4_layer *w, int32_t expert, int32_t proj, float *out,
                   moe_q4_stream stream);

/* Residual step of a chain of layers: out[i] = bf16(float(x[i]) + y[i]) with
 * one float addition and round-to-nearest-even (x, out: bf16 bits). */
MOE_Q4_API int moe_q4_residual_bf16(const void *x, const float *y, int64_t n, void *out,
                         moe_q4_stream stream);

/* Static description of a status code. */
MOE_Q4_API const char *moe_q4_error_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_Q4_H */
