/*
 * moe.h -- C ABI of libmoe, a routed mixture-of-experts forward for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation ("Experts backends" page, opening paragraph): each token's
 * router scores pick k of the E experts, every picked expert transforms the
 * token's hidden state with its own weights, and the token's output is the
 * sum of those k results, each scaled by its routing weight.  Each expert is a gated MLP (backend table, row
 * deepgemm_megamoe; section "SonicMoE"): a gate and an up projection combined
 * as act(gate) * up, with act = silu (SwiGLU, the default), gelu (GeGLU) or
 * relu (ReGLU) as desc->gate_act selects, then a down projection.  Tokens are first ordered by their
 * selected expert so that all experts run as one grouped GEMM (backend table,
 * rows grouped_mm and deepgemm).
 *
 * Notation: T tokens, H hidden size, I expert intermediate size, E experts,
 * k experts per token, P = T*k (token, slot) pairs.
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     marked "host".  The library never allocates or frees device memory; it
 *     uses only the caller's buffers and the caller's workspace `ws`, sized by
 *     moe_workspace_bytes().  Buffers must stay alive until the stream has
 *     finished the call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     only enqueue work on it: they never synchronise and never read device
 *     memory back to the host, so a whole forward can be captured in a graph.
 *   - All tensors are dense and row-major.  x and out are [T,H]; w_router is
 *     [E,H]; w_gate and w_up are [E,I,H]; w_down is [E,H,I] (each matrix is
 *     [out_features, in_features]).
 *   - Validation happens on the host before anything is launched.  A bad
 *     argument returns MOE_EINVAL, an unsupported combination MOE_EUNSUPPORTED,
 *     a too-small workspace MOE_EWORKSPACE, a failed launch MOE_EHIP; in every
 *     error case nothing has been enqueued.  No C++ exception crosses the ABI.
 *     moe_last_error() describes the last failure of the calling thread.
 *   - T = 0 is valid: the calls write the empty results (zero counts and
 *     offsets) and return MOE_OK.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,          /* bad pointer, shape or enum value */
    MOE_EUNSUPPORTED = 2,    /* valid request this library does not implement */
    MOE_EWORKSPACE = 3,      /* ws is NULL or smaller than moe_workspace_bytes() */
    MOE_EHIP = 4             /* the HIP runtime reported an error at launch */
} moe_status;

/* FP4_E2M1: int8-packed FP4 expert weights (the paragraph under the backend
 * table and section "FP8 and FP4 quantized experts": FP4 experts packed in
 * int8 with UE8M0 scales): OCP e2m1 codes, two per byte along K with the even
 * K index in the low nibble, so w_gate, w_up are [E,I,H/2] bytes and w_down
 * [E,H,I/2]; one UE8M0 scale per row per 32 consecutive K (the OCP MX block;
 * the page gives no FP4 block size): w_gate_scales, w_up_scales [E,I,H/32],
 * w_down_scales [E,H,I/32] bytes.  Weights only (activations are e4m3). */
typedef enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1, MOE_DT_FP8_E4M3 = 2, MOE_DT_FP4_E2M1 = 3 } moe_dtype;

/* Router score, applied to key[e] = x . w_router[e] + router_bias[e].
 * Experts are selected by descending key, ties to the lowest expert index. */
typedef enum {
    MOE_SCORE_SOFTMAX = 0,   /* softmax over all E keys */
    MOE_SCORE_SIGMOID = 1    /* 1 / (1 + exp(-key)) */
} moe_score;

/* FP8 weight block scales (the paragraph under the backend table: float32 or
 * UE8M0 scales).  F32: one float per block.  UE8M0: one byte b per block with
 * value 2^(b-127) (0xff is NaN). */
typedef enum { MOE_SCALE_NONE = 0, MOE_SCALE_F32 = 1, MOE_SCALE_UE8M0 = 2 } moe_scale_fmt;

/* FP8 activation scheme (section "FP8 and FP4 quantized experts": dynamic
 * per-row scales are required, static per-tensor scales are rejected). */
typedef enum { MOE_ACT_NONE = 0, MOE_ACT_DYNAMIC = 1, MOE_ACT_STATIC = 2 } moe_act_scheme;

/* Expert-GEMM strategy (moe_forward and the two expert-GEMM calls).  GROUPED
 * runs tiled grouped GEMMs over the expert-sorted rows; STREAM reads every
 * touched expert's weights exactly once, split over all compute units, for
 * decode-sized batches (section "Decode-stage switching": small token counts
 * want a different scheme); it needs packed weights and T <= 64, and for fp8
 * experts H, I <= 8192 (else MOE_EUNSUPPORTED).  With few touched experts the
 * K range of each weight tile is split over several workgroups and the fp32
 * partial tiles are summed in a fixed order (results depend only on the
 * inputs).  AUTO picks STREAM wherever it applies. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_GROUPED = 1, MOE_PATH_STREAM = 2 } moe_path;

/* Layout of the expert weights passed to the expert GEMMs and moe_forward.
 * ROWMAJOR: w_gate, w_up [E,I,H] and w_down [E,H,I] as described above.
 * PACKED: the tile-contiguous layout written once by moe_pack_weights (a
 * model-load transform): every (expert, 256-row tile, 64-byte K step) is one
 * contiguous 16 KB chunk, so the GEMMs stream weights from HBM in long runs.
 * With PACKED, w_gate is the packed gate/up buffer (gate and up rows of the
 * same channels interleaved per tile), w_up is unused (pass NULL) and w_down
 * is the packed down buffer.  Block scales keep their layout. */
typedef enum { MOE_LAYOUT_ROWMAJOR = 0, MOE_LAYOUT_PACKED = 1 } moe_layout;

/* Gated activation of the expert MLP, h = act(x . w_gate) * (x . w_up)
 * ("Experts backends", section "SonicMoE": experts with a gated activation
 * silu, gelu or relu, i.e. SwiGLU, GeGLU or ReGLU).  SILU: g / (1 + e^-g).
 * GELU: the exact form g * Phi(g) = 0.5 g (1 + erf(g / sqrt 2)) (the page
 * does not say which form).  RELU: max(g, 0).  Zero (the default) is SILU. */
typedef enum { MOE_GATE_SILU = 0, MOE_GATE_GELU = 1, MOE_GATE_RELU = 2 } moe_gate_act;

typedef enum { MOE_PACK_GATE_UP = 0, MOE_PACK_DOWN = 1 } moe_pack_which;

typedef enum {
    MOE_OP_ROUTE = 0, MOE_OP_PERMUTE = 1, MOE_OP_GATE_UP = 2, MOE_OP_DOWN = 3,
    MOE_OP_COMBINE = 4, MOE_OP_FORWARD = 5, MOE_OP_BACKWARD = 6
} moe_op;

/* Layer description (host memory, read during the call only). */
typedef struct moe_desc {
    int64_t T;             /* tokens, >= 0 */
    int32_t H;             /* hidden size, multiple of 16 (of 128 for fp8) */
    int32_t I;             /* expert intermediate size, multiple of 16 (of 128 for fp8) */
    int32_t E;             /* experts, 1..256 */
    int32_t k;             /* experts per token, 1..min(E, 32) */
    int32_t score;         /* moe_score */
    int32_t renormalize;   /* 1: selected scores are divided by their sum */
    float routed_scale;    /* multiplies the final routing weights */
    int32_t act_dtype;     /* MOE_DT_F32 or MOE_DT_BF16: x, w_router and out */
    int32_t w_dtype;       /* expert weights: MOE_DT_F32, MOE_DT_BF16, MOE_DT_FP8_E4M3, MOE_DT_FP4_E2M1 */
    int32_t w_scale_fmt;   /* MOE_SCALE_NONE, or F32 / UE8M0 with FP8 weights, UE8M0 with FP4 */
    int32_t block;         /* FP8 weight block edge and activation group: 128 (FP4: the
                              activation group, 128); else 0 */
    int32_t act_scheme;    /* MOE_ACT_NONE, or MOE_ACT_DYNAMIC with FP8 / FP4 weights */
    int32_t y_dtype;       /* expert-output rows y_sorted: MOE_DT_F32 or MOE_DT_BF16 */
    int32_t path;          /* moe_path */
    int32_t w_layout;      /* moe_layout of the expert weights */
    int32_t gate_act;      /* moe_gate_act of the expert MLPs */
    int32_t reserved[1];   /* must be zero */
} moe_desc;

/* Supported combinations:
 *   act F32  + weights F32            (fp32 everywhere; h is fp32)
 *   act BF16 + weights BF16           (bf16 MFMA, fp32 accumulate; h is bf16)
 *   act BF16 + weights FP8_E4M3, scales F32 or UE8M0, block 128, act DYNAMIC
 *            (x and h are quantized to e4m3 per row per 128 channels with
 *             fp32 scales amax/448; fp8 MFMA, fp32 accumulate, block scales
 *             applied per 128-deep K chunk in fp32)
 *   act BF16 + weights FP4_E2M1, scales UE8M0, block 128, act DYNAMIC, PACKED
 *            layout only (x and h as for FP8; fp8 x fp4 MFMA with the weights'
 *            per-32 scales applied by the MFMA, activation scales per 128-deep
 *            K chunk in fp32; MOE_EUNSUPPORTED for row-major weights)
 * Intermediate h [P,I] is in the expert weight format (bf16/f32), or e4m3
 * codes plus fp32 scales [P,I/128] for FP8 and FP4 experts. */

/* ------------------------------------------------------------------------ */

/* Router (opening paragraph: the router picks k of the E experts per token).
 *   x           [T,H] act_dtype
 *   w_router    [E,H] act_dtype
 *   router_bias [E] fp32, added to the logits before scoring, or NULL
 *   topk_ids    [T,k] int32 out: selected experts, descending key, ties to
 *               the lowest index
 *   topk_w      [T,k] fp32 out: score of each selected expert (softmax over
 *               all E, or sigmoid), divided by the sum of the k selected scores
 *               if desc->renormalize, times desc->routed_scale
 *   ws, ws_bytes  workspace of moe_workspace_bytes(desc, MOE_OP_ROUTE) (bf16:
 *               partial logits of the K slices; fp32 needs none)
 * Logits accumulate in fp32; the K slices are added in a fixed order. */
moe_status moe_route_topk(const moe_desc* desc, const void* x, const void* w_router,
                          const float* router_bias, int32_t* topk_ids, float* topk_w,
                          void* ws, size_t ws_bytes, void* stream);

/* Order (token, slot) pairs by expert (backend table, rows grouped_mm and
 * deepgemm: tokens are ordered / sorted by selected expert).
 *   topk_ids        [T,k] int32 in, values in [0,E) (a pair with an id outside
 *                   that range is left out of counts and perm, and gets
 *                   inv = -1; moe_unpermute_combine skips such pairs)
 *   counts          [E] out: pairs per expert
 *   offsets         [E+1] out: exclusive prefix sum of counts
 *   perm            [P] out: perm[row] = t*k + i, rows of one expert in
 *                   ascending (t, i) order (stable)
 *   inv             [P] out: inv[t*k + i] = row
 *   x, x_sorted     optional gather ([T,H] in, [P,H] out), both NULL or both
 *                   set.  With FP8 weights x_sorted receives e4m3 codes and
 *                   x_sorted_scales [P,H/128] fp32 the dynamic per-row scales;
 *                   otherwise x_sorted has act_dtype and x_sorted_scales is NULL.
 *   ws, ws_bytes    workspace of moe_workspace_bytes(desc, MOE_OP_PERMUTE) */
moe_status moe_permute(const moe_desc* desc, const int32_t* topk_ids, const void* x,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv,
                       void* x_sorted, float* x_sorted_scales,
                       void* ws, size_t ws_bytes, void* stream);

/* Gate/up grouped GEMM with the gated-activation epilogue, all experts in one
 * launch.  Row r of expert e (offsets[e] <= r < offsets[e+1]):
 *   h[r, j] = act(g) * u,  g = x_sorted[r] . w_gate[e, j],  u = x_sorted[r] . w_up[e, j]
 *   act = silu (SwiGLU), gelu (exact erf form, GeGLU) or relu (ReGLU) per
 *   desc->gate_act
 *   x_sorted      [P,H] act_dtype, or e4m3 codes with x_scales [P,H/128] (FP8)
 *   offsets       [E+1] from moe_permute
 *   w_gate, w_up  [E,I,H]; with FP8 also w_gate_scales, w_up_scales
 *                 [E,I/128,H/128] (fp32 or UE8M0 bytes), else NULL
 *   h             [P,I] out: weight format (f32 / bf16), or e4m3 codes with
 *                 h_scales [P,I/128] fp32 (FP8: dynamic per-row quantization)
 *   ws, ws_bytes  workspace of moe_workspace_bytes(desc, MOE_OP_GATE_UP) */
moe_status moe_expert_gate_up_swiglu(const moe_desc* desc, const void* x_sorted,
                                     const float* x_scales, const int32_t* offsets,
                                     const void* w_gate, const void* w_up,
                                     const void* w_gate_scales, const void* w_up_scales,
                                     void* h, float* h_scales,
                                     void* ws, size_t ws_bytes, void* stream);

/* Down-projection grouped GEMM: y_sorted[r, o] = h[r] . w_down[e, o].
 *   h, h_scales   as written by moe_expert_gate_up_swiglu
 *   w_down        [E,H,I]; with FP8 w_down_scales [E,H/128,I/128], else NULL
 *   y_sorted      [P,H] out, desc->y_dtype
 *   ws, ws_bytes  workspace of moe_workspace_bytes(desc, MOE_OP_DOWN) */
moe_status moe_expert_down(const moe_desc* desc, const void* h, const float* h_scales,
                           const int32_t* offsets, const void* w_down,
                           const void* w_down_scales, void* y_sorted,
                           void* ws, size_t ws_bytes, void* stream);

/* Weighted combine back to token order (opening paragraph: the experts'
 * results are summed with the routing weights):
 *   out[t, :] = sum_{i<k} topk_w[t, i] * y_sorted[inv[t*k + i], :]
 * (pairs with inv outside [0, P) are skipped)
 * summed in fp32 in slot order, rounded once to act_dtype.  No atomics: the
 * result is bitwise reproducible. */
moe_status moe_unpermute_combine(const moe_desc* desc, const void* y_sorted,
                                 const int32_t* inv, const float* topk_w, void* out,
                                 void* stream);

/* The whole layer in one call: route, permute, (FP8: quantize x), gate/up +
 * SwiGLU, down, combine.  The gate/up GEMM reads x rows through the
 * permutation, so no sorted copy of x is made.
 *   topk_ids_out, topk_w_out  [T,k] optional copies of the routing (NULL: kept
 *                             in the workspace)
 *   counts_out                [E] optional pairs per expert
 *   ws, ws_bytes              workspace of moe_workspace_bytes(desc, MOE_OP_FORWARD) */
moe_status moe_forward(const moe_desc* desc, const void* x, const void* w_router,
                       const float* router_bias, const void* w_gate, const void* w_up,
                       const void* w_down, const void* w_gate_scales,
                       const void* w_up_scales, const void* w_down_scales, void* out,
                       int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                       void* ws, size_t ws_bytes, void* stream);

/* moe_forward for callers that cannot allocate device memory or hand over a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments and results as moe_forward without
 * ws / ws_bytes: the workspace is carved out of a static device array of
 * MOE_STATIC_SCRATCH_BYTES bytes inside the library, one per device, held from
 * the library's load until the process ends.  The call allocates nothing.
 *   - Layers with moe_workspace_bytes(desc, MOE_OP_FORWARD) above
 *     MOE_STATIC_SCRATCH_BYTES are rejected with MOE_EWORKSPACE (every
 *     decode-sized batch of the Qwen- and DeepSeek-like layers, T <= 64,
 *     and the Qwen-like prefill layer fit; the DeepSeek-like prefill layer
 *     does not).
 *   - The current device must be the stream's device (else MOE_EINVAL).
 *   - Every call on one device shares that device's array, and each call
 *     overwrites what the previous one left there: calls that can overlap on
 *     one device (two host threads, or two streams not ordered by events)
 *     race and must be serialised by the caller.
 *   - No stage timing is recorded for it (moe_timing_*). */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)256 << 20)
moe_status moe_forward_static(const moe_desc* desc, const void* x, const void* w_router,
                              const float* router_bias, const void* w_gate, const void* w_up,
                              const void* w_down, const void* w_gate_scales,
                              const void* w_up_scales, const void* w_down_scales, void* out,
                              int32_t* topk_ids_out, float* topk_w_out, int32_t* counts_out,
                              void* stream);

/* Backward of the whole layer ("Experts backends", section "SonicMoE": the
 * backend built for training gated-MLP experts).  Every gradient of the layer
 * for the output gradient d_out, with the top-k selection held fixed (it is
 * piecewise constant in the inputs):
 *   dw[t,i]     = d_out[t] . y(t,i)                    (routing-weight gradient)
 *   dy          = w[t,i] d_out[t],  da = W_down[e]^T dy
 *   dg          = da * u * act'(g),  du = da * act(g)   (act = desc->gate_act)
 *   dx[t]       = sum_i (W_gate[e]^T dg + W_up[e]^T du) + sum_e dkey[t,e] w_router[e]
 *   dw_gate[e]  = sum over the pairs of e of dg x^T, dw_up[e] = sum du x^T,
 *   dw_down[e]  = sum dy a^T (a = act(g) * u),
 *   dw_router   = dkey^T x,  d_bias = sum_t dkey[t,:]
 * where dkey is the gradient of the router key through the routed scale, the
 * renormalisation (if any) and the score (softmax over all E, or sigmoid).
 * Nothing of the forward is kept: routing, permutation and g, u are
 * recomputed from x and the weights (selection and routing weights come out
 * bitwise identical to moe_forward's).
 *   x, w_router, router_bias, w_gate, w_up, w_down  as for moe_forward (bf16
 *                 activations and bf16 row-major experts only)
 *   d_out         [T,H] bf16 in
 *   dx            [T,H] bf16 out
 *   dw_router     [E,H] bf16 out
 *   d_bias        [E] fp32 out, or NULL (not computed)
 *   dw_gate, dw_up [E,I,H] and dw_down [E,H,I] bf16 out (experts that no token
 *                 selected get zeros)
 *   ws, ws_bytes  workspace of moe_workspace_bytes(desc, MOE_OP_BACKWARD)
 * Products accumulate in fp32 (bf16 MFMA); g, u and W_down^T d_out stay
 * fp32, the gated-activation gradients and the scaled activations (inputs of
 * the next GEMMs) are rounded to bf16.
 * No atomics: results are bitwise reproducible.  T = 0 writes zero parameter
 * gradients (no workspace needed).  MOE_EUNSUPPORTED for fp32,
 * FP8 or FP4 experts, packed weights, or H, I not multiples of 128. */
moe_status moe_backward(const moe_desc* desc, const void* x, const void* w_router,
                        const float* router_bias, const void* w_gate, const void* w_up,
                        const void* w_down, const void* d_out, void* dx, void* dw_router,
                        float* d_bias, void* dw_gate, void* dw_up, void* dw_down,
                        void* ws, size_t ws_bytes, void* stream);

/* Bytes of the packed copy of one weight set (MOE_PACK_GATE_UP: w_gate and
 * w_up together; MOE_PACK_DOWN: w_down) for desc's shapes and weight dtype;
 * 0 if the description is invalid or uses fp32 weights. */
size_t moe_packed_weight_bytes(const moe_desc* desc, int which);

/* Writes the packed layout of one weight set into dst (device, at least
 * moe_packed_weight_bytes(desc, which) bytes, 256-byte aligned).
 *   which = MOE_PACK_GATE_UP: w0 = w_gate, w1 = w_up (row-major [E,I,H])
 *   which = MOE_PACK_DOWN:    w0 = w_down (row-major [E,H,I]), w1 = NULL
 * Packed tile t of gate/up holds channels 128t .. 128t+127 (gate rows first,
 * then the same channels of up); packed tile t of down holds output channels
 * 256t .. 256t+255; rows past the end are zero.  desc->T and desc->w_layout
 * are ignored.  bf16 and fp8 weights only. */
moe_status moe_pack_weights(const moe_desc* desc, int which, const void* w0, const void* w1,
                            void* dst, void* stream);

/* Workspace bytes needed by `op` (a moe_op) for this description; 0 if the
 * op needs none or the description is invalid (the call itself then reports
 * why). */
size_t moe_workspace_bytes(const moe_desc* desc, int op);

/* Static text for a moe_status value. */
const char* moe_status_str(int status);

/* Text of the last failure in the calling thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------------------ */
/* Stage timing, for measurement.  While enabled, moe_forward and moe_backward
 * bracket each of their kernels with HIP events on the caller's stream.  moe_timing_read waits
 * for the recorded events, adds their elapsed times into ms[stage] and the
 * number of timed launches into launches[stage] (both host arrays of
 * MOE_NUM_STAGES entries), and clears the record.  Not thread-safe.
 * When all T*k pairs fit one 1024-pair chunk, histogram, scan and scatter run
 * as one launch, timed under MOE_STAGE_SCAN; up to 32 chunks the histogram
 * runs inside the scan launch (MOE_STAGE_SCAN), and MOE_STAGE_HIST times a
 * histogram launch only past that.  A stage's time covers all of its
 * launches (the weight-streaming gate/up and down add a split-K reduction
 * launch each). */
enum {
    MOE_STAGE_ROUTE = 0, MOE_STAGE_HIST = 1, MOE_STAGE_SCAN = 2, MOE_STAGE_SCATTER = 3,
    MOE_STAGE_QUANT_X = 4, MOE_STAGE_GATE_UP = 5, MOE_STAGE_DOWN = 6, MOE_STAGE_COMBINE = 7,
    /* moe_backward: recompute of g and u; the two data-gradient GEMMs; the
     * weight-gradient GEMMs; the router's gradients; gathers, the
     * gated-activation gradient and the dx sum */
    MOE_STAGE_BWD_RECOMPUTE = 8, MOE_STAGE_BWD_DATA = 9, MOE_STAGE_BWD_WEIGHT = 10,
    MOE_STAGE_BWD_ROUTER = 11, MOE_STAGE_BWD_MISC = 12,
    MOE_NUM_STAGES = 13
};
moe_status moe_timing_enable(int on);
moe_status moe_timing_read(double* ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
