/*
 * moe.h - C ABI of a gfx950 (MI355X) library computing the forward pass of
 * one sparse mixture-of-experts layer.
 *
 * The operation (sources cited per entry point below):
 *   Treebeard, "How Treebeard routes Qwen3.6 MoE tokens":
 *     "Routing math"              z = W_router^T x, p = softmax(z), I = TopK(p, K),
 *                                 alpha = p_I / max(sum p_I, 2^-14)
 *     "Routed expert computation" e_i = W_down_i^T (SiLU(W_gate_i^T x) * W_up_i^T x),
 *                                 y_routed = sum_i alpha_i e_i
 *     "Shared expert computation" y_shared = sigmoid(w_shared^T x) * shared SwiGLU(x),
 *                                 r_next = r + (y_routed + y_shared)
 *     "Treebeard's execution optimization" / "Intel SYCL path": routing artefacts
 *                                 are final before expert execution; pairs are
 *                                 counted per expert, offset, listed and packed,
 *                                 and results written back to their token and slot.
 *   edge0, "MoE Routing and Experts":
 *     "Routing families"          softmax top-k, and sigmoid group top-k with
 *                                 expert_bias, n_group, topk_group, routed_scaling
 *     tier table                  "4-bit affine, group 64" weights.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller; matrices are
 *     row-major with the input (reduction) dimension contiguous.  The library
 *     never allocates device memory, never synchronises the host, never prints
 *     and never aborts; it returns a moe_status.
 *   - All argument checks run on the host before any launch.  A failed check
 *     returns an error code and launches nothing.  n_tokens == 0 returns MOE_OK
 *     with no launch.  After launching, a launch failure reported by the HIP
 *     runtime returns MOE_ERR_HIP; moe_last_error() gives a message.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *   - Scratch memory is the caller's `ws` of `ws_bytes` bytes (size it with
 *     moe_workspace_size).  Calls that share a workspace must be ordered on
 *     one stream.  The workspace needs no initialisation.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs run to run (fixed reduction orders, no floating-point atomics).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* identical to hipStream_t */

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,  /* null pointer, bad size or family parameter */
    MOE_ERR_UNSUPPORTED = 2,       /* shape or dtype mix this library does not build */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4                /* the HIP runtime reported a failure */
} moe_status;

typedef enum {
    MOE_F32 = 0,            /* float32 */
    MOE_BF16 = 1,           /* bfloat16 */
    MOE_U4_AFFINE_G64 = 2   /* 4-bit codes (two per byte, even element in the low
                               nibble) + bf16 scale and bf16 min per 64 consecutive
                               input elements: w = scale * q + min */
} moe_dtype;

typedef enum {
    MOE_ROUTE_SOFTMAX_TOPK = 0,      /* edge0 "Softmax top-k"; Treebeard "Routing math" */
    MOE_ROUTE_SIGMOID_GROUP_TOPK = 1 /* edge0 "Sigmoid group top-k" */
} moe_route_family;

/* Layer description.  Field names follow the GGUF keys quoted on the
 * Treebeard page ("Source map"): d_model = embedding_length, n_experts =
 * expert_count, top_k = expert_used_count, d_ff = expert_feed_forward_length,
 * d_ff_shared = expert_shared_feed_forward_length. */
typedef struct {
    int32_t n_tokens;       /* T >= 0 */
    int32_t d_model;        /* D */
    int32_t n_experts;      /* E, multiple of 16, <= 1024 */
    int32_t top_k;          /* K, 1 <= K <= min(E, 32) */
    int32_t d_ff;           /* F, routed expert intermediate width */
    int32_t d_ff_shared;    /* F_s, shared expert width; 0 = no shared expert */
    moe_route_family family;
    int32_t n_group;        /* sigmoid family: groups of E/n_group contiguous experts */
    int32_t topk_group;     /* sigmoid family: groups kept per token */
    float routed_scaling;   /* sigmoid family: factor on the renormalised weights */
    moe_dtype act_dtype;    /* x: MOE_F32 or MOE_BF16 */
    moe_dtype router_dtype; /* router and shared gate vector: same as act_dtype */
    moe_dtype expert_dtype; /* routed and shared banks: MOE_F32 (with F32 activations),
                               MOE_BF16 or MOE_U4_AFFINE_G64 (with BF16 activations;
                               d_model, d_ff, d_ff_shared <= 4096) */
} moe_config;

/* One weight matrix or bank.  For MOE_F32/MOE_BF16 only `w` is used
 * ([rows, in] per expert).  For MOE_U4_AFFINE_G64: w = codes uint8
 * [rows, in/2], scale and min = bf16 [rows, in/64]. */
typedef struct {
    const void* w;
    const void* scale;
    const void* min;
} moe_matrix;

typedef struct {
    const void* router;          /* [E, D] router_dtype (z = x W^T) */
    const float* expert_bias;    /* [E] fp32, sigmoid family selection bias; NULL = zeros */
    moe_matrix gate;             /* [E, F, D] */
    moe_matrix up;               /* [E, F, D] */
    moe_matrix down;             /* [E, D, F] */
    moe_matrix shared_gate;      /* [F_s, D] (ignored when d_ff_shared == 0) */
    moe_matrix shared_up;        /* [F_s, D] */
    moe_matrix shared_down;      /* [D, F_s] */
    const void* shared_gate_vec; /* [D] router_dtype; NULL => shared gate s_t = 1 */
} moe_weights;

/* Bytes of workspace every entry point below needs for `cfg` (the largest
 * need of any of them; 256-byte aligned regions).  Returns MOE_OK or
 * MOE_ERR_INVALID_ARGUMENT / MOE_ERR_UNSUPPORTED for a config no entry
 * point accepts. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* Routing (Treebeard "Routing math"; edge0 "Routing families").
 * x [T, D] act_dtype; router [E, D] router_dtype; expert_bias [E] fp32 or NULL.
 * Outputs topk_ids [T, K] int32 (slots in descending selection score, ties
 * to the lower expert index) and topk_weights [T, K] fp32 (softmax family:
 * renormalised probabilities with the 2^-14 floor; sigmoid family:
 * routed_scaling * raw sigmoid scores renormalised with the same floor,
 * bias excluded).  Logits are computed in fp32 from exact products. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* router,
                     const float* expert_bias, int32_t* topk_ids, float* topk_weights,
                     void* ws, size_t ws_bytes, moe_stream_t stream);

/* Permute (Treebeard "Intel SYCL path", steps 1-3): counts the T*K
 * (token, slot) pairs per expert and writes
 *   expert_offsets [E+1] int32   exclusive prefix sum of the counts,
 *   active_experts [E] int32     experts with count > 0, ascending (first n_active used),
 *   n_active       [1] int32,
 *   sorted_pairs   [T*K] int32   flat pair ids t*K + k grouped by expert,
 *                                ascending inside each expert (stable).
 * Ids outside [0, E) are not counted and get no row.  ws may be NULL; with a
 * workspace of moe_workspace_size bytes, 4096 or more pairs are permuted in
 * parallel chunks (count, scan, scatter) instead of by one workgroup. */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* active_experts, int32_t* n_active,
                       int32_t* sorted_pairs, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Routed experts (Treebeard "Routed expert computation"; edge0 "Experts"):
 * for every pair p = t*K + k of expert e = topk_ids[t, k],
 *   slot_out[p, :] = topk_weights[p] * W_down[e]^T (SiLU(W_gate[e]^T x_t) * W_up[e]^T x_t)
 * slot_out [T, K, D] fp32.  Inputs are the permute outputs above (only the
 * first n_active entries of active_experts are read) and the flat weights
 * [T*K] fp32.  Only active experts' weights are read, each once per tile of
 * up to 16 of its pairs (small T), 128 (bf16 weights, experts averaging >= 16
 * pairs; 4-bit weights averaging >= 64 pairs when d_model and d_ff are 256 ..
 * 2048, 64 from 16 pairs) or 64 (other 4-bit and fp32 weights, >= 64
 * pairs).  4-bit codes are
 * dequantised to bf16 (scale * q + min, rounded to nearest even) inside the
 * GEMM kernels.  The SwiGLU intermediate is rounded to bf16 for bf16/u4
 * weights and kept fp32 for fp32 weights. */
moe_status moe_experts(const moe_config* cfg, const void* x, const moe_weights* weights,
                       const int32_t* expert_offsets, const int32_t* active_experts,
                       const int32_t* n_active, const int32_t* sorted_pairs,
                       const float* topk_weights, float* slot_out,
                       void* ws, size_t ws_bytes, moe_stream_t stream);

/* Shared expert (Treebeard "Shared expert computation"):
 *   shared_out[t, :] = s_t * W_sd^T (SiLU(W_sg^T x_t) * W_su^T x_t),
 *   s_t = sigmoid(shared_gate_vec . x_t), or 1 when shared_gate_vec is NULL.
 * shared_out [T, D] fp32.  Requires d_ff_shared > 0. */
moe_status moe_shared_expert(const moe_config* cfg, const void* x, const moe_weights* weights,
                             float* shared_out, void* ws, size_t ws_bytes, moe_stream_t stream);

/* Combine (Treebeard "Shared expert computation", last block):
 *   out[t, :] = residual[t, :] + (sum_{k=0..K-1} slot_out[t, k, :] + shared_out[t, :])
 * with the slots summed in ascending k in fp32.  shared_out may be NULL
 * (treated as zeros); out may alias residual. */
moe_status moe_combine(const moe_config* cfg, const float* slot_out, const float* shared_out,
                       const float* residual, float* out, moe_stream_t stream);

/* The whole layer: route -> permute -> experts -> combine, with the shared
 * expert.  residual [T, D] fp32; out [T, D] fp32 (may alias residual).
 * topk_ids_out [T, K] and topk_weights_out [T, K] receive the routing when
 * non-NULL.  Internally the routed slot rows are staged in bf16 for bf16/u4
 * weights.  Schedules:
 *   T*K <= 256 (and experts averaging < 16 pairs for bf16 weights, < 64
 *     otherwise): a single stream (at most 32 pairs: the gate/up launch takes
 *     one work item per pair instead of one per expert); the
 *     shared expert is one more work item of the routed gate/up and down
 *     launches, its sigmoid gate logit is computed with the routing, and each
 *     GEMM workgroup finds its expert and pairs from the routing ids itself
 *     (no separate permute launch).  aux_stream is not used.
 *   otherwise: the shared expert runs on aux_stream when it is non-NULL
 *     (forked from and joined back into `stream` with library-owned events;
 *     otherwise on `stream`) while routing and the permute run. */
moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* weights, const void* x,
                             const float* residual, float* out, int32_t* topk_ids_out,
                             float* topk_weights_out, void* ws, size_t ws_bytes,
                             moe_stream_t stream, moe_stream_t aux_stream);

/* The layer with direct (per-pair) execution of the routed experts, for
 * small batches (Treebeard, "Intel SYCL path": below a few token columns the
 * fused kernel runs one (token, slot) pair at a time instead of bucketing
 * pairs by expert).  Same arguments, outputs and tolerances as
 * moe_layer_forward (no aux stream: one stream); the routed gate/up and down
 * projections take one work item per (token, slot) pair, each reading its
 * expert's weights, where moe_layer_forward groups the pairs of an expert so
 * its weights are read once; the combine is a separate launch.  Only for
 * layers moe_layer_forward runs on its single-stream small-T schedule
 * (T*K <= 256 and fewer than 16 pairs per expert on average for bf16 banks,
 * 64 otherwise); MOE_ERR_UNSUPPORTED beyond.  The routing and the SwiGLU
 * intermediate equal moe_layer_forward's bit for bit (same selection, same
 * tile shape and sum order per pair); the routed down projection is the
 * unfused one, so the output matches moe_layer_forward's within the layer
 * tolerance (bit for bit with fp32 weights). */
moe_status moe_layer_forward_direct(const moe_config* cfg, const moe_weights* weights, const void* x,
                                    const float* residual, float* out, int32_t* topk_ids_out,
                                    float* topk_weights_out, void* ws, size_t ws_bytes, moe_stream_t stream);

/* RMS normalisation of the attention residual (Treebeard "Routing math": x_t
 * is the post-attention, RMS-normalised hidden state; "Editable Mermaid
 * flowchart" and "Pseudocode": x = rms_norm(attention residual) before the
 * router).  The pages fix neither an epsilon nor a weight; this library computes
 *   x[t, j] = residual[t, j] / sqrt(mean_j residual[t, j]^2 + eps) * norm_weight[j]
 * residual [T, D] fp32; norm_weight [D] fp32, or NULL for ones; x [T, D]
 * act_dtype, written once (bf16: rounded to nearest even from the fp32
 * value).  The row's sum of squares is accumulated in fp32 in a fixed order.
 * eps must be finite and > 0.  residual, norm_weight and x must be 16-byte
 * aligned and x must not overlap residual.  Reads n_tokens, d_model and
 * act_dtype of cfg. */
moe_status moe_rms_norm(const moe_config* cfg, const float* residual, const float* norm_weight, float eps,
                        void* x, moe_stream_t stream);

/* The layer from the attention residual: x = moe_rms_norm(residual), then
 * moe_layer_forward(x, residual) (Treebeard "Pseudocode": the layer function
 * starts from the attention residual and returns residual + routed + shared).
 * x_out [T, D] act_dtype receives x when non-NULL (it must not overlap
 * residual or out); otherwise x is kept in ws.  Outputs, aliasing of out and
 * residual, and schedules are those of moe_layer_forward; the normalisation
 * runs first, on `stream`. */
moe_status moe_layer_forward_norm(const moe_config* cfg, const moe_weights* weights, const float* norm_weight,
                                  float eps, const float* residual, void* x_out, float* out,
                                  int32_t* topk_ids_out, float* topk_weights_out, void* ws, size_t ws_bytes,
                                  moe_stream_t stream, moe_stream_t aux_stream);

/* moe_layer_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, outputs and results as moe_layer_forward,
 * without the workspace and the aux stream: everything runs on `stream`.
 * Scratch memory is a 32 MiB array inside the library, one per device (held
 * until the process ends); a layer whose moe_workspace_size exceeds 32 MiB
 * (at Qwen3.6 shape: bf16 weights beyond T = 256) returns
 * MOE_ERR_WORKSPACE_TOO_SMALL and launches nothing.  The call allocates
 * nothing: no hipMalloc, hipFree, event or stream creation.  Every call on a
 * device shares that device's array, so calls that overlap on one device
 * (different streams, or different host threads) race: order them on one
 * stream. */
moe_status moe_layer_forward_noalloc(const moe_config* cfg, const moe_weights* weights, const void* x,
                                     const float* residual, float* out, int32_t* topk_ids_out,
                                     float* topk_weights_out, moe_stream_t stream);

/* Stages of moe_layer_forward that moe_layer_stage can re-launch. */
typedef enum {
    MOE_STAGE_ROUTER_LOGITS = 0, /* router GEMM: x [T,D] -> fp32 logits in ws */
    MOE_STAGE_GATE_UP = 1,       /* routed gate/up GEMM + SwiGLU -> h in ws, the launch the
                                    layer runs (where the layer folds the selection into it,
                                    so does the stage: it selects again from the router logits
                                    in ws; at most 32 pairs it is the per-pair launch) */
    MOE_STAGE_DOWN = 2,          /* routed down GEMM x alpha -> staged slot rows in ws (small T
                                    with bf16/4-bit weights: the down projection fused with the
                                    combine, writing a [T, D] scratch in ws) */
    MOE_STAGE_GATE_UP_DIRECT = 3, /* small T*K only (<= 256 pairs, fewer than 64 per expert):
                                    the gate/up stage with every (token, slot) pair as its
                                    own work item, no grouping by expert (Treebeard, "Intel
                                    SYCL path": direct versus bucketed execution); writes
                                    the same h as MOE_STAGE_GATE_UP (and selects inside the
                                    launch when that stage does).  MOE_ERR_UNSUPPORTED
                                    otherwise. */
    MOE_STAGE_DOWN_GROUPED = 4,  /* small T*K only: the down projection x alpha into slot rows
                                    in ws, one work item per active expert (the unfused
                                    grouped form; with fp32 weights the one the layer runs) */
    MOE_STAGE_DOWN_DIRECT = 5    /* small T*K only: the same with one work item per (token,
                                    slot) pair (moe_layer_forward_direct's down projection) */
} moe_stage;

/* Measurement aid: re-launches one kernel stage of the last
 * moe_layer_forward that ran with this cfg, weights, x and ws, reading the
 * stage's inputs from the workspace (routing, permutation or tile list, h)
 * and rewriting the same workspace outputs, so the stage can be timed alone
 * on the real routing of that call.  It has no effect on the caller's
 * out/residual or routing outputs. */
moe_status moe_layer_stage(const moe_config* cfg, const moe_weights* weights, const void* x, moe_stage stage,
                           void* ws, size_t ws_bytes, moe_stream_t stream);

/* Measurement aid, not part of the layer: one streaming read of `bytes`
 * bytes of device memory at `buf`, the reference rate for the layer's
 * HBM-bound kernels (a buffer larger than the 256 MB last-level cache is
 * read from HBM; a smaller one read again comes from that cache).  Each
 * 64 KB block is read by one wave in 16-byte loads whose requests cover
 * whole 128-byte lines; the XOR of the 16-byte words lane l of block b read
 * (the four 32-bit halves folded into one word) is written to
 * sink[64 b + l], so the reads cannot be elided.
 * buf: device pointer, 16-byte aligned; bytes: a non-zero multiple of
 * 262144; sink: device pointer to sink_words >= bytes / 1024 uint32 words.
 * MOE_ERR_INVALID_ARGUMENT (nothing launched) otherwise. */
moe_status moe_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, moe_stream_t stream);

/* Measurement aid, not part of the layer: the bf16 MFMA issue rate of this
 * chip, the reference for the MFMA-bound side of the grouped GEMMs.  Launches
 * `workgroups` workgroups of 4 waves (256 of them put one wave on each SIMD
 * of the 256 compute units, 512 two); every wave runs 8 independent
 * accumulator chains of `iterations` back-to-back MFMAs of one shape
 * (shape 0: v_mfma_f32_16x16x32_bf16, 2*16*16*32 flops; 1:
 * v_mfma_f32_32x32x16_bf16, 2*32*32*16 flops) on operands equal to 1.0, and
 * each lane writes the sum of its accumulators to sink[256 w + t] (w the
 * workgroup, t the thread): iterations * 8 * 4 * 32 for shape 0 and
 * iterations * 8 * 16 * 16 for shape 1.  The caller times the launch.
 * Every partial sum is a multiple of 16 below 2^27, so the stated value is
 * exact in fp32 for every allowed count.
 * shape: 0 or 1; workgroups: 1 .. 65536; iterations: 1 .. 65536; sink: device
 * pointer to sink_words >= 256 * workgroups floats.
 * MOE_ERR_INVALID_ARGUMENT (nothing launched) otherwise. */
moe_status moe_mfma_rate(int32_t shape, int32_t workgroups, int32_t iterations, float* sink, size_t sink_words,
                         moe_stream_t stream);

/* Measurement aid, not part of the layer: the vector-memory read rate from
 * the L2 for three ways of mapping lanes to addresses, the reference for the
 * load layouts of the register-streaming GEMMs.  Launches `workgroups`
 * workgroups of 4 waves; every wave reads a 64 KB region laid out as 16 rows
 * of 4096 bytes, `iterations` passes of 64 load instructions (16 bytes per
 * lane each, issued in groups of eight):
 *   pattern 0: instruction c reads bytes 1024 c .. 1024 c + 1023 of the
 *     region, lane l the 16 at 1024 c + 16 l;
 *   pattern 1: instruction c reads bytes 64 c .. 64 c + 63 of every row,
 *     lane l row l % 16 at 64 c + 16 (l / 16) (the lane order of a 16x16x32
 *     MFMA operand fragment);
 *   pattern 2: the same bytes as pattern 1, lane l row l / 4 at
 *     64 c + 16 (l % 4).
 * Workgroup w's wave v reads region 4 ((w / 256) % 4) + v of buf (1 MiB: 16
 * regions), starting each pass at chunk (8 w) % 64.  Each lane adds the
 * 32-bit words it read, modulo 2^32, into sink[256 w + 64 v + l]:
 * `iterations` times the sum of the words of its 64 chunks.  The caller
 * times the launch; 1 MiB fits every XCD's L2 (4 MB), so after the first
 * pass the loads are served from there.
 * pattern: 0, 1 or 2; workgroups: 1 .. 65536; iterations: 1 .. 65536; buf:
 * device pointer, 16-byte aligned, buf_bytes >= 1048576; sink: device
 * pointer to sink_words >= 256 * workgroups uint32 words.
 * MOE_ERR_INVALID_ARGUMENT (nothing launched) otherwise. */
moe_status moe_l2_read_rate(int32_t pattern, int32_t workgroups, int32_t iterations, const void* buf,
                            size_t buf_bytes, uint32_t* sink, size_t sink_words, moe_stream_t stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status status);

/* Message describing the last failure on the calling host thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
