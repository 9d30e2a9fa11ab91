/*
 * eagle.h -- C ABI of the EAGLE-3 draft-and-verify hot path for MI355X (gfx950).
 *
 * The library computes, on one GPU, the four parts of one speculation round:
 *   (1) multi-layer feature fusion, g = W_R [l; m; h]
 *       ("EAGLE-3 ... Training-Time Test" summary page, 3.4 "Feature
 *        Extraction: What Changes from EAGLE to EAGLE-3", Change 2;
 *        "M7.5 - EAGLE Feature Drafting ..." page, 0x08B);
 *   (2) draft steps of a single-layer drafter joined with the token embedding,
 *       u = W_I [g | a; e(x)], followed by the reused LM head with a fused top-k
 *       (EAGLE-3 summary page, "The Draft Model Architecture in Detail" and
 *        "The Inference Pipeline: Drafting and Verification");
 *   (3) EAGLE-2 dynamic tree growth: cumulative log-confidence values, per
 *       layer expansion of the best K nodes, final top-N rerank, flatten with
 *       positions and ancestry mask (M7.5 page, 0x06A-0x06B, 0x05B-0x05C);
 *   (4) tree verification against per-node target logits: greedy match or
 *       multi-round rejection sampling with residual resampling, plus the
 *       commit of the accepted path into the draft KV cache
 *       ("EAGLE: Speculative Sampling Requires Rethinking Feature Uncertainty"
 *        summary page, "Verification Phase: Multi-Round Speculative Sampling
 *        on Trees", Algorithm 1; M7.5 page, 0x05D).
 *
 * Conventions (every entry point):
 *  - All tensor arguments are DEVICE pointers owned by the caller, row-major,
 *    contiguous, and must stay valid until the work enqueued on `stream` ends.
 *    The library never allocates or frees device memory; its scratch space is
 *    the caller's workspace given to eagle_create.
 *  - Weights, target feature taps (low/mid/high) and the draft KV cache are
 *    in the config's dtype (bf16 stored as its 16-bit pattern, or fp32).
 *    Activations that cross the boundary -- the fused feature g, seed rows,
 *    draft states a -- are fp32, as are target logits and uniforms; indices
 *    are int32.  Inside, every activation stays fp32 and a bf16 GEMM takes
 *    it as a hi + lo bf16 pair, so results track an fp32-activation
 *    reference to ~1e-5 relative.
 *  - Work is asynchronous on `stream`; nothing synchronises except
 *    eagle_get_device_status.  A context is not re-entrant: calls on one
 *    context must be ordered (one stream, or explicit stream ordering).
 *  - Host-side argument errors return an error code and enqueue nothing.
 *    Errors found on the device (KV capacity, non-finite target logits) are
 *    recorded in the context's device status word and the affected sequence
 *    reports accept_len = -1.
 */
#ifndef EAGLE_H_
#define EAGLE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  EAGLE_OK = 0,
  EAGLE_EINVAL = 1,        /* null pointer, bad size or value               */
  EAGLE_EUNSUPPORTED = 2,  /* shape outside the supported envelope          */
  EAGLE_EHIP = 3,          /* a HIP launch or copy failed                   */
  EAGLE_ECAPACITY = 4,     /* device: KV cache too small for the rows       */
  EAGLE_ENONFINITE = 5,    /* device: NaN/Inf in target logits              */
  EAGLE_EWORKSPACE = 6     /* workspace smaller than eagle_workspace_bytes  */
} eagle_status;

typedef enum { EAGLE_BF16 = 0, EAGLE_FP32 = 1 } eagle_dtype;

/* Drafter shape and tree policy.
 * Supported envelope: head_dim in {64, 128}; n_q_heads % n_kv_heads == 0;
 * hidden, ffn, vocab multiples of 16 (ffn and head_dim/2 multiples of 8);
 * 1 <= topk <= 16; (depth - 1) * topk <= 64 (one 64-bit scratch mask);
 * budget + 1 <= 128; vocab >= topk; max_seed in [1, 4];
 * fp32 requires max_batch * max(max_seed, topk) <= 64.                     */
typedef struct {
  int32_t hidden;      /* H: draft width = target hidden width               */
  int32_t n_q_heads;   /* query heads                                        */
  int32_t n_kv_heads;  /* key/value heads (GQA)                              */
  int32_t head_dim;    /* hd                                                 */
  int32_t ffn;         /* F: SwiGLU width                                    */
  int32_t vocab;       /* V                                                  */
  int32_t dtype;       /* eagle_dtype                                        */
  float rope_theta;    /* RoPE base                                          */
  float rms_eps;       /* RMSNorm epsilon                                    */
  int32_t depth;       /* D: draft passes per tree (>= 0)                    */
  int32_t topk;        /* K: children per expanded node = expansion width    */
  int32_t budget;      /* N: tree nodes kept for verification (>= 0)         */
  int32_t max_batch;   /* largest batch any call will use                    */
  int32_t max_seed;    /* largest number of seed rows per sequence           */
} eagle_config;

/* Weights, device pointers in the config dtype, layout [out, in] row-major:
 *  w_fuse [H, 3H]  fusion FC over [low; mid; high]       (no bias)
 *  w_in   [H, 2H]  input FC over [g or a; embedding]     (no bias)
 *  embed  [V, H]   token embedding
 *  wq [nq*hd, H], wk [nkv*hd, H], wv [nkv*hd, H], wo [H, nq*hd]
 *  w_gate [F, H], w_up [F, H], w_down [H, F]
 *  w_lm   [V, H]   LM head (no bias)
 *  g_attn, g_mlp, g_final [H]  RMSNorm gains (attention, MLP, before head) */
typedef struct {
  const void *w_fuse, *w_in, *embed, *wq, *wk, *wv, *wo;
  const void *w_gate, *w_up, *w_down, *w_lm;
  const void *g_attn, *g_mlp, *g_final;
} eagle_weights;

/* Draft KV cache: k, v [B, n_kv, cap, hd] in the config dtype.  Rows
 * [0, len) are committed; a draft call appends its seed rows there and uses
 * rows [len_out, len_out + (D-1)K) as tree scratch.  len_in is read, len_out
 * written, so a call can be replayed with the same inputs. */
typedef struct {
  void *k;
  void *v;
  int32_t cap;
  const int32_t *len_in;  /* [B] device; may be NULL where unused           */
  int32_t *len_out;       /* [B] device                                     */
} eagle_kv;

/* Flattened tree, one per sequence, N+1 rows (row 0 = root).  Rows 1..n are
 * the selected nodes in (depth, parent row, token id) order; rows > n hold -1
 * (0 for score, n_child and mask).  mask is [B, N+1, W], W = ceil((N+1)/64):
 * bit j of row r is set iff row j is row r or one of its ancestors.
 * kv_slot is the node's draft-KV scratch slot (cache row len_out + slot), or
 * -1 if the node was never expanded (and for the root). */
typedef struct {
  int32_t *token, *parent, *depth, *position, *kv_slot, *first_child,
      *n_child;          /* [B, N+1] */
  float *score;          /* [B, N+1] cumulative float32 log confidence       */
  uint64_t *mask;        /* [B, N+1, W]                                      */
  int32_t *n_nodes;      /* [B] */
} eagle_tree;

typedef struct eagle_ctx eagle_ctx;

/* Bytes of device workspace eagle_create needs for this config. 0 if the
 * config is invalid. */
size_t eagle_workspace_bytes(const eagle_config *cfg);

/* Validates cfg, records the weight pointers (not copied; they must outlive
 * the context) and takes `workspace` (device, >= eagle_workspace_bytes,
 * 256-byte aligned) for the context's lifetime.  Clears the workspace's
 * counters with a kernel on `stream`.  *out receives a host-allocated
 * context. Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP. */
eagle_status eagle_create(const eagle_config *cfg, const eagle_weights *w,
                          void *workspace, size_t ws_bytes, hipStream_t stream,
                          eagle_ctx **out);

void eagle_destroy(eagle_ctx *ctx);

const char *eagle_status_str(eagle_status s);

/* Synchronises `stream`, copies the device status word (bit i set for error
 * code i, 0 = all good) to *host_status and clears it. */
eagle_status eagle_get_device_status(eagle_ctx *ctx, int32_t *host_status,
                                     hipStream_t stream);

/* (1) Fusion: g[r] = W_R [low[r]; mid[r]; high[r]], r < rows.
 * low, mid, high: [rows, H] config dtype; g_out: [rows, H] fp32.
 * rows in [0, 65536]. */
eagle_status eagle_fuse_features(eagle_ctx *ctx, int32_t rows,
                                 const void *low, const void *mid,
                                 const void *high, void *g_out,
                                 hipStream_t stream);

/* (2) One draft step over rows = batch * rows_per_seq query rows; row
 * b * rows_per_seq + i belongs to sequence b.  Per row (all device, [rows]):
 *   src [rows, H]   fp32 state joined with the token: g (seed) or parent's a
 *   token           token id whose embedding joins the row; < 0 = padding
 *   position        RoPE position
 *   dest            cache row receiving the row's K/V (< cap)
 *   prefix_len      row sees cache rows [0, prefix_len)
 *   scratch_base    [batch] first scratch cache row of the sequence
 *   scratch_mask    row also sees scratch_base + j for every set bit j
 * Outputs: a_out [rows, H] fp32 (decoder output state), topk_id / topk_logit
 * [rows, K] ordered by (-logit, id), lse [rows] (log-sum-exp of the row's
 * fp32 logits).  The row's own K/V must be visible to it through prefix_len
 * or scratch_mask.  rows_per_seq in [1, 16]. */
eagle_status eagle_draft_step(eagle_ctx *ctx, int32_t batch,
                              int32_t rows_per_seq, const void *src,
                              const int32_t *token, const int32_t *position,
                              const int32_t *dest, const int32_t *prefix_len,
                              const int32_t *scratch_base,
                              const uint64_t *scratch_mask, const eagle_kv *kv,
                              void *a_out, int32_t *topk_id, float *topk_logit,
                              float *lse, hipStream_t stream);

/* (2)+(3) Draft one EAGLE-2 tree per sequence.
 *   seed_src   [B, max_seed, H]  fp32 fused target features of the seed rows
 *   seed_token [B, max_seed]     tokens joined with them
 *   seed_len   [B]               rows used, 1..max_seed; the last is the root
 * Seed rows go to cache rows len_in[b] + i and attend causally; len_out[b] =
 * len_in[b] + seed_len[b]; the root sits at position len_out[b] - 1.  Then D
 * passes grow the tree as described at the top of this file; tree rows use
 * scratch cache rows [len_out, len_out + (D-1)K).  Needs
 * len_out + (D-1)K <= cap (device-checked: ECAPACITY).
 * D == 0 or N == 0 still commits the seed rows and returns a root-only tree.
 * batch in [1, max_batch]. */
eagle_status eagle_draft_tree(eagle_ctx *ctx, int32_t batch,
                              const void *seed_src, const int32_t *seed_token,
                              const int32_t *seed_len, const eagle_kv *kv,
                              const eagle_tree *out, hipStream_t stream);

/* (4) Verify each sequence's tree.
 *   target_logits [B, N+1, V] fp32: row r = target next-token logits after
 *                 tree row r.
 *   temperature   0 = greedy (argmax, lowest id on ties); > 0 = rejection
 *                 sampling of Algorithm 1 with the deterministic children as
 *                 point-mass proposals, tested in ascending token id, then an
 *                 inverse-CDF residual draw over ascending token id.
 *   uniforms      [B, N+1, K+1] fp32 in [0,1): column i < K is the draw for
 *                 the i-th child of that row, column K the residual draw.
 *                 May be NULL when temperature == 0.
 *   kv_or_null    if given: accepted rows are compacted from scratch into
 *                 cache row = position (rows that exist in scratch) and
 *                 kv->len_out[b] receives the new committed length.
 * Outputs: accept_len [B] (0..D, -1 on a device error), accepted_rows [B, D]
 * (tree rows, -1 padded), out_tokens [B, D+1] (accepted tokens then the
 * emitted one, -1 padded), next_seed_rows / next_seed_tokens [B, 2] and
 * next_seed_len [B]: the seed rows of the next round as (tree row whose
 * target feature is fused, token joined with it). */
eagle_status eagle_verify_tree(eagle_ctx *ctx, int32_t batch,
                               const eagle_tree *tree,
                               const float *target_logits, float temperature,
                               const float *uniforms,
                               const eagle_kv *kv_or_null, int32_t *accept_len,
                               int32_t *accepted_rows, int32_t *out_tokens,
                               int32_t *next_seed_rows,
                               int32_t *next_seed_tokens,
                               int32_t *next_seed_len, hipStream_t stream);

/* Measurement hook.  While profiling is on, every kernel the context enqueues
 * is bracketed by a pair of HIP events on its stream (up to 4096 launches
 * between reads).  eagle_profile(ctx, 1) clears the record and starts;
 * eagle_profile(ctx, 0) stops.  eagle_profile_read synchronises on the last
 * event and returns, per kernel class, the summed event time (ms), launch
 * count, algorithmic bytes (weights once + activations in/out; the target
 * logits for verification) and algorithmic flops, then clears the record.
 * Classes: 0 draft-layer GEMMs, 1 fusion GEMM, 2 tree attention, 3 LM-head
 * top-k merge, 4 tree growth/rerank/flatten, 5 verification.  Returns
 * EWORKSPACE if launches were dropped because the record was full. */
eagle_status eagle_profile(eagle_ctx *ctx, int32_t on);
eagle_status eagle_profile_read(eagle_ctx *ctx, int32_t n_classes, float *ms,
                                int32_t *launches, double *bytes,
                                double *flops);

#ifdef __cplusplus
}
#endif

#endif /* EAGLE_H_ */
