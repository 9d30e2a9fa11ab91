/*
 * eagle.h -- C ABI of the EAGLE-3 draft-and-verify hot path for MI355X (gfx950).
 *
 * One speculation round, on one GPU: (1) multi-layer feature fusion,
 * (2) draft steps of a single-layer drafter with a fused LM-head top-k,
 * (3) EAGLE-2 dynamic tree growth and rerank, (4) tree verification against
 * per-node target logits, with the commit of the accepted path.  Each entry
 * point below names the passage of the pages that defines its operation.
 * Pages are cited by title and section:
 *   [E3]  "EAGLE-3: Scaling up Inference Acceleration of Large Language Models
 *         via Training-Time Test" (paper summary page)
 *   [E1]  "EAGLE: Speculative Sampling Requires Rethinking Feature
 *         Uncertainty" (paper summary page)
 *   [M75] "M7.5 - EAGLE Feature Drafting: Uncertainty, Dynamic Trees, HASS,
 *         and EAGLE-3"
 *
 * Conventions (every entry point):
 *  - Tensor arguments are DEVICE pointers owned by the caller, row-major and
 *    contiguous; they must stay valid until the work enqueued on `stream`
 *    ends.  The library never allocates or frees device memory: its scratch
 *    space is the workspace the caller hands to eagle_create.
 *  - Weights, target feature taps (low/mid/high) and the draft KV cache are
 *    in the config's dtype (bf16 as its 16-bit pattern, or fp32).
 *    Activations that cross the boundary -- the fused feature g, seed rows,
 *    draft states a -- are fp32, as are target logits; ids are int32.
 *    Inside, every activation stays fp32; a bf16 GEMM takes it as a hi + lo
 *    bf16 pair, so results track an fp32-activation reference to ~1e-5.
 *  - Work is asynchronous on `stream`; nothing synchronises except
 *    eagle_create (with a reduced vocabulary) and eagle_get_device_status.
 *    A context is not re-entrant: calls on one context must be ordered.
 *  - Host-side argument errors return an error code and enqueue nothing.
 *    Errors found on the device (KV capacity, non-finite target logits, a
 *    malformed tree) are recorded in the context's device status word and
 *    the affected sequence reports accept_len = -1 / n_nodes = -1.
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
  EAGLE_ENONFINITE = 5,    /* device: NaN/Inf in target logits, bad tree    */
  EAGLE_EWORKSPACE = 6     /* workspace smaller than eagle_workspace_bytes  */
} eagle_status;

typedef enum { EAGLE_BF16 = 0, EAGLE_FP32 = 1 } eagle_dtype;

/* What the verification commits for the next round ([M75] 0x05D: commit the
 * accepted state, discard unaccepted tree rows, reseed).
 *  KEEP:   accepted draft-KV rows that were computed move to their position;
 *          the next seed supplies only the 1-2 rows still missing.
 *  RESEED: no draft row is kept; every verified row's target feature is
 *          fused again and seeds the next round ([E3] 3.4 "The Inference
 *          Pipeline", Stage 2), a + 1 seed rows. */
typedef enum { EAGLE_COMMIT_KEEP = 0, EAGLE_COMMIT_RESEED = 1 } eagle_commit_mode;

/* Random streams of eagle_draw_uniforms (second key word of Philox). */
typedef enum { EAGLE_STREAM_VERIFY = 0, EAGLE_STREAM_DRAFT = 1 } eagle_stream_id;

/* Drafter shape and tree policy ([E3] "The Draft Model Architecture in
 * Detail": width H, one decoder layer, the target's LM head; [M75] 0x06D:
 * expansion width, depth and verification budget are separate knobs).
 * Supported envelope: head_dim in {64, 128}; n_q_heads % n_kv_heads == 0;
 * hidden, vocab multiples of 16; ffn multiple of 8; 1 <= topk <= 16;
 * (depth - 1) * topk <= 64 (one 64-bit scratch mask); budget + 1 <= 128;
 * vocab >= topk; 1 <= max_seed <= 16 and max(max_seed, topk) * (n_q/n_kv)
 * <= 128; fp32 requires max_batch * max(max_seed, topk) <= 64 and hd 64.  */
typedef struct {
  int32_t hidden;      /* H: draft width = target hidden width               */
  int32_t n_q_heads;   /* query heads                                        */
  int32_t n_kv_heads;  /* key/value heads (GQA)                              */
  int32_t head_dim;    /* hd                                                 */
  int32_t ffn;         /* F: SwiGLU width                                    */
  int32_t vocab;       /* V: rows of the LM head (the draft vocabulary)      */
  int32_t dtype;       /* eagle_dtype                                        */
  float rope_theta;    /* RoPE base                                          */
  float rms_eps;       /* RMSNorm epsilon                                    */
  int32_t depth;       /* D: draft passes per tree (>= 0)                    */
  int32_t topk;        /* K: children per expanded node = expansion width    */
  int32_t budget;      /* N: tree nodes kept for verification (>= 0)         */
  int32_t max_batch;   /* largest batch any call will use                    */
  int32_t max_seed;    /* seed rows per sequence (>= 2 to verify with KEEP,
                          >= depth + 1 with RESEED)                          */
  int32_t target_vocab;/* token-id space of the tree, the embedding and the
                          target logits; 0 = vocab.  > vocab needs d2t.      */
} eagle_config;

/* Weights, device pointers in the config dtype, layout [out, in] row-major:
 *  w_fuse [H, 3H]  fusion FC over [low; mid; high]       (no bias)
 *  w_in   [H, 2H]  input FC over [g or a; embedding]     (no bias)
 *  embed  [TV, H]  token embedding (TV = target_vocab or vocab)
 *  wq [nq*hd, H], wk [nkv*hd, H], wv [nkv*hd, H], wo [H, nq*hd]
 *  w_gate [F, H], w_up [F, H], w_down [H, F]
 *  w_lm   [V, H]   LM head (no bias)
 *  g_attn, g_mlp, g_final [H]  RMSNorm gains (attention, MLP, before head)
 *  d2t    [V] int32, strictly increasing draft id -> target id map of a
 *         reduced draft vocabulary ([M75] 0x08C), or NULL when the draft and
 *         target vocabularies are the same.                                  */
typedef struct {
  const void *w_fuse, *w_in, *embed, *wq, *wk, *wv, *wo;
  const void *w_gate, *w_up, *w_down, *w_lm;
  const void *g_attn, *g_mlp, *g_final;
  const int32_t *d2t;
} eagle_weights;

/* Draft KV cache ([M75] 0x03C: the drafter keeps its own K/V state,
 * separate from the target's), config dtype: k [B, n_kv, cap, hd] (row r of
 * a head is key r) and v [B, n_kv, hd, cap] (stored transposed: column r of
 * a head is value r), so that tree attention reads both as matrix-core
 * operands directly.  cap is a multiple of 8 and at least 32 (else EINVAL).
 * Rows [0, len) are committed; a draft call appends its seed rows there and
 * uses rows [len_out, len_out + (D-1)K) as tree scratch.  len_in is read, len_out
 * written, so a call can be replayed with the same inputs. */

typedef struct {
  void *k;
  void *v;
  int32_t cap;
  const int32_t *len_in;  /* [B] device; may be NULL where unused           */
  int32_t *len_out;       /* [B] device                                     */
} eagle_kv;

/* Flattened tree ([M75] 0x05C and 0x09: rows, positions, ancestry mask,
 * retrieve map), one per sequence, N+1 rows, row 0 = root.  Rows 1..n are
 * the selected nodes in (depth, parent row, token id) order; rows > n hold
 * -1 (0 for score, n_child and mask).  mask is [B, N+1, W],
 * W = ceil((N+1)/64): bit j of row r is set iff row j is row r or one of its
 * ancestors.  token holds target ids.  kv_slot is the node's draft-KV
 * scratch slot (cache row len_out + slot), or -1 if the node was never
 * expanded (and for the root).  score is the float32 cumulative
 * log-confidence ([M75] 0x06A). */
typedef struct {
  int32_t *token, *parent, *depth, *position, *kv_slot, *first_child,
      *n_child;          /* [B, N+1] */
  float *score;          /* [B, N+1] */
  uint64_t *mask;        /* [B, N+1, W]                                      */
  int32_t *n_nodes;      /* [B] */
} eagle_tree;

typedef struct eagle_ctx eagle_ctx;

/* Bytes of device workspace eagle_create needs for this config; 0 if the
 * config is invalid. */
size_t eagle_workspace_bytes(const eagle_config *cfg);

/* Validates cfg, takes `workspace` (device, >= eagle_workspace_bytes,
 * 256-byte aligned) for the context's lifetime and copies the seven GEMM
 * weight matrices (w_fuse, w_in, wq/wk/wv, wo, w_gate/w_up, w_down, w_lm)
 * into it in the tile order the kernels stream, with kernels on `stream`;
 * later writes to those buffers are not seen.  embed, the gains and d2t are
 * read in place and must outlive the context.  Clears the workspace's
 * counters; with a d2t map it synchronises `stream` and checks the map on
 * the host.  *out receives a host-allocated context.
 * Errors: EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP. */
eagle_status eagle_create(const eagle_config *cfg, const eagle_weights *w,
                          void *workspace, size_t ws_bytes, hipStream_t stream,
                          eagle_ctx **out);

void eagle_destroy(eagle_ctx *ctx);

const char *eagle_status_str(eagle_status s);

/* Synchronises `stream`, copies the device status word (bit i set for error
 * code i, 0 = all good) to *host_status and clears it. */
eagle_status eagle_get_device_status(eagle_ctx *ctx, int32_t *host_status,
                                     hipStream_t stream);

/* (1) Fusion ([E3] 3.4 "Feature Extraction: What Changes from EAGLE to
 * EAGLE-3", Change 2; [M75] 0x08B): g[r] = W_R [low[r]; mid[r]; high[r]],
 * the three target taps concatenated and projected 3H -> H, no bias.
 * low, mid, high: [rows, H] config dtype; g_out: [rows, H] fp32.
 * rows in [0, 65536]; 0 enqueues nothing. */
eagle_status eagle_fuse_features(eagle_ctx *ctx, int32_t rows,
                                 const void *low, const void *mid,
                                 const void *high, void *g_out,
                                 hipStream_t stream);

/* (2) One draft step ([E3] "The Draft Model Architecture in Detail": join
 * u = W_I [g | a; e(x)], one decoder layer, the reused LM head; [M75] 0x05B:
 * several nodes of one depth in one pass under tree attention) over
 * rows = batch * rows_per_seq query rows; row b * rows_per_seq + i belongs
 * to sequence b.  Per row (device, [rows]):
 *   src [rows, H]   fp32 state joined with the token: g (seed) or parent's a
 *   token           target id whose embedding joins the row; < 0 = padding
 *   position        RoPE position
 *   dest            cache row receiving the row's K/V (< cap)
 *   prefix_len      row sees cache rows [0, prefix_len)
 *   scratch_base    [batch] first scratch cache row of the sequence
 *   scratch_mask    row also sees scratch_base + j for every set bit j
 * Outputs: a_out [rows, H] fp32 (decoder output state), topk_id / topk_logit
 * [rows, K] ordered by (-logit, id) with draft-vocabulary ids, lse [rows]
 * (log-sum-exp of the row's fp32 logits).  The row's own K/V must be visible
 * to it through prefix_len or scratch_mask.  rows_per_seq in
 * [1, max(max_seed, topk)]. */
eagle_status eagle_draft_step(eagle_ctx *ctx, int32_t batch,
                              int32_t rows_per_seq, const void *src,
                              const int32_t *token, const int32_t *position,
                              const int32_t *dest, const int32_t *prefix_len,
                              const int32_t *scratch_base,
                              const uint64_t *scratch_mask, const eagle_kv *kv,
                              void *a_out, int32_t *topk_id, float *topk_logit,
                              float *lse, hipStream_t stream);

/* (2)+(3) Draft one EAGLE-2 tree per sequence ([M75] 0x06A-0x06B: value =
 * float32 sum of log(max(confidence, 1e-12)); each pass expands the K best
 * nodes of the newest layer under (-value, depth, node id); the final tree
 * is the global top-N, flattened; [E3] 3.4 Stage 1: the draft state a stands
 * in for g at drafted positions; [M75] 0x05A: seed rows [f_t, e(x_t+1)]).
 *   seed_src   [B, max_seed, H]  fp32 fused target features of the seed rows
 *   seed_token [B, max_seed]     target ids joined with them
 *   seed_len   [B]               rows used, 1..max_seed; the last is the root
 * Seed rows go to cache rows len_in[b] + i and attend causally; len_out[b] =
 * len_in[b] + seed_len[b]; the root sits at position len_out[b] - 1.  Then D
 * passes grow the tree; tree rows use scratch cache rows
 * [len_out, len_out + (D-1)K).  Needs len_out + (D-1)K <= cap (checked on
 * the device: ECAPACITY, n_nodes = -1).  D == 0 or N == 0 still commits the
 * seed rows and returns a root-only tree.  batch in [1, max_batch]. */
eagle_status eagle_draft_tree(eagle_ctx *ctx, int32_t batch,
                              const void *seed_src, const int32_t *seed_token,
                              const int32_t *seed_len, const eagle_kv *kv,
                              const eagle_tree *out, hipStream_t stream);

/* (2)+(3) eagle_draft_tree with sampled children ([E1] 3.4 "Tree-Structured
 * Draft Generation": at temperature > 0 the k children of a node are sampled
 * from the draft distribution).  Each expanded node (the root, then the K
 * nodes each pass expands) draws its K children from q = softmax(logits /
 * temperature) without replacement, by Gumbel-top-k: the K largest
 * logits[x] / temperature - log(-log u_x), ties to the lower id, in that
 * order; u_x = (top 24 bits of Philox4x64-10 word x % 4 + 1/2) * 2^-24 with
 * key (seed, EAGLE_STREAM_DRAFT) and counter (x / 4, key row, b, round), the
 * key row 0 for the root and 1 + the node's creation index (the order in
 * which the passes create candidates, K per expanded node) otherwise.  A
 * child's value is its parent's plus log q(x).  Every draw stays in the tree:
 * needs budget >= K + (D-1) K^2 (so the final top-N keeps all) and no d2t,
 * else EUNSUPPORTED; depth >= 1; temperature > 0 (EINVAL).  Siblings are
 * flattened in draw order (rows still ordered by depth, then parent row).
 *   draft_logits [B, 1 + (D-1) K, vocab] fp32, written: row 0 the root's
 *                logits, row 1 + s those of the node with scratch slot s --
 *                the q of every row that has children, for
 *                eagle_verify_tree_sampled.
 * Other arguments as eagle_draft_tree. */
eagle_status eagle_draft_tree_sampled(eagle_ctx *ctx, int32_t batch,
                                      const void *seed_src,
                                      const int32_t *seed_token,
                                      const int32_t *seed_len,
                                      const eagle_kv *kv, const eagle_tree *out,
                                      float temperature, uint64_t seed,
                                      uint64_t round, float *draft_logits,
                                      hipStream_t stream);

/* (4) Verify each sequence's tree ([E1] "Verification Phase: Multi-Round
 * Speculative Sampling on Trees", Algorithm 1; "The Full Inference Loop":
 * a >= 0 accepted draft tokens plus one emitted token) and commit.
 *   target_logits [B, N+1, TV] fp32: row r = target next-token logits after
 *                 tree row r.
 *   temperature   0 = greedy (argmax, lowest id on ties; the child carrying
 *                 it is accepted); > 0 = Algorithm 1 at p = softmax(l / T)
 *                 with the deterministic top-k children as point-mass
 *                 proposals, tested in ascending token id (accept child c
 *                 when u < p(c), else remove c's mass and renormalise), then
 *                 an inverse-CDF draw over ascending id from what is left.
 *   seed, round   draw j of row v of sequence b is Philox4x64-10 with key
 *                 (seed, EAGLE_STREAM_VERIFY) at counter (j, v, b, round):
 *                 j = child index, 63 for the residual draw; the value is
 *                 the first word's top 24 bits times 2^-24.
 *   commit_mode   eagle_commit_mode.
 *   kv_or_null    if given: with KEEP, accepted rows that hold computed draft
 *                 K/V move from scratch to cache row = position; with either
 *                 mode kv->len_out[b] receives the new committed length.
 * Outputs: accept_len [B] (0..D, -1 on a device error), accepted_rows [B, D]
 * (tree rows, -1 padded), out_tokens [B, D+1] (accepted tokens then the
 * emitted one, -1 padded), next_seed_rows / next_seed_tokens [B, max_seed]
 * and next_seed_len [B]: the next round's seed rows as (tree row whose target
 * feature is fused, target id joined with it), -1 padded. */
eagle_status eagle_verify_tree(eagle_ctx *ctx, int32_t batch,
                               const eagle_tree *tree,
                               const float *target_logits, float temperature,
                               uint64_t seed, uint64_t round,
                               int32_t commit_mode, const eagle_kv *kv_or_null,
                               int32_t *accept_len, int32_t *accepted_rows,
                               int32_t *out_tokens, int32_t *next_seed_rows,
                               int32_t *next_seed_tokens,
                               int32_t *next_seed_len, hipStream_t stream);

/* eagle_verify_tree for trees drafted by eagle_draft_tree_sampled:
 * Algorithm 1 of [E1] ("Verification Phase: Multi-Round Speculative Sampling
 * on Trees") with p = softmax(target_logits / T) and, for the i-th child (in
 * draw order) of a row, p_hat_i = softmax(draft_logits[row] / T) with the
 * earlier children's tokens removed and renormalised: child i is accepted
 * when u_i < p(t_i) / p_hat_i(t_i), else p <- norm(max(0, p - p_hat_i)); if
 * all are rejected (or the row has no children) the emitted token is drawn
 * from p by inverse CDF over ascending ids.  A residual of zero mass
 * restarts from the target distribution.  Draws, commit and outputs as
 * eagle_verify_tree.  draft_logits as eagle_draft_tree_sampled wrote them.
 * temperature > 0, else EINVAL; a context with d2t is EUNSUPPORTED. */
eagle_status eagle_verify_tree_sampled(
    eagle_ctx *ctx, int32_t batch, const eagle_tree *tree,
    const float *target_logits, const float *draft_logits, float temperature,
    uint64_t seed, uint64_t round, int32_t commit_mode,
    const eagle_kv *kv_or_null, int32_t *accept_len, int32_t *accepted_rows,
    int32_t *out_tokens, int32_t *next_seed_rows, int32_t *next_seed_tokens,
    int32_t *next_seed_len, hipStream_t stream);

/* eagle_verify_tree with explicit draws instead of Philox (the same
 * Algorithm 1 of [E1]): uniforms [B, N+1, K+1] fp32 in [0,1), column i < K
 * the draw for the i-th child of that row, column K the residual draw; may
 * be NULL when temperature == 0.  For replaying externally drawn numbers. */
eagle_status eagle_verify_tree_uniforms(
    eagle_ctx *ctx, int32_t batch, const eagle_tree *tree,
    const float *target_logits, float temperature, const float *uniforms,
    int32_t commit_mode, const eagle_kv *kv_or_null, int32_t *accept_len,
    int32_t *accepted_rows, int32_t *out_tokens, int32_t *next_seed_rows,
    int32_t *next_seed_tokens, int32_t *next_seed_len, hipStream_t stream);

/* eagle_verify_tree for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no context and no workspace.  The same verification and
 * commit, with the row statistics in a static device buffer of this library
 * (about 320 KB per GPU, held until the process ends).  Limits: batch *
 * (budget + 1) <= 16384, else EUNSUPPORTED; cfg is validated as by
 * eagle_create.  Calls that overlap on one GPU share that buffer and race;
 * order them.  Device-detected errors show only as accept_len = -1 (there is
 * no status word to read).  Allocates nothing. */
eagle_status eagle_verify_tree_noalloc(
    const eagle_config *cfg, int32_t batch, const eagle_tree *tree,
    const float *target_logits, float temperature, uint64_t seed,
    uint64_t round, int32_t commit_mode, const eagle_kv *kv_or_null,
    int32_t *accept_len, int32_t *accepted_rows, int32_t *out_tokens,
    int32_t *next_seed_rows, int32_t *next_seed_tokens, int32_t *next_seed_len,
    hipStream_t stream);

/* (5) The target's verification forward over the flattened tree ([E1] "The
 * Full Inference Loop", Phase 2: the target processes the prompt plus the
 * draft tree in one forward pass under tree attention; [E3] 3.4 "The
 * Inference Pipeline", Stage 2; [M75] 0x05C Target Verification), for a
 * synthetic one-layer target: the context's weights are the target's (an
 * eagle_create'd context of the target's shape; w_fuse and w_in are not
 * used here).  For every sequence b and tree row r <= n_nodes[b]:
 *   input      embed[token[b, r]]
 *   RoPE       at position[b, r]
 *   K/V        written to target cache row kv->len_in[b] + r
 *   attends    the committed prefix [0, len_in[b]) and the cache rows
 *              len_in[b] + j for the set bits j of mask[b, r, 0] (the row's
 *              ancestors and itself, as eagle_draft_tree flattens them)
 * then the decoder block and the LM head as in eagle_draft_step.
 *   tree        the flattened trees (token, position, mask, n_nodes read)
 *   kv          target cache, layout as eagle_kv; len_in [B] read, len_out
 *               unused; needs len_in + budget + 1 <= cap (else ECAPACITY in
 *               the status word and that sequence's rows are padding)
 *   workspace   device, >= eagle_target_layer_workspace_bytes(cfg, batch)
 *               bytes, 256-byte aligned, owned by the caller (scratch only)
 *   hidden_out  [B, N+1, H] fp32 block outputs, or NULL
 *   logits_out  [B, N+1, vocab] fp32 next-token logits after each row: the
 *               target_logits eagle_verify_tree takes.
 * Rows past n_nodes[b] are padding (zero logits).  Needs budget + 1 <= 64
 * (one mask word), else EUNSUPPORTED.  Asynchronous on `stream`. */
size_t eagle_target_layer_workspace_bytes(const eagle_config *cfg, int32_t batch);
eagle_status eagle_target_tree_layer(eagle_ctx *ctx, int32_t batch,
                                     const eagle_tree *tree, const eagle_kv *kv,
                                     void *workspace, size_t ws_bytes,
                                     float *hidden_out, float *logits_out,
                                     hipStream_t stream);

/* The draws the sampling steps use ([E1] Algorithm 1: "draw r ~ U(0,1)"):
 * out[b, r, j] = U(seed, stream_id; counter (j, r, b, round)) for b < batch,
 * r < rows, j < draws, as described at eagle_verify_tree.  out is fp32
 * [batch, rows, draws]; batch, rows <= 65535.  No context needed. */
eagle_status eagle_draw_uniforms(uint64_t seed, uint64_t stream_id,
                                 uint64_t round, int32_t batch, int32_t rows,
                                 int32_t draws, float *out, hipStream_t stream);

/* Measurement hook.  While profiling is on, every kernel the context enqueues
 * is bracketed by a pair of HIP events on its stream (up to 8192 launches
 * between reads).  eagle_profile(ctx, 1) clears the record and starts,
 * eagle_profile(ctx, 2) resumes adding to it, eagle_profile(ctx, 0) stops
 * and keeps it (so a caller can sample some launches of a longer run); other
 * values are EINVAL.  eagle_profile_read
 * synchronises on the last event and returns, per kernel class, the summed
 * event time (ms), launch count, algorithmic bytes (weights once +
 * activations in/out; the target logits for verification) and algorithmic
 * flops, then clears the record.
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
