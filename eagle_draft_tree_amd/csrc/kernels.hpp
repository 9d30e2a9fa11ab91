// Internal launch interfaces of the gfx950 kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eagle {

enum Epi : int {
  EPI_STORE = 0,   // out = round(C)            (+ row sum of squares)
  EPI_RESID = 1,   // out = round(C + resid)    (+ row sum of squares)
  EPI_QKV = 2,     // RoPE on q/k, q -> buffer, k/v -> draft KV cache
  EPI_SWIGLU = 3,  // out = round(silu(gate) * up)
  EPI_LMHEAD = 4   // per-64-column top-k candidates + (max, sumexp)
};
enum ColMap : int { MAP_IDENT = 0, MAP_QKV = 1, MAP_SWIGLU = 2 };

// One K-range segment of the A operand (rows of activations).
struct ASeg {
  const void* base = nullptr;     // [rows, ld] elements
  int64_t ld = 0;
  const int32_t* rowidx = nullptr;  // optional row gather; <0 or >= rowlimit -> zero row
  int rowlimit = 0;
  int width = 0;                  // K elements in this segment (multiple of 8)
  const float* ss = nullptr;      // optional RMSNorm: per-row sums of squares of
  int ss_tiles = 0;               //   the producer, [rows, ss_tiles] partials
  const void* gain = nullptr;     // RMSNorm gain [width] (weight type)
  int f32 = 1;                    // elements are float activations (else weight type)
};

struct GemmParams {
  int M = 0, N = 0, K = 0;        // N: logical output columns (multiple of 16)
  int nseg = 1;
  ASeg seg[3];
  const void* wpack = nullptr;    // weights packed by launch_pack (read by the GEMM)
  const void* w0 = nullptr;       // weights [rows, K]; see ColMap (read by the packer)
  const void* w1 = nullptr;
  const void* w2 = nullptr;
  int colmap = MAP_IDENT;
  int qkv_n0 = 0, qkv_n1 = 0;     // columns served by w0, then w1, rest w2
  int hd = 0;
  // launch plan (plan_gemm): row tiles MT x 16 rows per chunk, CT 16-column
  // tiles per wave (a workgroup covers 64 CT columns), S splits of K of KS
  // elements each (KS a multiple of 128)
  int MT = 1, CT = 1, S = 1, KS = 128;
  int piece_steps = 8;            // k steps of A staged in LDS at a time
  int Mtot = 0;                   // padded rows of the partial buffer
  float* part = nullptr;          // [S, Mtot, N] split-K partials
  int64_t part_elems = 0;         // capacity of part (floats)
  int* cnt = nullptr;             // per (row chunk, column group) arrival counters (zero)
  // dense path (more than 64 rows): A staged once per launch as bf16 hi/lo
  // fragments, [rows/16][k steps][4][2 KB]; apack_rows rows fit
  void* apack = nullptr;
  int apack_rows = 0;
  int dense = 0;                  // set by plan_gemm
  int epi = EPI_STORE;
  void* out = nullptr;            // float activations (q: weight type)
  int64_t ldo = 0;
  const int32_t* out_row = nullptr;  // STORE: output row of row m (< 0: dropped), or identity
  const float* resid = nullptr;
  int64_t ldr = 0;
  float* ss = nullptr;            // [M, N/16] sums of squares per 16-column tile
  float eps = 1e-5f;              // RMSNorm epsilon of the A operand
  // QKV epilogue
  const int32_t* pos = nullptr;
  const int32_t* dest = nullptr;
  const int32_t* tok = nullptr;   // row valid iff tok[m] >= 0
  int rows_per_seq = 1;
  void* kc = nullptr;
  void* vc = nullptr;
  int cap = 0, nq = 0, nkv = 0, batch = 0;
  float theta = 10000.f;
  int* status = nullptr;
  // LM-head epilogue
  float* lm_logits = nullptr;     // [M, 64 ntile_lm] LM-head logits
  float* stat = nullptr;          // [M, ntile_lm, 2]: per 64-column tile max, sum exp
  int ntile_lm = 0;
};

void plan_gemm(GemmParams& p, int num_cus, bool fp32);
// Weights of one GEMM (w0..w2, colmap, N, K of p) copied into dst in the
// MFMA fragment order the GEMM streams; packed_elems(N, K) elements.
int64_t packed_elems(int N, int K);
template <typename T> hipError_t launch_pack(const GemmParams& p, void* dst, hipStream_t s);
template <typename T> hipError_t launch_gemm(const GemmParams& p, hipStream_t s);

// tree attention --------------------------------------------------------------
struct AttnParams {
  int batch = 0, rows_per_seq = 0;
  int nq = 0, nkv = 0, hd = 0, cap = 0;
  const void* q = nullptr;          // [rows, nq, hd]
  float* o = nullptr;               // [rows, nq, hd] float
  const void* kc = nullptr;         // [B, nkv, cap, hd]
  const void* vc = nullptr;         // [B, nkv, hd, cap] (V stored transposed)
  const int32_t* tok = nullptr;     // row valid iff tok >= 0
  const int32_t* plen = nullptr;    // [rows]
  const int32_t* sbase = nullptr;   // [B]
  const uint64_t* smask = nullptr;  // [rows]
  int nsplit = 1;                   // prefix splits (plus one scratch split)
  int split_keys = 64;              // keys per prefix split (multiple of 64)
                                    // cap: a multiple of 8, at least 32
  float* part_o = nullptr;          // [B, nkv, nsplit+1, QG, hd]
  float* part_ml = nullptr;         // [B, nkv, nsplit+1, QG, 2]
  float scale = 1.f;
};
template <typename T> hipError_t launch_attention(const AttnParams& p, hipStream_t s);

// LM-head merge, tree growth, verification -----------------------------------
struct MergeParams {
  int rows = 0, ntile = 0, topk = 0, V = 0;
  const float* logits = nullptr;     // [rows, 64 ntile]
  const float* stat = nullptr;       // [rows, ntile, 2]
  const int32_t* tok = nullptr;      // only rows with tok >= 0 are merged
  int32_t* out_id = nullptr;         // [rows, topk]
  float* out_val = nullptr;          // [rows, topk]
  float* out_lse = nullptr;          // [rows]
};
hipError_t launch_merge(const MergeParams& p, hipStream_t s);

struct TreeState {
  // candidates [B, ncand_max]
  int32_t* c_token; int32_t* c_parent; int32_t* c_slot; int32_t* c_row;
  float* c_score; uint64_t* c_mask; int32_t* c_depth;
  int32_t* n_cand;        // [B]
  int32_t* p_root;        // [B] root position
  int32_t* len_out;       // [B]
  int ncand_max;
};

struct QueryDesc {  // one pass's query rows, [B * rows_per_seq] each
  int32_t* tok; int32_t* src_row; int32_t* pos; int32_t* dest; int32_t* plen;
  uint64_t* mask; int32_t* node;
};

struct SeedParams {
  int batch, s_max, K, D, cap;
  const int32_t* seed_token; const int32_t* seed_len; const int32_t* len_in;
  int32_t* len_out;
  QueryDesc q;        // pass-1 rows [B * s_max]
  int32_t* sbase;     // [B] scratch base = len_out
  TreeState ts;
  int* status;
};
hipError_t launch_seed_setup(const SeedParams& p, hipStream_t s);

struct GrowParams {
  int batch, K, D, N, pass, rows_per_seq, s_max;
  int sampled = 0;      // children in draw order (sampled), else by token id
  const int32_t* d2t;   // draft id -> target id, or null (same vocabulary)
  const int32_t* topk_id; const float* topk_val; const float* lse;
  QueryDesc cur;      // this pass's rows
  QueryDesc nxt;      // next pass's rows [B * K]
  TreeState ts;
  const int32_t* seed_token; const int32_t* seed_len;
  // final outputs
  int32_t *t_token, *t_parent, *t_depth, *t_pos, *t_slot, *t_first, *t_nchild;
  float* t_score; uint64_t* t_mask; int32_t* t_n;
  int mask_words;
};
hipError_t launch_grow(const GrowParams& p, hipStream_t s);

struct VerifyParams {
  int batch, N, K, D, V;
  float T;
  const float* logits;      // [B, N+1, V]
  const float* uniforms;    // [B, N+1, K+1] or null: Philox draws of (seed, round)
  uint64_t seed, round;
  int commit_mode;          // 0 keep computed draft rows, 1 full reseed
  int S;                    // seed slots per sequence in the seed outputs
  const int32_t *t_token, *t_parent, *t_depth, *t_pos, *t_slot, *t_first,
      *t_nchild, *t_n;
  float* row_max; double* row_sum; int32_t* row_arg; int32_t* row_bad;
  int32_t *accept_len, *accepted_rows, *out_tokens, *seed_rows, *seed_tokens,
      *seed_len;
  void* kc; void* vc; int cap, nkv, hd; int32_t* kv_len;  // kc null: no commit
  int elem_bytes;
  int* status;
  // sampled children: draft logits of the expanded nodes [B, NE, V] (row 0
  // the root, 1 + kv_slot a drafted node), or null for point-mass children
  const float* draft_rows = nullptr;
  int NE = 0;
};
hipError_t launch_verify(const VerifyParams& p, hipStream_t s);

// sampled children of one pass: per query row with a draft-logit row
// (out_row >= 0), K draws without replacement from softmax(logits / T) by
// Gumbel-top-k with Philox (seed, draft stream) noise at counter
// (token / 4, key row, sequence, round); writes the tokens in draw order,
// logits / T of the drawn tokens and log-sum-exp(logits / T), in the layout
// of the LM-head merge
struct SampleParams {
  int rows = 0, rows_per_seq = 0, pass = 0, K = 0, V = 0, NE = 0;
  float T = 1.f;
  uint64_t seed = 0, round = 0;
  const int32_t* tok = nullptr;      // query rows (tok < 0: padding)
  const int32_t* dest = nullptr;
  const int32_t* plen = nullptr;
  const int32_t* node = nullptr;     // candidate id of a pass >= 2 row
  int32_t* out_row = nullptr;        // [rows] draft-logit row of each query row
  const float* logits = nullptr;     // [B * NE, V]
  int32_t* topk_id = nullptr;        // [rows, K]
  float* topk_val = nullptr;
  float* lse = nullptr;
};
hipError_t launch_slot_rows(const SampleParams& p, hipStream_t s);
hipError_t launch_sample_children(const SampleParams& p, hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s);

// target tree layer: per-row descriptors from the flattened tree, and the
// block input x = E[token] (fp32) with its per-16-column sums of squares
struct TargetRowsParams {
  int batch = 0, n1 = 0, cap = 0, mask_words = 1;
  const int32_t* len_in = nullptr;     // [B] committed length = first tree cache row
  const int32_t* token = nullptr;      // tree arrays [B, n1]
  const int32_t* position = nullptr;
  const uint64_t* mask = nullptr;      // [B, n1, mask_words]
  const int32_t* n_nodes = nullptr;    // [B]
  int32_t *tok = nullptr, *pos = nullptr, *dest = nullptr, *plen = nullptr;  // [B*n1]
  uint64_t* rmask = nullptr;           // [B*n1]
  int32_t* sbase = nullptr;            // [B]
  int* status = nullptr;
};
hipError_t launch_target_rows(const TargetRowsParams& p, hipStream_t s);
template <typename T>
hipError_t launch_embed_rows(const T* embed, int vocab, const int32_t* tok, int rows, int H,
                             float* x, float* ss, hipStream_t s);
hipError_t launch_uniforms(uint64_t seed, uint64_t stream, uint64_t rnd, int batch, int rows,
                           int draws, float* out, hipStream_t s);

}  // namespace eagle
