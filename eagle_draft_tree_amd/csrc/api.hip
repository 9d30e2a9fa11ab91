// C ABI: argument validation, workspace layout and the launch sequence of a
// draft pass, a tree and a verification.  No device memory is allocated here;
// everything lives in the caller's workspace.
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>

#include "../../include/eagle.h"
#include "common.hpp"
#include "kernels.hpp"

using namespace eagle;

namespace {

// Most prefix splits of the tree attention for a batch: enough waves to fill
// the chip at batch 1, a bounded partial-sum buffer at large batch.
int attn_max_split(int batch, int nkv) {
  const int w = 4096 / std::max(1, batch * nkv);
  return std::min(64, std::max(4, w));
}
constexpr size_t kAlign = 256;

struct Layout {
  size_t total = 0;
  size_t take(size_t bytes) {
    const size_t o = total;
    total += (bytes + kAlign - 1) / kAlign * kAlign;
    return o;
  }
};

struct Offsets {
  size_t x, h, a0, a1, q, o, t, ss, part, lm_logits,
      lm_stat, tk_id, tk_val, lse, at_o, at_ml, desc[2][7], sbase, c_token,
      c_parent, c_slot, c_row, c_score, c_mask, c_depth, n_cand, p_root,
      len_out, v_max, v_sum, v_arg, v_bad, status, counters_begin, counters_end,
      cnt_gemm, pack[7], apack, orow;
  int R, Rpad, ncnt, ntile_lm, qg, ncand, max_split, apack_rows;
  int64_t part_elems;
  size_t total;
};

int esize(const eagle_config& c) { return c.dtype == EAGLE_BF16 ? 2 : 4; }

// The seven weight matrices the GEMMs stream, each packed once into the
// workspace at create time.
enum GemmId { G_FUSE = 0, G_IN, G_QKV, G_O, G_GU, G_DOWN, G_LM, G_COUNT };

// N, K, sources and column map of GEMM `id` (sources only when w != null)
void gemm_shape(const eagle_config& c, const eagle_weights* w, int id, GemmParams& p) {
  const int H = c.hidden, F = c.ffn, V = c.vocab;
  const int qd = c.n_q_heads * c.head_dim, kd = c.n_kv_heads * c.head_dim;
  p.colmap = MAP_IDENT;
  switch (id) {
    case G_FUSE: p.N = H; p.K = 3 * H; if (w) p.w0 = w->w_fuse; break;
    case G_IN: p.N = H; p.K = 2 * H; if (w) p.w0 = w->w_in; break;
    case G_QKV:
      p.N = qd + 2 * kd; p.K = H; p.colmap = MAP_QKV; p.qkv_n0 = qd; p.qkv_n1 = kd;
      p.hd = c.head_dim;
      if (w) { p.w0 = w->wq; p.w1 = w->wk; p.w2 = w->wv; }
      break;
    case G_O: p.N = H; p.K = qd; if (w) p.w0 = w->wo; break;
    case G_GU:
      p.N = 2 * F; p.K = H; p.colmap = MAP_SWIGLU;
      if (w) { p.w0 = w->w_gate; p.w1 = w->w_up; }
      break;
    case G_DOWN: p.N = H; p.K = F; if (w) p.w0 = w->w_down; break;
    default: p.N = V; p.K = H; if (w) p.w0 = w->w_lm; break;
  }
}
// token ids of the tree, the embedding and the target logits
int tvocab(const eagle_config& c) { return c.target_vocab > 0 ? c.target_vocab : c.vocab; }

eagle_status check_config(const eagle_config* c) {
  if (c == nullptr) return EAGLE_EINVAL;
  if (c->hidden <= 0 || c->n_q_heads <= 0 || c->n_kv_heads <= 0 ||
      c->head_dim <= 0 || c->ffn <= 0 || c->vocab <= 0 || c->depth < 0 ||
      c->topk < 1 || c->budget < 0 || c->max_batch < 1 || c->max_seed < 1 ||
      !(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f))
    return EAGLE_EINVAL;
  if (c->dtype != EAGLE_BF16 && c->dtype != EAGLE_FP32) return EAGLE_EINVAL;
  if (c->head_dim != 64 && c->head_dim != 128) return EAGLE_EUNSUPPORTED;
  if (c->n_q_heads % c->n_kv_heads) return EAGLE_EUNSUPPORTED;
  if (c->hidden % 16 || c->ffn % 8 || c->vocab % 16) return EAGLE_EUNSUPPORTED;
  if (c->topk > kMaxTopK || c->vocab < c->topk) return EAGLE_EUNSUPPORTED;
  if (c->depth > 0 && (c->depth - 1) * c->topk > 64) return EAGLE_EUNSUPPORTED;
  if (c->budget + 1 > 128 || c->max_seed > 16) return EAGLE_EUNSUPPORTED;
  const int rps = std::max(c->max_seed, c->topk);
  const int G = c->n_q_heads / c->n_kv_heads;
  if (rps * G > 128) return EAGLE_EUNSUPPORTED;
  if (c->dtype == EAGLE_FP32 && (c->max_batch * rps > 64 || c->head_dim != 64))
    return EAGLE_EUNSUPPORTED;
  if (c->max_batch > 4096) return EAGLE_EUNSUPPORTED;
  if (c->target_vocab < 0) return EAGLE_EINVAL;
  if (c->target_vocab != 0 && c->target_vocab < c->vocab) return EAGLE_EINVAL;
  return EAGLE_OK;
}

Offsets make_layout(const eagle_config& c) {
  Offsets f;
  Layout L;
  const int es = esize(c);
  const int H = c.hidden, F = c.ffn, V = c.vocab, B = c.max_batch;
  const int qd = c.n_q_heads * c.head_dim, kd = c.n_kv_heads * c.head_dim;
  const int rps = std::max(c.max_seed, c.topk);
  f.R = B * rps;
  f.Rpad = (f.R + 63) / 64 * 64;
  const size_t R = f.Rpad;
  // activations are float; q is stored in the weight type like the KV cache
  f.x = L.take(R * H * 4);
  f.h = L.take(R * H * 4);
  f.a0 = L.take(R * H * 4);
  f.a1 = L.take(R * H * 4);
  f.q = L.take(R * qd * es);
  f.o = L.take(R * qd * 4);
  f.t = L.take(R * F * 4);
  f.ss = L.take(R * (H / 16) * 4);
  // split-K partials: up to 16 splits of 32 rows of the widest GEMM
  const int maxN = std::max(std::max(V, 2 * F), std::max(3 * H, qd + 2 * kd));
  f.part_elems = static_cast<int64_t>(16) * std::min<int64_t>(R, 32) * maxN;
  f.part = L.take(static_cast<size_t>(f.part_elems) * 4);
  // dense path (bf16, more than 64 rows): A as packed bf16 hi/lo fragments,
  // 4 bytes per element of the widest K
  f.apack_rows = (c.dtype == EAGLE_BF16 && f.R > 64) ? (f.R + 63) / 64 * 64 : 0;
  {
    const int kmax = std::max(std::max(3 * H, F), qd);
    f.apack = L.take(static_cast<size_t>(f.apack_rows) * ((kmax + 127) / 128 * 128) * 4);
  }
  f.orow = L.take(R * 4);
  f.ntile_lm = (V + 63) / 64;
  f.lm_logits = L.take(static_cast<size_t>(R) * f.ntile_lm * 64 * 4);
  f.lm_stat = L.take(R * f.ntile_lm * 2 * 4);
  f.tk_id = L.take(R * c.topk * 4);
  f.tk_val = L.take(R * c.topk * 4);
  f.lse = L.take(R * 4);
  f.qg = rps * (c.n_q_heads / c.n_kv_heads);
  f.max_split = attn_max_split(B, c.n_kv_heads);
  const size_t bk = static_cast<size_t>(B) * c.n_kv_heads * (f.max_split + 1) * f.qg;
  f.at_o = L.take(bk * c.head_dim * 4);
  f.at_ml = L.take(bk * 2 * 4);
  for (int s = 0; s < 2; ++s)
    for (int k = 0; k < 7; ++k) f.desc[s][k] = L.take(R * (k == 5 ? 8 : 4));
  f.sbase = L.take(B * 4);
  f.ncand = c.depth > 0 ? c.topk + (c.depth - 1) * c.topk * c.topk : 1;
  const size_t BC = static_cast<size_t>(B) * f.ncand;
  f.c_token = L.take(BC * 4);
  f.c_parent = L.take(BC * 4);
  f.c_slot = L.take(BC * 4);
  f.c_row = L.take(BC * 4);
  f.c_score = L.take(BC * 4);
  f.c_mask = L.take(BC * 8);
  f.c_depth = L.take(BC * 4);
  f.n_cand = L.take(B * 4);
  f.p_root = L.take(B * 4);
  f.len_out = L.take(B * 4);
  const size_t BN = static_cast<size_t>(B) * (c.budget + 1);
  f.v_max = L.take(BN * 4);
  f.v_sum = L.take(BN * 8);
  f.v_arg = L.take(BN * 4);
  f.v_bad = L.take(BN * 4);
  // counters: zeroed once, every user resets what it touches
  f.counters_begin = L.total;
  f.cnt_gemm = L.take(static_cast<size_t>(f.Rpad / 16 + 1) * (maxN / 64 + 1) * 4);
  f.status = L.take(4);
  f.counters_end = L.total;
  for (int id = 0; id < G_COUNT; ++id) {
    GemmParams p;
    gemm_shape(c, nullptr, id, p);
    f.pack[id] = L.take(static_cast<size_t>(packed_elems(p.N, p.K)) * es);
  }
  f.ncnt = static_cast<int>((f.counters_end - f.counters_begin) / 4);
  f.total = L.total;
  return f;
}

}  // namespace

// Optional per-launch timing: HIP events around each kernel of a context.
struct Profiler {
  static constexpr int kPairs = 8192;
  bool on = false;
  int used = 0;
  bool overflow = false;
  hipEvent_t ev[2 * kPairs] = {};
  int cls[kPairs] = {};
  double bytes[kPairs] = {};
  double flops[kPairs] = {};
  bool created = false;
};

struct eagle_ctx {
  eagle_config cfg;
  eagle_weights w;
  char* ws;
  Offsets off;
  int num_cus;
  Profiler prof;
  template <typename P> P* at(size_t o) const { return reinterpret_cast<P*>(ws + o); }
  int* status() const { return at<int>(off.status); }
  // shape, column map and packed weights of GEMM `id`
  void shape(int id, GemmParams& p) const {
    gemm_shape(cfg, nullptr, id, p);
    p.wpack = at<char>(off.pack[id]);
  }
};

namespace {

// Activation, partial-sum and candidate buffers of one layer pass: the
// context's workspace for draft passes, the caller's for the target layer.
struct Scratch {
  char *x = nullptr, *h = nullptr, *o = nullptr, *t = nullptr, *q = nullptr;
  float* ss = nullptr;
  float* part = nullptr;
  int64_t part_elems = 0;
  int* cnt = nullptr;
  char* apack = nullptr;
  int apack_rows = 0;
  float *at_o = nullptr, *at_ml = nullptr;
  int max_split = 1;
  float* lm_logits = nullptr;
  float* lm_stat = nullptr;
  int ntile_lm = 0;
};

Scratch ctx_scratch(eagle_ctx* c) {
  const Offsets& f = c->off;
  Scratch r;
  r.x = c->at<char>(f.x); r.h = c->at<char>(f.h); r.o = c->at<char>(f.o);
  r.t = c->at<char>(f.t); r.q = c->at<char>(f.q); r.ss = c->at<float>(f.ss);
  r.part = c->at<float>(f.part); r.part_elems = f.part_elems;
  r.cnt = c->at<int>(f.cnt_gemm);
  r.apack = f.apack_rows > 0 ? c->at<char>(f.apack) : nullptr;
  r.apack_rows = f.apack_rows;
  r.at_o = c->at<float>(f.at_o); r.at_ml = c->at<float>(f.at_ml); r.max_split = f.max_split;
  r.lm_logits = c->at<float>(f.lm_logits);
  r.lm_stat = c->at<float>(f.lm_stat); r.ntile_lm = f.ntile_lm;
  return r;
}

// kernel classes reported by eagle_profile_read
enum ProfClass { PC_GEMM = 0, PC_FUSE = 1, PC_ATTN = 2, PC_MERGE = 3, PC_TREE = 4,
                 PC_VERIFY = 5, PC_COUNT = 6 };

int prof_begin(eagle_ctx* c, int cls, double bytes, double flops, hipStream_t s) {
  Profiler& p = c->prof;
  if (!p.on) return -1;
  if (p.used >= Profiler::kPairs) {
    p.overflow = true;
    return -1;
  }
  const int i = p.used++;
  p.cls[i] = cls;
  p.bytes[i] = bytes;
  p.flops[i] = flops;
  if (hipEventRecord(p.ev[2 * i], s) != hipSuccess) p.overflow = true;
  return i;
}
void prof_end(eagle_ctx* c, int i, hipStream_t s) {
  if (i >= 0 && hipEventRecord(c->prof.ev[2 * i + 1], s) != hipSuccess)
    c->prof.overflow = true;
}

// Sampled children of a tree pass: where the expanded nodes' draft logits
// go ([B, 1 + (D-1) K, V]) and the draw parameters.
struct SampleSpec {
  float* rows;
  float T;
  uint64_t seed, round;
};

struct Rows {  // one pass's query rows
  int batch, rps;
  const void* src;           // rows gathered through src_row (or identity)
  const int32_t* src_row;    // may be null: row r reads src row r
  int src_rows;              // rows addressable in src
  const int32_t *tok, *pos, *dest, *plen, *sbase;
  const uint64_t* mask;
  void* a_out;
  int32_t* topk_id;
  float* topk_val;
  float* lse;
  const int32_t* node = nullptr;   // candidate id of each row (tree passes)
  int pass = 0;                    // tree pass (1 = seed rows)
  const SampleSpec* sample = nullptr;
};

template <typename T>
hipError_t run_gemm(eagle_ctx* c, const Scratch& scr, GemmParams& p, hipStream_t s,
                    int cls = PC_GEMM) {
  double a_bytes = 0;
  for (int i = 0; i < p.nseg; ++i)
    a_bytes += static_cast<double>(p.M) * p.seg[i].width * (p.seg[i].f32 ? 4 : sizeof(T));
  p.Mtot = (p.M + 15) / 16 * 16;
  p.part = scr.part;
  p.part_elems = scr.part_elems;
  p.cnt = scr.cnt;
  p.eps = c->cfg.rms_eps;
  p.apack = scr.apack;
  p.apack_rows = scr.apack_rows;
  plan_gemm(p, c->num_cus, sizeof(T) == 4);
  // algorithmic bytes: weights once, activation rows in, results out
  const double w_bytes = static_cast<double>(p.N) * p.K * sizeof(T);
  const double out_bytes = p.epi == EPI_LMHEAD ? 0.0 : static_cast<double>(p.M) * p.N * 4;
  const int pi = prof_begin(c, cls, w_bytes + a_bytes + out_bytes,
                            2.0 * p.M * static_cast<double>(p.N) * p.K, s);
  hipError_t e = launch_gemm<T>(p, s);
  prof_end(c, pi, s);
  return e;
}

#define EAGLE_TRY(x)                        \
  do {                                      \
    if ((x) != hipSuccess) return EAGLE_EHIP; \
  } while (0)

// One decoder block over rows r whose input x already sits in scr.x (with
// its per-16-column sums of squares in scr.ss): RMSNorm -> QKV -> RoPE ->
// cache rows, tree attention, O-projection + residual, RMSNorm -> SwiGLU ->
// down + residual into a_out, then the final norm and the LM head: per-row
// top-k and log-sum-exp into r.topk_* / r.lse, or (logits != null) every
// logit, fp32 [rows, V].
template <typename T>
eagle_status run_block(eagle_ctx* c, const Scratch& scr, const Rows& r, const eagle_kv* kv,
                       void* a_out, float* logits, hipStream_t s) {
  const eagle_config& cf = c->cfg;
  const int H = cf.hidden, F = cf.ffn;
  const int qd = cf.n_q_heads * cf.head_dim;
  const int R = r.batch * r.rps;
  // a3 RMSNorm -> QKV -> RoPE -> q buffer + KV cache rows
  {
    GemmParams p;
    c->shape(G_QKV, p);
    p.M = R; p.nseg = 1;
    p.seg[0].base = scr.x; p.seg[0].ld = H; p.seg[0].width = H;
    p.seg[0].ss = scr.ss; p.seg[0].ss_tiles = H / 16;
    p.seg[0].gain = c->w.g_attn;
    p.epi = EPI_QKV; p.out = scr.q; p.ldo = qd;
    p.pos = r.pos; p.dest = r.dest; p.tok = r.tok; p.rows_per_seq = r.rps;
    p.kc = kv->k; p.vc = kv->v; p.cap = kv->cap; p.nq = cf.n_q_heads;
    p.nkv = cf.n_kv_heads; p.batch = r.batch; p.theta = cf.rope_theta;
    p.status = c->status();
    EAGLE_TRY(run_gemm<T>(c, scr, p, s));
  }
  // a4 tree attention
  {
    AttnParams p;
    p.batch = r.batch; p.rows_per_seq = r.rps; p.nq = cf.n_q_heads;
    p.nkv = cf.n_kv_heads; p.hd = cf.head_dim; p.cap = kv->cap;
    p.q = scr.q; p.o = reinterpret_cast<float*>(scr.o);
    p.kc = kv->k; p.vc = kv->v; p.tok = r.tok; p.plen = r.plen;
    p.sbase = r.sbase; p.smask = r.mask;
    // splits: about 2048 workgroups over the batch (each stages 32-key
    // steps of K and V for up to four 16-query blocks), at least 128 keys
    // each (shorter splits cost more in the merge than they save: 3 us per
    // pass at one sequence of 2048 keys)
    constexpr int kMinSplitKeys = 128;
    const int G = cf.n_q_heads / cf.n_kv_heads;
    const int nrounds = ((r.rps * G + 15) / 16 + 3) / 4;
    const int want = std::max(1, 2048 / std::max(1, r.batch * cf.n_kv_heads * nrounds));
    int nsplit = std::min(
        {scr.max_split, std::max(1, (kv->cap + kMinSplitKeys - 1) / kMinSplitKeys), want});
    const int split_keys =
        std::max(kMinSplitKeys, ((kv->cap + nsplit - 1) / nsplit + 63) / 64 * 64);
    nsplit = (kv->cap + split_keys - 1) / split_keys;
    p.nsplit = nsplit; p.split_keys = split_keys;
    p.part_o = scr.at_o; p.part_ml = scr.at_ml;
    p.scale = 1.0f / sqrtf(static_cast<float>(cf.head_dim));
    const int pi = prof_begin(c, PC_ATTN, 0.0, 0.0, s);
    EAGLE_TRY(launch_attention<T>(p, s));
    prof_end(c, pi, s);
  }
  // a5 h = x + Wo o
  {
    GemmParams p;
    c->shape(G_O, p);
    p.M = R; p.nseg = 1;
    p.seg[0].base = scr.o; p.seg[0].ld = qd; p.seg[0].width = qd;
    p.epi = EPI_RESID; p.out = scr.h; p.ldo = H;
    p.resid = reinterpret_cast<const float*>(scr.x); p.ldr = H;
    p.ss = scr.ss;
    EAGLE_TRY(run_gemm<T>(c, scr, p, s));
  }
  // a6 t = silu(Wg n2) * (Wu n2)
  {
    GemmParams p;
    c->shape(G_GU, p);
    p.M = R; p.nseg = 1;
    p.seg[0].base = scr.h; p.seg[0].ld = H; p.seg[0].width = H;
    p.seg[0].ss = scr.ss; p.seg[0].ss_tiles = H / 16;
    p.seg[0].gain = c->w.g_mlp;
    p.epi = EPI_SWIGLU; p.out = scr.t; p.ldo = F;
    EAGLE_TRY(run_gemm<T>(c, scr, p, s));
  }
  //    a = h + Wd t
  {
    GemmParams p;
    c->shape(G_DOWN, p);
    p.M = R; p.nseg = 1;
    p.seg[0].base = scr.t; p.seg[0].ld = F; p.seg[0].width = F;
    p.epi = EPI_RESID; p.out = a_out; p.ldo = H;
    p.resid = reinterpret_cast<const float*>(scr.h); p.ldr = H;
    p.ss = scr.ss;
    EAGLE_TRY(run_gemm<T>(c, scr, p, s));
  }
  // a7 final norm -> LM head (logits + per-tile max / sum exp) -> merge (or every logit)
  {
    GemmParams p;
    c->shape(G_LM, p);
    p.M = R; p.nseg = 1;
    p.seg[0].base = a_out; p.seg[0].ld = H; p.seg[0].width = H;
    p.seg[0].ss = scr.ss; p.seg[0].ss_tiles = H / 16;
    p.seg[0].gain = c->w.g_final;
    if (logits != nullptr) {
      p.epi = EPI_STORE; p.out = logits; p.ldo = cf.vocab;
      EAGLE_TRY(run_gemm<T>(c, scr, p, s));
      return EAGLE_OK;
    }
    if (r.sample != nullptr) {
      // sampled children: every logit of the expanded rows is kept (the
      // verification needs their distributions), then K Gumbel-top-k draws
      SampleParams sp;
      sp.rows = R; sp.rows_per_seq = r.rps; sp.pass = r.pass; sp.K = cf.topk;
      sp.V = cf.vocab; sp.NE = 1 + std::max(cf.depth - 1, 0) * cf.topk;
      sp.T = r.sample->T; sp.seed = r.sample->seed; sp.round = r.sample->round;
      sp.tok = r.tok; sp.dest = r.dest; sp.plen = r.plen; sp.node = r.node;
      sp.out_row = c->at<int32_t>(c->off.orow); sp.logits = r.sample->rows;
      sp.topk_id = r.topk_id; sp.topk_val = r.topk_val; sp.lse = r.lse;
      EAGLE_TRY(launch_slot_rows(sp, s));
      p.epi = EPI_STORE; p.out = r.sample->rows; p.ldo = cf.vocab; p.out_row = sp.out_row;
      EAGLE_TRY(run_gemm<T>(c, scr, p, s));
      const int pi = prof_begin(c, PC_MERGE, 0.0, 0.0, s);
      EAGLE_TRY(launch_sample_children(sp, s));
      prof_end(c, pi, s);
      return EAGLE_OK;
    }
    p.epi = EPI_LMHEAD;
    p.lm_logits = scr.lm_logits; p.stat = scr.lm_stat; p.ntile_lm = scr.ntile_lm;
    EAGLE_TRY(run_gemm<T>(c, scr, p, s));
    MergeParams m;
    m.rows = R; m.ntile = scr.ntile_lm; m.topk = cf.topk; m.V = cf.vocab;
    m.logits = p.lm_logits; m.stat = p.stat;
    m.tok = r.tok; m.out_id = r.topk_id; m.out_val = r.topk_val; m.out_lse = r.lse;
    const int pi = prof_begin(c, PC_MERGE, 0.0, 0.0, s);
    EAGLE_TRY(launch_merge(m, s));
    prof_end(c, pi, s);
  }
  return EAGLE_OK;
}

// One draft pass: a2 join x = W_I [src ; E[tok]], then the block.
template <typename T>
eagle_status run_layer(eagle_ctx* c, const Rows& r, const eagle_kv* kv, hipStream_t s) {
  const eagle_config& cf = c->cfg;
  const int H = cf.hidden;
  const Scratch scr = ctx_scratch(c);
  {
    GemmParams p;
    c->shape(G_IN, p);
    p.M = r.batch * r.rps; p.nseg = 2;
    p.seg[0].base = r.src; p.seg[0].ld = H; p.seg[0].rowidx = r.src_row;
    p.seg[0].rowlimit = r.src_rows; p.seg[0].width = H;
    p.seg[1].base = c->w.embed; p.seg[1].ld = H; p.seg[1].rowidx = r.tok;
    p.seg[1].rowlimit = tvocab(cf); p.seg[1].width = H; p.seg[1].f32 = 0;
    p.epi = EPI_STORE; p.out = scr.x; p.ldo = H;
    p.ss = scr.ss;
    EAGLE_TRY(run_gemm<T>(c, scr, p, s));
  }
  return run_block<T>(c, scr, r, kv, r.a_out, nullptr, s);
}

QueryDesc desc_of(eagle_ctx* c, int set) {
  QueryDesc d;
  const size_t* o = c->off.desc[set];
  d.tok = c->at<int32_t>(o[0]);
  d.src_row = c->at<int32_t>(o[1]);
  d.pos = c->at<int32_t>(o[2]);
  d.dest = c->at<int32_t>(o[3]);
  d.plen = c->at<int32_t>(o[4]);
  d.mask = c->at<uint64_t>(o[5]);
  d.node = c->at<int32_t>(o[6]);
  return d;
}

TreeState tree_state(eagle_ctx* c) {
  TreeState t;
  const Offsets& f = c->off;
  t.c_token = c->at<int32_t>(f.c_token);
  t.c_parent = c->at<int32_t>(f.c_parent);
  t.c_slot = c->at<int32_t>(f.c_slot);
  t.c_row = c->at<int32_t>(f.c_row);
  t.c_score = c->at<float>(f.c_score);
  t.c_mask = c->at<uint64_t>(f.c_mask);
  t.c_depth = c->at<int32_t>(f.c_depth);
  t.n_cand = c->at<int32_t>(f.n_cand);
  t.p_root = c->at<int32_t>(f.p_root);
  t.len_out = c->at<int32_t>(f.len_out);
  t.ncand_max = f.ncand;
  return t;
}

template <typename T>
eagle_status draft_tree_impl(eagle_ctx* c, int batch, const void* seed_src,
                             const int32_t* seed_token, const int32_t* seed_len,
                             const eagle_kv* kv, const eagle_tree* out,
                             hipStream_t s, const SampleSpec* sample = nullptr) {
  const eagle_config& cf = c->cfg;
  const Offsets& f = c->off;
  const int K = cf.topk, D = cf.depth, N = cf.budget;
  SeedParams sp;
  sp.batch = batch; sp.s_max = cf.max_seed; sp.K = K; sp.D = D; sp.cap = kv->cap;
  sp.seed_token = seed_token; sp.seed_len = seed_len; sp.len_in = kv->len_in;
  sp.len_out = kv->len_out; sp.q = desc_of(c, 0);
  sp.sbase = c->at<int32_t>(f.sbase); sp.ts = tree_state(c); sp.status = c->status();
  {
    const int pi = prof_begin(c, PC_TREE, 0.0, 0.0, s);
    if (launch_seed_setup(sp, s) != hipSuccess) return EAGLE_EHIP;
    prof_end(c, pi, s);
  }

  const int passes = (D == 0 || N == 0) ? 1 : D;
  for (int d = 1; d <= passes; ++d) {
    const int rps = d == 1 ? cf.max_seed : K;
    QueryDesc cur = desc_of(c, (d - 1) & 1), nxt = desc_of(c, d & 1);
    Rows r;
    r.batch = batch; r.rps = rps;
    if (d == 1) {
      r.src = seed_src; r.src_row = cur.src_row; r.src_rows = batch * cf.max_seed;
    } else {
      r.src = c->at<char>((d - 1) % 2 ? f.a1 : f.a0);
      r.src_row = cur.src_row; r.src_rows = f.Rpad;
    }
    r.tok = cur.tok; r.pos = cur.pos; r.dest = cur.dest; r.plen = cur.plen;
    r.sbase = c->at<int32_t>(f.sbase); r.mask = cur.mask;
    r.a_out = c->at<char>(d % 2 ? f.a1 : f.a0);
    r.topk_id = c->at<int32_t>(f.tk_id); r.topk_val = c->at<float>(f.tk_val);
    r.lse = c->at<float>(f.lse);
    r.node = cur.node; r.pass = d; r.sample = sample;
    eagle_status st = run_layer<T>(c, r, kv, s);
    if (st != EAGLE_OK) return st;
    GrowParams g;
    g.batch = batch; g.K = K; g.D = (D == 0 || N == 0) ? 0 : D; g.N = N;
    g.pass = (D == 0 || N == 0) ? 1 : d;
    g.rows_per_seq = rps; g.s_max = cf.max_seed;
    g.topk_id = r.topk_id; g.topk_val = r.topk_val; g.lse = r.lse;
    g.cur = cur; g.nxt = nxt; g.ts = tree_state(c);
    g.seed_token = seed_token; g.seed_len = seed_len; g.d2t = c->w.d2t;
    g.sampled = sample != nullptr;
    g.t_token = out->token; g.t_parent = out->parent; g.t_depth = out->depth;
    g.t_pos = out->position; g.t_slot = out->kv_slot; g.t_first = out->first_child;
    g.t_nchild = out->n_child; g.t_score = out->score; g.t_mask = out->mask;
    g.t_n = out->n_nodes; g.mask_words = (N + 1 + 63) / 64;
    const int pi = prof_begin(c, PC_TREE, 0.0, 0.0, s);
    if (launch_grow(g, s) != hipSuccess) return EAGLE_EHIP;
    prof_end(c, pi, s);
  }
  return EAGLE_OK;
}

// Workspace of the target tree layer for `batch` sequences of budget + 1
// flattened rows: the block's activation buffers, split-K partials and
// counters, the packed A of the dense path, attention partials and the
// per-row descriptors.
struct TargetLayout {
  size_t x, h, a, o, t, ss, q, part, cnt, apack, at_o, at_ml, tok, pos, dest, plen, mask,
      sbase, total;
  int R, n1, max_split, apack_rows, ncnt;
  int64_t part_elems;
};

TargetLayout target_layout(const eagle_config& c, int batch) {
  TargetLayout f;
  Layout L;
  const int es = esize(c);
  const int H = c.hidden, F = c.ffn, V = c.vocab;
  const int qd = c.n_q_heads * c.head_dim, kd = c.n_kv_heads * c.head_dim;
  f.n1 = c.budget + 1;
  f.R = batch * f.n1;
  const size_t R = static_cast<size_t>((f.R + 63) / 64 * 64);
  f.x = L.take(R * H * 4);
  f.h = L.take(R * H * 4);
  f.a = L.take(R * H * 4);
  f.o = L.take(R * qd * 4);
  f.t = L.take(R * F * 4);
  f.ss = L.take(R * (H / 16) * 4);
  f.q = L.take(R * qd * es);
  const int maxN = std::max(std::max(V, 2 * F), std::max(H, qd + 2 * kd));
  f.part_elems = static_cast<int64_t>(16) * std::min<int64_t>(R, 32) * maxN;
  f.part = L.take(static_cast<size_t>(f.part_elems) * 4);
  f.ncnt = static_cast<int>((R / 16 + 1) * (maxN / 64 + 1));
  f.cnt = L.take(static_cast<size_t>(f.ncnt) * 4);
  f.apack_rows = (c.dtype == EAGLE_BF16 && f.R > 64) ? static_cast<int>(R) : 0;
  const int kmax = std::max(std::max(H, qd), F);
  f.apack = L.take(static_cast<size_t>(f.apack_rows) * ((kmax + 127) / 128 * 128) * 4);
  // attention partials: as many splits as the draft passes use, within
  // about 64 MB
  const int G = c.n_q_heads / c.n_kv_heads;
  const double per_split = static_cast<double>(batch) * c.n_kv_heads * f.n1 * G *
                           (c.head_dim + 2) * 4.0;
  const int cap_split = static_cast<int>(std::max(1.0, (64.0 * (1 << 20)) / per_split - 1.0));
  f.max_split = std::max(1, std::min(attn_max_split(batch, c.n_kv_heads), cap_split));
  const size_t bk = static_cast<size_t>(batch) * c.n_kv_heads * (f.max_split + 1) * f.n1 * G;
  f.at_o = L.take(bk * c.head_dim * 4);
  f.at_ml = L.take(bk * 2 * 4);
  f.tok = L.take(R * 4);
  f.pos = L.take(R * 4);
  f.dest = L.take(R * 4);
  f.plen = L.take(R * 4);
  f.mask = L.take(R * 8);
  f.sbase = L.take(static_cast<size_t>(batch) * 4);
  f.total = L.total;
  return f;
}

template <typename T>
eagle_status target_layer_impl(eagle_ctx* c, int batch, const eagle_tree* tree,
                               const eagle_kv* kv, char* ws, float* hidden_out,
                               float* logits_out, hipStream_t s) {
  const eagle_config& cf = c->cfg;
  const TargetLayout f = target_layout(cf, batch);
  auto at = [&](size_t o) { return ws + o; };
  EAGLE_TRY(launch_fill_i32(reinterpret_cast<int32_t*>(at(f.cnt)), 0, f.ncnt, s));
  TargetRowsParams tp;
  tp.batch = batch; tp.n1 = f.n1; tp.cap = kv->cap; tp.mask_words = (f.n1 + 63) / 64;
  tp.len_in = kv->len_in; tp.token = tree->token; tp.position = tree->position;
  tp.mask = reinterpret_cast<const uint64_t*>(tree->mask); tp.n_nodes = tree->n_nodes;
  tp.tok = reinterpret_cast<int32_t*>(at(f.tok)); tp.pos = reinterpret_cast<int32_t*>(at(f.pos));
  tp.dest = reinterpret_cast<int32_t*>(at(f.dest));
  tp.plen = reinterpret_cast<int32_t*>(at(f.plen));
  tp.rmask = reinterpret_cast<uint64_t*>(at(f.mask));
  tp.sbase = reinterpret_cast<int32_t*>(at(f.sbase)); tp.status = c->status();
  EAGLE_TRY(launch_target_rows(tp, s));
  EAGLE_TRY(launch_embed_rows<T>(static_cast<const T*>(c->w.embed), tvocab(cf), tp.tok, f.R,
                                 cf.hidden, reinterpret_cast<float*>(at(f.x)),
                                 reinterpret_cast<float*>(at(f.ss)), s));
  Scratch scr;
  scr.x = at(f.x); scr.h = at(f.h); scr.o = at(f.o); scr.t = at(f.t); scr.q = at(f.q);
  scr.ss = reinterpret_cast<float*>(at(f.ss));
  scr.part = reinterpret_cast<float*>(at(f.part)); scr.part_elems = f.part_elems;
  scr.cnt = reinterpret_cast<int*>(at(f.cnt));
  scr.apack = f.apack_rows > 0 ? at(f.apack) : nullptr; scr.apack_rows = f.apack_rows;
  scr.at_o = reinterpret_cast<float*>(at(f.at_o));
  scr.at_ml = reinterpret_cast<float*>(at(f.at_ml)); scr.max_split = f.max_split;
  Rows r;
  r.batch = batch; r.rps = f.n1;
  r.tok = tp.tok; r.pos = tp.pos; r.dest = tp.dest; r.plen = tp.plen;
  r.sbase = tp.sbase; r.mask = tp.rmask;
  void* a_out = hidden_out != nullptr ? static_cast<void*>(hidden_out) : at(f.a);
  return run_block<T>(c, scr, r, kv, a_out, logits_out, s);
}

bool null_tree(const eagle_tree* t) {
  return t == nullptr || !t->token || !t->parent || !t->depth || !t->position ||
         !t->kv_slot || !t->first_child || !t->n_child || !t->score || !t->mask ||
         !t->n_nodes;
}

// A draft KV cache holds whole 16-byte runs of keys (cap a multiple of 8)
// and at least one 32-key attention step.
bool bad_draft_cap(int32_t cap) { return cap < 32 || cap % 8 != 0; }

}  // namespace

extern "C" {

size_t eagle_workspace_bytes(const eagle_config* cfg) {
  if (check_config(cfg) != EAGLE_OK) return 0;
  return make_layout(*cfg).total;
}

eagle_status eagle_create(const eagle_config* cfg, const eagle_weights* w,
                          void* workspace, size_t ws_bytes, hipStream_t stream,
                          eagle_ctx** out) {
  if (out == nullptr || w == nullptr || workspace == nullptr) return EAGLE_EINVAL;
  *out = nullptr;
  eagle_status st = check_config(cfg);
  if (st != EAGLE_OK) return st;
  const void* ptrs[] = {w->w_fuse, w->w_in, w->embed, w->wq, w->wk, w->wv, w->wo,
                        w->w_gate, w->w_up, w->w_down, w->w_lm, w->g_attn,
                        w->g_mlp, w->g_final};
  for (const void* p : ptrs)
    if (p == nullptr) return EAGLE_EINVAL;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return EAGLE_EINVAL;
  if ((w->d2t == nullptr) != (cfg->target_vocab == 0 || cfg->target_vocab == cfg->vocab))
    return EAGLE_EINVAL;
  if (w->d2t != nullptr) {
    // the map must be strictly increasing into [0, target_vocab)
    int32_t* h = static_cast<int32_t*>(malloc(sizeof(int32_t) * cfg->vocab));
    if (h == nullptr) return EAGLE_EINVAL;
    if (hipStreamSynchronize(stream) != hipSuccess ||
        hipMemcpy(h, w->d2t, sizeof(int32_t) * cfg->vocab, hipMemcpyDeviceToHost) != hipSuccess) {
      free(h);
      return EAGLE_EHIP;
    }
    bool ok = h[0] >= 0 && h[cfg->vocab - 1] < cfg->target_vocab;
    for (int i = 1; i < cfg->vocab && ok; ++i) ok = h[i] > h[i - 1];
    free(h);
    if (!ok) return EAGLE_EINVAL;
  }
  Offsets off = make_layout(*cfg);
  if (ws_bytes < off.total) return EAGLE_EWORKSPACE;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess) return EAGLE_EHIP;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return EAGLE_EHIP;
  eagle_ctx* c = new (std::nothrow) eagle_ctx;
  if (c == nullptr) return EAGLE_EINVAL;
  c->cfg = *cfg;
  c->w = *w;
  c->ws = static_cast<char*>(workspace);
  c->off = off;
  c->num_cus = cus;
  const int64_t n = static_cast<int64_t>((off.counters_end - off.counters_begin) / 4);
  if (launch_fill_i32(c->at<int32_t>(off.counters_begin), 0, n, stream) != hipSuccess) {
    delete c;
    return EAGLE_EHIP;
  }
  for (int id = 0; id < G_COUNT; ++id) {
    GemmParams p;
    gemm_shape(*cfg, w, id, p);
    const hipError_t e = cfg->dtype == EAGLE_BF16
                             ? launch_pack<uint16_t>(p, c->at<char>(off.pack[id]), stream)
                             : launch_pack<float>(p, c->at<char>(off.pack[id]), stream);
    if (e != hipSuccess) {
      delete c;
      return EAGLE_EHIP;
    }
  }
  *out = c;
  return EAGLE_OK;
}

void eagle_destroy(eagle_ctx* ctx) {
  if (ctx == nullptr) return;
  if (ctx->prof.created)
    for (int i = 0; i < 2 * Profiler::kPairs; ++i) (void)hipEventDestroy(ctx->prof.ev[i]);
  delete ctx;
}

const char* eagle_status_str(eagle_status s) {
  switch (s) {
    case EAGLE_OK: return "ok";
    case EAGLE_EINVAL: return "invalid argument";
    case EAGLE_EUNSUPPORTED: return "unsupported shape";
    case EAGLE_EHIP: return "HIP launch or copy failed";
    case EAGLE_ECAPACITY: return "draft KV cache capacity exceeded";
    case EAGLE_ENONFINITE: return "non-finite target logits";
    case EAGLE_EWORKSPACE: return "workspace too small";
  }
  return "unknown status";
}

eagle_status eagle_get_device_status(eagle_ctx* ctx, int32_t* host_status,
                                     hipStream_t stream) {
  if (ctx == nullptr || host_status == nullptr) return EAGLE_EINVAL;
  if (hipStreamSynchronize(stream) != hipSuccess) return EAGLE_EHIP;
  if (hipMemcpy(host_status, ctx->status(), sizeof(int32_t), hipMemcpyDeviceToHost) !=
      hipSuccess)
    return EAGLE_EHIP;
  if (launch_fill_i32(ctx->status(), 0, 1, stream) != hipSuccess) return EAGLE_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return EAGLE_EHIP;
  return EAGLE_OK;
}

eagle_status eagle_fuse_features(eagle_ctx* ctx, int32_t rows, const void* low,
                                 const void* mid, const void* high, void* g_out,
                                 hipStream_t stream) {
  if (ctx == nullptr) return EAGLE_EINVAL;
  if (rows < 0 || rows > 65536) return EAGLE_EINVAL;
  if (rows == 0) return EAGLE_OK;
  if (!low || !mid || !high || !g_out) return EAGLE_EINVAL;
  const int H = ctx->cfg.hidden;
  const int es = esize(ctx->cfg);
  const int step = ctx->off.Rpad;
  for (int r0 = 0; r0 < rows; r0 += step) {
    const int m = std::min(step, rows - r0);
    GemmParams p;
    ctx->shape(G_FUSE, p);
    p.M = m; p.nseg = 3;
    const void* src[3] = {low, mid, high};
    for (int i = 0; i < 3; ++i) {
      p.seg[i].base = static_cast<const char*>(src[i]) + static_cast<size_t>(r0) * H * es;
      p.seg[i].ld = H;
      p.seg[i].width = H;
      p.seg[i].f32 = 0;
    }
    p.epi = EPI_STORE;
    p.out = static_cast<float*>(g_out) + static_cast<size_t>(r0) * H;
    p.ldo = H;
    const Scratch scr = ctx_scratch(ctx);
    hipError_t e = ctx->cfg.dtype == EAGLE_BF16
                       ? run_gemm<uint16_t>(ctx, scr, p, stream, PC_FUSE)
                       : run_gemm<float>(ctx, scr, p, stream, PC_FUSE);
    if (e != hipSuccess) return EAGLE_EHIP;
  }
  return EAGLE_OK;
}

eagle_status eagle_draft_step(eagle_ctx* ctx, int32_t batch, int32_t rows_per_seq,
                              const void* src, const int32_t* token,
                              const int32_t* position, const int32_t* dest,
                              const int32_t* prefix_len, const int32_t* scratch_base,
                              const uint64_t* scratch_mask, const eagle_kv* kv,
                              void* a_out, int32_t* topk_id, float* topk_logit,
                              float* lse, hipStream_t stream) {
  if (ctx == nullptr || kv == nullptr) return EAGLE_EINVAL;
  const eagle_config& cf = ctx->cfg;
  if (batch < 1 || batch > cf.max_batch || rows_per_seq < 1 ||
      rows_per_seq > std::max(cf.max_seed, cf.topk))
    return EAGLE_EINVAL;
  if (!src || !token || !position || !dest || !prefix_len || !scratch_base ||
      !scratch_mask || !kv->k || !kv->v || bad_draft_cap(kv->cap) || !a_out || !topk_id ||
      !topk_logit || !lse)
    return EAGLE_EINVAL;
  Rows r;
  r.batch = batch; r.rps = rows_per_seq; r.src = src; r.src_row = nullptr;
  r.src_rows = batch * rows_per_seq; r.tok = token; r.pos = position; r.dest = dest;
  r.plen = prefix_len; r.sbase = scratch_base; r.mask = scratch_mask; r.a_out = a_out;
  r.topk_id = topk_id; r.topk_val = topk_logit; r.lse = lse;
  return cf.dtype == EAGLE_BF16 ? run_layer<uint16_t>(ctx, r, kv, stream)
                                : run_layer<float>(ctx, r, kv, stream);
}

eagle_status eagle_draft_tree(eagle_ctx* ctx, int32_t batch, const void* seed_src,
                              const int32_t* seed_token, const int32_t* seed_len,
                              const eagle_kv* kv, const eagle_tree* out,
                              hipStream_t stream) {
  if (ctx == nullptr || kv == nullptr || null_tree(out)) return EAGLE_EINVAL;
  const eagle_config& cf = ctx->cfg;
  if (batch < 1 || batch > cf.max_batch) return EAGLE_EINVAL;
  if (!seed_src || !seed_token || !seed_len || !kv->k || !kv->v || !kv->len_in ||
      !kv->len_out || bad_draft_cap(kv->cap))
    return EAGLE_EINVAL;
  return cf.dtype == EAGLE_BF16
             ? draft_tree_impl<uint16_t>(ctx, batch, seed_src, seed_token, seed_len, kv,
                                         out, stream)
             : draft_tree_impl<float>(ctx, batch, seed_src, seed_token, seed_len, kv, out,
                                      stream);
}

eagle_status eagle_draft_tree_sampled(eagle_ctx* ctx, int32_t batch, const void* seed_src,
                                      const int32_t* seed_token, const int32_t* seed_len,
                                      const eagle_kv* kv, const eagle_tree* out,
                                      float temperature, uint64_t seed, uint64_t round,
                                      float* draft_logits, hipStream_t stream) {
  if (ctx == nullptr || kv == nullptr || null_tree(out) || draft_logits == nullptr)
    return EAGLE_EINVAL;
  const eagle_config& cf = ctx->cfg;
  if (batch < 1 || batch > cf.max_batch) return EAGLE_EINVAL;
  if (!seed_src || !seed_token || !seed_len || !kv->k || !kv->v || !kv->len_in ||
      !kv->len_out || bad_draft_cap(kv->cap))
    return EAGLE_EINVAL;
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return EAGLE_EINVAL;
  // every draw stays in the tree, in draw order; one vocabulary
  const int ncand = cf.depth > 0 ? cf.topk + (cf.depth - 1) * cf.topk * cf.topk : 0;
  if (cf.budget < ncand || ctx->w.d2t != nullptr || cf.depth < 1) return EAGLE_EUNSUPPORTED;
  const SampleSpec spec{draft_logits, temperature, seed, round};
  return cf.dtype == EAGLE_BF16
             ? draft_tree_impl<uint16_t>(ctx, batch, seed_src, seed_token, seed_len, kv,
                                         out, stream, &spec)
             : draft_tree_impl<float>(ctx, batch, seed_src, seed_token, seed_len, kv, out,
                                      stream, &spec);
}

}  // extern "C"

namespace {

// Row statistics of a verification: where they live.
struct VerifyScratch {
  float* row_max;
  double* row_sum;
  int32_t* row_arg;
  int32_t* row_bad;
  int* status;
};

eagle_status verify_core(const eagle_config& cf, const VerifyScratch& ws, eagle_ctx* prof,
                         int32_t batch, const eagle_tree* tree, const float* target_logits,
                         float temperature, const float* uniforms, uint64_t seed,
                         uint64_t round, int32_t commit_mode, const eagle_kv* kv_or_null,
                         int32_t* accept_len, int32_t* accepted_rows, int32_t* out_tokens,
                         int32_t* next_seed_rows, int32_t* next_seed_tokens,
                         int32_t* next_seed_len, hipStream_t stream,
                         const float* draft_rows = nullptr) {
  if (null_tree(tree)) return EAGLE_EINVAL;
  if (batch < 1 || batch > cf.max_batch) return EAGLE_EINVAL;
  if (!(temperature >= 0.f) || !std::isfinite(temperature)) return EAGLE_EINVAL;
  if (!target_logits || !accept_len || !accepted_rows || !out_tokens ||
      !next_seed_rows || !next_seed_tokens || !next_seed_len)
    return EAGLE_EINVAL;
  if (commit_mode != EAGLE_COMMIT_KEEP && commit_mode != EAGLE_COMMIT_RESEED)
    return EAGLE_EINVAL;
  // seed outputs hold max_seed slots per sequence: 2 for the keep policy,
  // D + 1 for a full reseed
  if (cf.max_seed < (commit_mode == EAGLE_COMMIT_RESEED ? cf.depth + 1 : 2))
    return EAGLE_EUNSUPPORTED;
  if (kv_or_null && (!kv_or_null->k || !kv_or_null->v || !kv_or_null->len_out ||
                     bad_draft_cap(kv_or_null->cap)))
    return EAGLE_EINVAL;
  VerifyParams p;
  p.batch = batch; p.N = cf.budget; p.K = cf.topk; p.D = cf.depth; p.V = tvocab(cf);
  p.T = temperature; p.logits = target_logits; p.uniforms = uniforms;
  p.seed = seed; p.round = round; p.commit_mode = commit_mode; p.S = cf.max_seed;
  p.t_token = tree->token; p.t_parent = tree->parent; p.t_depth = tree->depth;
  p.t_pos = tree->position; p.t_slot = tree->kv_slot; p.t_first = tree->first_child;
  p.t_nchild = tree->n_child; p.t_n = tree->n_nodes;
  p.row_max = ws.row_max; p.row_sum = ws.row_sum;
  p.row_arg = ws.row_arg; p.row_bad = ws.row_bad;
  p.accept_len = accept_len; p.accepted_rows = accepted_rows; p.out_tokens = out_tokens;
  p.seed_rows = next_seed_rows; p.seed_tokens = next_seed_tokens;
  p.seed_len = next_seed_len;
  p.kc = kv_or_null ? kv_or_null->k : nullptr;
  p.vc = kv_or_null ? kv_or_null->v : nullptr;
  p.cap = kv_or_null ? kv_or_null->cap : 0;
  p.kv_len = kv_or_null ? kv_or_null->len_out : nullptr;
  p.nkv = cf.n_kv_heads; p.hd = cf.head_dim; p.elem_bytes = esize(cf);
  p.status = ws.status;
  p.draft_rows = draft_rows;
  p.NE = 1 + std::max(cf.depth - 1, 0) * cf.topk;
  int pi = -1;
  if (prof != nullptr) {
    const double vbytes = static_cast<double>(batch) * (cf.budget + 1) * p.V * 4.0;
    pi = prof_begin(prof, PC_VERIFY, vbytes, 0.0, stream);
  }
  const hipError_t e = launch_verify(p, stream);
  if (prof != nullptr) prof_end(prof, pi, stream);
  return e == hipSuccess ? EAGLE_OK : EAGLE_EHIP;
}

eagle_status verify_impl(eagle_ctx* ctx, int32_t batch, const eagle_tree* tree,
                         const float* target_logits, float temperature,
                         const float* uniforms, uint64_t seed, uint64_t round,
                         int32_t commit_mode, const eagle_kv* kv_or_null,
                         int32_t* accept_len, int32_t* accepted_rows, int32_t* out_tokens,
                         int32_t* next_seed_rows, int32_t* next_seed_tokens,
                         int32_t* next_seed_len, hipStream_t stream,
                         const float* draft_rows = nullptr) {
  if (ctx == nullptr) return EAGLE_EINVAL;
  const Offsets& f = ctx->off;
  VerifyScratch ws;
  ws.row_max = ctx->at<float>(f.v_max);
  ws.row_sum = ctx->at<double>(f.v_sum);
  ws.row_arg = ctx->at<int32_t>(f.v_arg);
  ws.row_bad = ctx->at<int32_t>(f.v_bad);
  ws.status = ctx->status();
  return verify_core(ctx->cfg, ws, ctx, batch, tree, target_logits, temperature, uniforms,
                     seed, round, commit_mode, kv_or_null, accept_len, accepted_rows,
                     out_tokens, next_seed_rows, next_seed_tokens, next_seed_len, stream,
                     draft_rows);
}

// ---------------------------------------------------------------------------
// Verification without a context or workspace: the row statistics live in a
// fixed static device array, one copy per GPU, whose address is looked up
// once per device and kept.
// ---------------------------------------------------------------------------
constexpr int kNoAllocRows = 16384;   // batch * (budget + 1) at most
constexpr size_t kNaSum = 0;                                   // double [rows]
constexpr size_t kNaMax = kNaSum + 8 * kNoAllocRows;           // float  [rows]
constexpr size_t kNaArg = kNaMax + 4 * kNoAllocRows;           // int    [rows]
constexpr size_t kNaBad = kNaArg + 4 * kNoAllocRows;           // int    [rows]
constexpr size_t kNaStatus = kNaBad + 4 * kNoAllocRows;        // int
constexpr size_t kNoAllocBytes = kNaStatus + 256;
constexpr int kMaxDevices = 64;

}  // namespace

// the row statistics of eagle_verify_tree_noalloc (one copy per GPU)
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};

// Device address of this GPU's copy of `scratch`.  Host code must never pass
// the array's own name to a kernel: on the host it only stands in for it.
eagle_status scratch_on_current_device(unsigned char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return EAGLE_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return EAGLE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return EAGLE_EHIP;
    g_scratch_ptr[dev] = static_cast<unsigned char*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return EAGLE_OK;
}

}  // namespace

extern "C" {

eagle_status eagle_verify_tree(eagle_ctx* ctx, int32_t batch, const eagle_tree* tree,
                               const float* target_logits, float temperature,
                               uint64_t seed, uint64_t round, int32_t commit_mode,
                               const eagle_kv* kv_or_null, int32_t* accept_len,
                               int32_t* accepted_rows, int32_t* out_tokens,
                               int32_t* next_seed_rows, int32_t* next_seed_tokens,
                               int32_t* next_seed_len, hipStream_t stream) {
  return verify_impl(ctx, batch, tree, target_logits, temperature, nullptr, seed, round,
                     commit_mode, kv_or_null, accept_len, accepted_rows, out_tokens,
                     next_seed_rows, next_seed_tokens, next_seed_len, stream);
}

eagle_status eagle_verify_tree_sampled(eagle_ctx* ctx, int32_t batch, const eagle_tree* tree,
                                       const float* target_logits, const float* draft_logits,
                                       float temperature, uint64_t seed, uint64_t round,
                                       int32_t commit_mode, const eagle_kv* kv_or_null,
                                       int32_t* accept_len, int32_t* accepted_rows,
                                       int32_t* out_tokens, int32_t* next_seed_rows,
                                       int32_t* next_seed_tokens, int32_t* next_seed_len,
                                       hipStream_t stream) {
  if (ctx == nullptr || draft_logits == nullptr) return EAGLE_EINVAL;
  if (!(temperature > 0.f)) return EAGLE_EINVAL;
  if (ctx->w.d2t != nullptr) return EAGLE_EUNSUPPORTED;
  return verify_impl(ctx, batch, tree, target_logits, temperature, nullptr, seed, round,
                     commit_mode, kv_or_null, accept_len, accepted_rows, out_tokens,
                     next_seed_rows, next_seed_tokens, next_seed_len, stream, draft_logits);
}

eagle_status eagle_verify_tree_uniforms(eagle_ctx* ctx, int32_t batch, const eagle_tree* tree,
                                        const float* target_logits, float temperature,
                                        const float* uniforms, int32_t commit_mode,
                                        const eagle_kv* kv_or_null, int32_t* accept_len,
                                        int32_t* accepted_rows, int32_t* out_tokens,
                                        int32_t* next_seed_rows, int32_t* next_seed_tokens,
                                        int32_t* next_seed_len, hipStream_t stream) {
  if (temperature > 0.f && uniforms == nullptr) return EAGLE_EINVAL;
  return verify_impl(ctx, batch, tree, target_logits, temperature, uniforms, 0, 0,
                     commit_mode, kv_or_null, accept_len, accepted_rows, out_tokens,
                     next_seed_rows, next_seed_tokens, next_seed_len, stream);
}

eagle_status eagle_verify_tree_noalloc(const eagle_config* cfg, int32_t batch,
                                       const eagle_tree* tree, const float* target_logits,
                                       float temperature, uint64_t seed, uint64_t round,
                                       int32_t commit_mode, const eagle_kv* kv_or_null,
                                       int32_t* accept_len, int32_t* accepted_rows,
                                       int32_t* out_tokens, int32_t* next_seed_rows,
                                       int32_t* next_seed_tokens, int32_t* next_seed_len,
                                       hipStream_t stream) {
  const eagle_status st = check_config(cfg);
  if (st != EAGLE_OK) return st;
  if (batch < 1 || batch > cfg->max_batch) return EAGLE_EINVAL;
  if (static_cast<int64_t>(batch) * (cfg->budget + 1) > kNoAllocRows)
    return EAGLE_EUNSUPPORTED;
  unsigned char* base = nullptr;
  const eagle_status sp = scratch_on_current_device(&base);
  if (sp != EAGLE_OK) return sp;
  VerifyScratch ws;
  ws.row_sum = reinterpret_cast<double*>(base + kNaSum);
  ws.row_max = reinterpret_cast<float*>(base + kNaMax);
  ws.row_arg = reinterpret_cast<int32_t*>(base + kNaArg);
  ws.row_bad = reinterpret_cast<int32_t*>(base + kNaBad);
  ws.status = reinterpret_cast<int*>(base + kNaStatus);
  // the status word collects error bits with atomics: start it from zero
  if (launch_fill_i32(ws.status, 0, 1, stream) != hipSuccess) return EAGLE_EHIP;
  return verify_core(*cfg, ws, nullptr, batch, tree, target_logits, temperature, nullptr,
                     seed, round, commit_mode, kv_or_null, accept_len, accepted_rows,
                     out_tokens, next_seed_rows, next_seed_tokens, next_seed_len, stream);
}

size_t eagle_target_layer_workspace_bytes(const eagle_config* cfg, int32_t batch) {
  if (check_config(cfg) != EAGLE_OK || batch < 1 || batch > cfg->max_batch ||
      cfg->budget + 1 > 64)
    return 0;
  return target_layout(*cfg, batch).total;
}

eagle_status eagle_target_tree_layer(eagle_ctx* ctx, int32_t batch, const eagle_tree* tree,
                                     const eagle_kv* kv, void* workspace, size_t ws_bytes,
                                     float* hidden_out, float* logits_out,
                                     hipStream_t stream) {
  if (ctx == nullptr || tree == nullptr || kv == nullptr || workspace == nullptr ||
      logits_out == nullptr)
    return EAGLE_EINVAL;
  if (!tree->token || !tree->position || !tree->mask || !tree->n_nodes || !kv->k || !kv->v ||
      !kv->len_in || kv->cap <= 0)
    return EAGLE_EINVAL;
  const eagle_config& cf = ctx->cfg;
  if (batch < 1 || batch > cf.max_batch) return EAGLE_EINVAL;
  if (cf.budget + 1 > 64) return EAGLE_EUNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return EAGLE_EINVAL;
  if (ws_bytes < target_layout(cf, batch).total) return EAGLE_EWORKSPACE;
  char* ws = static_cast<char*>(workspace);
  return cf.dtype == EAGLE_BF16
             ? target_layer_impl<uint16_t>(ctx, batch, tree, kv, ws, hidden_out, logits_out, stream)
             : target_layer_impl<float>(ctx, batch, tree, kv, ws, hidden_out, logits_out, stream);
}

eagle_status eagle_draw_uniforms(uint64_t seed, uint64_t stream_id, uint64_t round,
                                 int32_t batch, int32_t rows, int32_t draws, float* out,
                                 hipStream_t stream) {
  if (batch < 0 || rows < 0 || draws < 0 || batch > 65535 || rows > 65535) return EAGLE_EINVAL;
  if (batch == 0 || rows == 0 || draws == 0) return EAGLE_OK;
  if (out == nullptr) return EAGLE_EINVAL;
  return launch_uniforms(seed, stream_id, round, batch, rows, draws, out, stream) == hipSuccess
             ? EAGLE_OK
             : EAGLE_EHIP;
}

eagle_status eagle_profile(eagle_ctx* ctx, int32_t on) {
  if (ctx == nullptr) return EAGLE_EINVAL;
  Profiler& p = ctx->prof;
  if (on && !p.created) {
    for (int i = 0; i < 2 * Profiler::kPairs; ++i)
      if (hipEventCreate(&p.ev[i]) != hipSuccess) return EAGLE_EHIP;
    p.created = true;
  }
  // 1 starts a new record, 2 resumes the current one, 0 stops (the record
  // stays for eagle_profile_read)
  if (on < 0 || on > 2) return EAGLE_EINVAL;
  if (on == 1) {
    p.used = 0;
    p.overflow = false;
  }
  p.on = on != 0;
  return EAGLE_OK;
}

eagle_status eagle_profile_read(eagle_ctx* ctx, int32_t n_classes, float* ms,
                                int32_t* launches, double* bytes, double* flops) {
  if (ctx == nullptr || ms == nullptr || launches == nullptr || bytes == nullptr ||
      flops == nullptr || n_classes < 1)
    return EAGLE_EINVAL;
  Profiler& p = ctx->prof;
  for (int k = 0; k < n_classes; ++k) {
    ms[k] = 0.f;
    launches[k] = 0;
    bytes[k] = 0.0;
    flops[k] = 0.0;
  }
  if (p.used > 0 && hipEventSynchronize(p.ev[2 * p.used - 1]) != hipSuccess)
    return EAGLE_EHIP;
  for (int i = 0; i < p.used; ++i) {
    const int k = p.cls[i];
    if (k >= n_classes) continue;
    float t = 0.f;
    if (hipEventElapsedTime(&t, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess) return EAGLE_EHIP;
    ms[k] += t;
    launches[k] += 1;
    bytes[k] += p.bytes[i];
    flops[k] += p.flops[i];
  }
  const bool ovf = p.overflow;
  p.used = 0;
  p.overflow = false;
  return ovf ? EAGLE_EWORKSPACE : EAGLE_OK;
}

}  // extern "C"
