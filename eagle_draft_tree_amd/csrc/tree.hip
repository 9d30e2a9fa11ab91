// LM-head top-k merge, EAGLE-2 tree growth / rerank / flatten, and tree
// verification with the accepted-path commit.  These kernels move little
// data; they are latency kernels built from wave shuffles and LDS counting.
#include "common.hpp"
#include "kernels.hpp"

namespace eagle {

constexpr int kMaxCand = 16 + 7 * 256;  // >= K + (D-1) K^2 when (D-1)K <= 64
constexpr int kBonusDraw = 63;          // draw index of a row's residual draw
constexpr int kMaxPath = 72;            // >= D + 1 when (D-1)K <= 64

// ============================================================================
// merge: per row, top-k over the LM-head tiles' candidates + log-sum-exp
// ============================================================================
// The LM head left the row's logits and, per 64-column tile, (max, sum of
// exp).  The row's top-k is found from few tiles: with theta the k-th
// largest tile maximum, k tiles hold an element >= theta, so every element of
// the row's top-k is >= theta and sits in a tile whose maximum is >= theta.
// Those tiles' elements >= theta (a few dozen) are sorted by one wave.  If
// more than kSurv survive (massive ties), the whole row is scanned instead.
constexpr int kSurv = 64;

// Thread-local sorted top-K of this thread's share of the row's logits, then
// a merge across the workgroup; lane i of wave 0 ends with the i-th best.
__device__ void merge_scan_row(const MergeParams& p, int row, float* sv, int* si,
                               float& v_out, int& id_out) {
  const int K = p.topk;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const float* lg = p.logits + static_cast<int64_t>(row) * p.ntile * 64;
  float lv[kMaxTopK];
  int li[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
  for (int id = threadIdx.x; id < p.V; id += 256) {
    float v = lg[id];
    if (v != v) v = -INFINITY;
#pragma unroll
    for (int j = kMaxTopK - 1; j >= 0; --j) {
      if (j >= K) continue;
      if (better(v, id, lv[j], li[j])) {
        if (j > 0 && better(v, id, lv[j - 1], li[j - 1])) {
          lv[j] = lv[j - 1];
          li[j] = li[j - 1];
        } else {
          lv[j] = v;
          li[j] = id;
        }
      }
    }
  }
  for (int r = 0; r < K; ++r) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = shfl_xor(bv, m);
      const int oi = shfl_xor(bi, m);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lv[0] == bv && li[0] == bi) {
#pragma unroll
      for (int j = 0; j < kMaxTopK - 1; ++j) { lv[j] = lv[j + 1]; li[j] = li[j + 1]; }
      lv[kMaxTopK - 1] = -INFINITY;
      li[kMaxTopK - 1] = 0x7fffffff;
    }
    if (lane == 0) { sv[wave * K + r] = bv; si[wave * K + r] = bi; }
  }
  __syncthreads();
  v_out = lane < 4 * K ? sv[lane] : -INFINITY;
  id_out = lane < 4 * K ? si[lane] : 0x7fffffff;
}

__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  __shared__ float sv[kSurv];
  __shared__ int si[kSurv];
  __shared__ float red_a[4], red_b[4];
  __shared__ int nsurv, ntl;
  __shared__ int stile[kSurv];
  const int row = blockIdx.x;
  if (p.tok[row] < 0) return;
  const int K = p.topk;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int64_t base = static_cast<int64_t>(row) * p.ntile;
  if (threadIdx.x == 0) { nsurv = 0; ntl = 0; }

  // ---- tile statistics: log-sum-exp, and this thread's tile maxima.  All
  // of a thread's (max, sum) pairs are loaded before any is used (indices
  // clamped into the row), so they cost one memory round trip ----
  constexpr int kTPT = 8;   // tile maxima per thread in registers
  const bool fast = p.ntile <= 256 * kTPT;
  float hmax[kTPT];
  float M = -INFINITY, S = 0.f;
  {
    float2 st[kTPT];
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      const int t = min(static_cast<int>(threadIdx.x) + 256 * u, p.ntile - 1);
      st[u] = *reinterpret_cast<const float2*>(p.stat + (base + t) * 2);
    }
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      const int t = threadIdx.x + 256 * u;
      const float mx = t < p.ntile ? st[u].x : -INFINITY, se = st[u].y;
      hmax[u] = mx;
      if (mx == -INFINITY) continue;
      const float nm = fmaxf(M, mx);
      S = (M == -INFINITY ? 0.f : S * expf(M - nm)) + se * expf(mx - nm);
      M = nm;
    }
  }
  for (int t = threadIdx.x + 256 * kTPT; t < p.ntile; t += 256) {
    const float mx = p.stat[(base + t) * 2], se = p.stat[(base + t) * 2 + 1];
    if (mx == -INFINITY) continue;
    const float nm = fmaxf(M, mx);
    S = (M == -INFINITY ? 0.f : S * expf(M - nm)) + se * expf(mx - nm);
    M = nm;
  }
  {
    const float wm = wave_max(M);
    float ws = wave_sum(M == -INFINITY ? 0.f : S * expf(M - wm));
    if (wm == -INFINITY) ws = 0.f;
    if (lane == 0) { red_a[wave] = wm; red_b[wave] = ws; }
  }
  // ---- theta: the K-th largest tile maximum.  Each wave takes its K
  // largest (K rounds: the wave maximum, given up by the lowest lane holding
  // it), then one wave sorts the four lists ----
  unsigned taken = 0;
  for (int r = 0; r < K; ++r) {
    float mine = -INFINITY;
#pragma unroll
    for (int u = 0; u < kTPT; ++u)
      if (!((taken >> u) & 1u)) mine = fmaxf(mine, hmax[u]);
    const float m1 = wave_max(mine);
    const uint64_t own = __ballot(mine == m1);
    if (lane == __ffsll(static_cast<long long>(own)) - 1) {
      bool done = false;
#pragma unroll
      for (int u = 0; u < kTPT; ++u)
        if (!done && !((taken >> u) & 1u) && hmax[u] == m1) {
          taken |= 1u << u;
          done = true;
        }
    }
    if (lane == 0) sv[wave * K + r] = m1;
  }
  __syncthreads();
  float theta;
  {
    float v = lane < 4 * K ? sv[lane] : -INFINITY;
    int id = lane;
    wave_sort_desc(v, id);
    theta = __shfl(v, K - 1, 64);
  }
  if (!fast) theta = -INFINITY;
  __syncthreads();
  // ---- survivors: candidates >= theta of tiles whose maximum is >= theta.
  // The surviving tiles are listed in LDS first (from the maxima still in
  // registers), then one thread per (tile, rank) reads one candidate, so all
  // of them arrive in one memory round trip ----
  if (fast && theta != -INFINITY) {
#pragma unroll
    for (int u = 0; u < kTPT; ++u) {
      const int t = threadIdx.x + 256 * u;
      if (t < p.ntile && hmax[u] >= theta) {
        const int slot = atomicAdd(&ntl, 1);
        if (slot < kSurv) stile[slot] = t;
      }
    }
  }
  __syncthreads();
  const int nt = ntl;
  if (fast && theta != -INFINITY && nt <= kSurv) {
    // the listed tiles' elements, 16 per thread, all requested before any
    // is tested (indices clamped into the list)
    const float* lg = p.logits + static_cast<int64_t>(row) * p.ntile * 64;
    constexpr int kPer = kSurv * 64 / 256;
    float cv[kPer];
    int ci[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = min(static_cast<int>(threadIdx.x) + 256 * k, nt * 64 - 1);
      ci[k] = stile[idx >> 6] * 64 + (idx & 63);
      cv[k] = lg[min(ci[k], p.V - 1)];
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      float v = cv[k];
      if (v != v) v = -INFINITY;
      if (static_cast<int>(threadIdx.x) + 256 * k < nt * 64 && ci[k] < p.V && v >= theta) {
        const int slot = atomicAdd(&nsurv, 1);
        if (slot < kSurv) {
          sv[slot] = v;
          si[slot] = ci[k];
        }
      }
    }
  } else if (threadIdx.x == 0) {
    nsurv = kSurv + 1;   // too many tied tiles: scan the whole row
  }
  __syncthreads();
  const int n = nsurv;
  float v;
  int id;
  if (n <= kSurv && theta != -INFINITY) {
    v = lane < n ? sv[lane] : -INFINITY;
    id = lane < n ? si[lane] : 0x7fffffff;
  } else {
    __syncthreads();
    merge_scan_row(p, row, sv, si, v, id);
  }
  if (wave == 0) {
    wave_sort_desc(v, id);
    if (lane < K) {
      p.out_id[static_cast<int64_t>(row) * K + lane] = id;
      p.out_val[static_cast<int64_t>(row) * K + lane] = v;
    }
    if (lane == 0) {
      float Mt = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) Mt = fmaxf(Mt, red_a[w]);
      float St = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        if (red_a[w] != -INFINITY) St += red_b[w] * expf(red_a[w] - Mt);
      p.out_lse[row] = Mt + logf(St);
    }
  }
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(p.rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ============================================================================
// pass-1 query rows from the seed rows
// ============================================================================
__global__ void seed_setup_kernel(SeedParams p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.batch) return;
  const int len_in = p.len_in[b];
  const int sl = p.seed_len[b];
  const int scratch = p.D > 0 ? (p.D - 1) * p.K : 0;
  bool ok = sl >= 1 && sl <= p.s_max && len_in >= 0 &&
            static_cast<int64_t>(len_in) + sl + scratch <= p.cap;
  if (!ok && p.status != nullptr) atomicOr(p.status, 1 << 4);
  const int len_out = ok ? len_in + sl : max(len_in, 0);
  p.len_out[b] = len_out;
  p.ts.len_out[b] = len_out;
  p.ts.p_root[b] = ok ? len_out - 1 : -1;
  p.ts.n_cand[b] = 0;
  p.sbase[b] = len_out;
  for (int i = 0; i < p.s_max; ++i) {
    const int r = b * p.s_max + i;
    const int tok = (ok && i < sl) ? p.seed_token[r] : -1;
    p.q.tok[r] = tok;
    p.q.src_row[r] = r;
    p.q.pos[r] = len_in + i;
    p.q.dest[r] = len_in + i;
    p.q.plen[r] = len_in + i + 1;
    p.q.mask[r] = 0ull;
    p.q.node[r] = -1;
  }
}

hipError_t launch_seed_setup(const SeedParams& p, hipStream_t s) {
  hipLaunchKernelGGL(seed_setup_kernel, dim3((p.batch + 63) / 64), dim3(64), 0, s, p);
  return hipGetLastError();
}

// ============================================================================
// tree growth after one draft pass; final rerank + flatten after the last
// ============================================================================
__device__ __forceinline__ bool cand_better(float sa, int ia, float sb, int ib) {
  // (-value, depth, node id): node ids grow with depth, so id breaks both ties
  return sa > sb || (sa == sb && ia < ib);
}

__global__ __launch_bounds__(256) void grow_kernel(GrowParams p) {
  __shared__ float s_score[kMaxCand];
  __shared__ int s_flag[kMaxCand];
  __shared__ int s_scan[256];
  __shared__ int s_prow[128], s_first[128], s_nch[128];
  __shared__ int s_ntok[kMaxTopK * kMaxTopK], s_nrow[kMaxTopK * kMaxTopK];
  __shared__ uint64_t s_nmask[kMaxTopK * kMaxTopK];
  const int b = blockIdx.x;
  const int K = p.K, D = p.D, N = p.N;
  const int tid = threadIdx.x;
  const TreeState& ts = p.ts;
  const int64_t cb = static_cast<int64_t>(b) * ts.ncand_max;
  const int p_root = ts.p_root[b];
  const int len_out = ts.len_out[b];
  const bool last = p.pass >= D;
  const int rows1 = p.N + 1;
  const int W = p.mask_words;

  auto write_root_only = [&](bool valid) {
    for (int r = tid; r < rows1; r += 256) {
      const int64_t o = static_cast<int64_t>(b) * rows1 + r;
      const bool root = r == 0 && valid;
      p.t_token[o] = root ? p.seed_token[b * p.s_max + p.seed_len[b] - 1] : -1;
      p.t_parent[o] = -1;
      p.t_depth[o] = root ? 0 : -1;
      p.t_pos[o] = root ? p_root : -1;
      p.t_slot[o] = -1;
      p.t_first[o] = -1;
      p.t_nchild[o] = 0;
      p.t_score[o] = 0.f;
      for (int w = 0; w < W; ++w) p.t_mask[o * W + w] = (root && w == 0) ? 1ull : 0ull;
    }
    if (tid == 0) p.t_n[b] = valid ? 0 : -1;
  };

  if (p_root < 0) {  // sequence rejected at seed time
    if (!last) {
      for (int r = tid; r < K; r += 256) p.nxt.tok[b * K + r] = -1;
    } else {
      write_root_only(false);
    }
    return;
  }
  if (N == 0 || D == 0) {
    write_root_only(true);
    return;
  }

  // ---- create this pass's children ----
  const int first = ts.n_cand[b];
  const int nrows = p.pass == 1 ? 1 : K;
  const int nnew = nrows * K;
  if (tid < nnew) {
    const int rr = tid / K, cc = tid % K;
    const int row = p.pass == 1 ? b * p.s_max + p.seed_len[b] - 1 : b * K + rr;
    const int* ids = p.topk_id + static_cast<int64_t>(row) * K;
    const int my = ids[cc];
    // children are created by ascending token id, or in draw order when
    // they were sampled
    int rank = cc;
    if (!p.sampled) {
      rank = 0;
      for (int j = 0; j < K; ++j) rank += ids[j] < my;
    }
    const int node = first + rr * K + rank;
    const int parent = p.pass == 1 ? -1 : p.cur.node[row];
    const float ps = parent < 0 ? 0.f : ts.c_score[cb + parent];
    float lp = p.topk_val[static_cast<int64_t>(row) * K + cc] - p.lse[row];
    lp = fmaxf(lp, kLogEps);
    const int tok_out = p.d2t != nullptr ? p.d2t[my] : my;
    const uint64_t pmask = parent < 0 ? 0ull : ts.c_mask[cb + parent];
    ts.c_token[cb + node] = tok_out;
    ts.c_parent[cb + node] = parent;
    ts.c_depth[cb + node] = p.pass;
    ts.c_score[cb + node] = ps + lp;
    ts.c_slot[cb + node] = -1;
    ts.c_row[cb + node] = row;
    ts.c_mask[cb + node] = pmask;
    // the new layer also in LDS, for the expansion below (no reload)
    const int i = node - first;
    s_score[i] = ps + lp;
    s_ntok[i] = tok_out;
    s_nrow[i] = row;
    s_nmask[i] = pmask;
  }
  __threadfence_block();
  __syncthreads();
  const int ncand = first + nnew;
  if (tid == 0) ts.n_cand[b] = ncand;

  if (!last) {
    // ---- expand the K best of the new layer ----
    for (int i = tid; i < nnew; i += 256) {
      int rank = 0;
      const float si = s_score[i];
      for (int j = 0; j < nnew; ++j) rank += cand_better(s_score[j], j, si, i);
      s_flag[i] = rank < K;
    }
    __syncthreads();
    for (int i = tid; i < nnew; i += 256) {
      if (!s_flag[i]) continue;
      int r = 0;
      for (int j = 0; j < i; ++j) r += s_flag[j];
      const int node = first + i;
      const int slot = (p.pass - 1) * K + r;
      const uint64_t m = s_nmask[i] | (1ull << slot);
      ts.c_slot[cb + node] = slot;
      ts.c_mask[cb + node] = m;
      const int q = b * K + r;
      p.nxt.tok[q] = s_ntok[i];
      p.nxt.src_row[q] = s_nrow[i];
      p.nxt.pos[q] = p_root + p.pass;
      p.nxt.dest[q] = len_out + slot;
      p.nxt.plen[q] = len_out;
      p.nxt.mask[q] = m;
      p.nxt.node[q] = node;
    }
    return;
  }

  // ---- final: top-N of all candidates, flatten ----
  for (int i = tid; i < ncand; i += 256) s_score[i] = ts.c_score[cb + i];
  __syncthreads();
  for (int i = tid; i < ncand; i += 256) {
    int rank = 0;
    const float si = s_score[i];
    for (int j = 0; j < ncand; ++j) rank += cand_better(s_score[j], j, si, i);
    s_flag[i] = rank < N;
  }
  __syncthreads();
  // exclusive scan of the flags over contiguous chunks
  const int per = (ncand + 255) / 256;
  const int lo = tid * per, hi = min(ncand, lo + per);
  int cnt = 0;
  for (int i = lo; i < hi; ++i) cnt += s_flag[i];
  s_scan[tid] = cnt;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  int run = s_scan[tid] - cnt;
  for (int i = lo; i < hi; ++i) {
    if (s_flag[i]) {
      s_flag[i] = 1 + run;  // row of node i
      ++run;
    } else {
      s_flag[i] = 0;
    }
  }
  const int nsel = s_scan[255];
  for (int r = tid; r < 128; r += 256) { s_prow[r] = -1; s_first[r] = 0x7fffffff; s_nch[r] = 0; }
  __syncthreads();
  const int64_t ob = static_cast<int64_t>(b) * rows1;
  for (int i = tid; i < ncand; i += 256) {
    const int r = s_flag[i];
    if (r == 0) continue;
    const int par = ts.c_parent[cb + i];
    const int prow = par < 0 ? 0 : s_flag[par];
    const int dep = ts.c_depth[cb + i];
    s_prow[r] = prow;
    atomicMin(&s_first[prow], r);
    atomicAdd(&s_nch[prow], 1);
    p.t_token[ob + r] = ts.c_token[cb + i];
    p.t_parent[ob + r] = prow;
    p.t_depth[ob + r] = dep;
    p.t_pos[ob + r] = p_root + dep;
    p.t_slot[ob + r] = ts.c_slot[cb + i];
    p.t_score[ob + r] = s_score[i];
  }
  __syncthreads();
  for (int r = tid; r < rows1; r += 256) {
    const int64_t o = ob + r;
    if (r == 0) {
      p.t_token[o] = p.seed_token[b * p.s_max + p.seed_len[b] - 1];
      p.t_parent[o] = -1;
      p.t_depth[o] = 0;
      p.t_pos[o] = p_root;
      p.t_slot[o] = -1;
      p.t_score[o] = 0.f;
    } else if (r > nsel) {
      p.t_token[o] = -1;
      p.t_parent[o] = -1;
      p.t_depth[o] = -1;
      p.t_pos[o] = -1;
      p.t_slot[o] = -1;
      p.t_score[o] = 0.f;
    }
    const bool live = r <= nsel;
    p.t_first[o] = (live && s_nch[r] > 0) ? s_first[r] : -1;
    p.t_nchild[o] = live ? s_nch[r] : 0;
    uint64_t bits[2] = {0ull, 0ull};
    if (live) {
      int a = r;
      while (a >= 0) {
        bits[a >> 6] |= 1ull << (a & 63);
        a = a == 0 ? -1 : s_prow[a];
      }
    }
    for (int w = 0; w < W; ++w) p.t_mask[o * W + w] = bits[w];
  }
  if (tid == 0) p.t_n[b] = nsel;
}

hipError_t launch_grow(const GrowParams& p, hipStream_t s) {
  hipLaunchKernelGGL(grow_kernel, dim3(p.batch), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ============================================================================
// sampled children
// ============================================================================
// Draft-logit row of each query row of a pass: the root's row (the last seed
// row of a sequence) in pass 1, 1 + scratch slot for a drafted node.
__global__ void slot_rows_kernel(SampleParams p) {
  const int m = blockIdx.x * blockDim.x + threadIdx.x;
  if (m >= p.rows) return;
  const int b = m / p.rows_per_seq, i = m - b * p.rows_per_seq;
  int orow = -1;
  if (p.tok[m] >= 0) {
    if (p.pass == 1) {
      if (i + 1 == p.rows_per_seq || p.tok[m + 1] < 0) orow = b * p.NE;
    } else {
      const int slot = p.dest[m] - p.plen[m];
      if (slot >= 0 && slot + 1 < p.NE) orow = b * p.NE + 1 + slot;
    }
  }
  p.out_row[m] = orow;
}

hipError_t launch_slot_rows(const SampleParams& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(slot_rows_kernel, dim3((p.rows + 255) / 256), dim3(256), 0, s, p);
  return hipGetLastError();
}

// Gumbel-top-k: the K largest logits[x] / T - log(-log u_x), best first,
// ties to the lower id, are K draws without replacement from
// softmax(logits / T) in draw order.  Each thread keeps a sorted top-K of
// its tokens; K rounds of a wave argmax and one sort over the four waves'
// lists give the row's.
__global__ __launch_bounds__(256) void sample_children_kernel(SampleParams p) {
  __shared__ float sv[4 * kMaxTopK];
  __shared__ int si[4 * kMaxTopK];
  __shared__ float red_m[4], red_s[4];
  const int m = blockIdx.x;
  const int orow = p.out_row[m];
  if (orow < 0) return;
  const int K = p.K;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const int b = m / p.rows_per_seq;
  const uint64_t key_row = p.pass == 1 ? 0ull : 1ull + static_cast<uint64_t>(p.node[m]);
  const float* lg = p.logits + static_cast<int64_t>(orow) * p.V;
  const float invT = 1.f / p.T;
  float lv[kMaxTopK];
  int li[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) { lv[j] = -INFINITY; li[j] = 0x7fffffff; }
  float mx = -INFINITY;
  for (int q4 = threadIdx.x; q4 * 4 < p.V; q4 += 256) {
    uint64_t w[4];
    philox4x64(static_cast<uint64_t>(q4), key_row, static_cast<uint64_t>(b), p.round, p.seed,
               kStreamDraft, w);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int x = q4 * 4 + k;
      if (x >= p.V) break;
      const float l = lg[x];
      mx = fmaxf(mx, l);
      const float u = (static_cast<float>(w[k] >> 40) + 0.5f) * 5.9604644775390625e-08f;
      const float key = l / p.T - logf(-logf(u));
#pragma unroll
      for (int j = kMaxTopK - 1; j >= 0; --j) {
        if (j >= K) continue;
        if (better(key, x, lv[j], li[j])) {
          if (j > 0 && better(key, x, lv[j - 1], li[j - 1])) {
            lv[j] = lv[j - 1];
            li[j] = li[j - 1];
          } else {
            lv[j] = key;
            li[j] = x;
          }
        }
      }
    }
  }
  // log-sum-exp of logits / T
  const float m_all = [&] {
    const float wm = wave_max(mx);
    if (lane == 0) red_m[wave] = wm;
    __syncthreads();
    return fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  }();
  float se = 0.f;
  for (int x = threadIdx.x; x < p.V; x += 256) se += expf((lg[x] - m_all) * invT);
  se = wave_sum(se);
  if (lane == 0) red_s[wave] = se;
  // the wave's K best, then all four waves' lists sorted by one wave
  for (int r = 0; r < K; ++r) {
    float bv = lv[0];
    int bi = li[0];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = shfl_xor(bv, o);
      const int oi = shfl_xor(bi, o);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (lv[0] == bv && li[0] == bi) {
#pragma unroll
      for (int j = 0; j < kMaxTopK - 1; ++j) { lv[j] = lv[j + 1]; li[j] = li[j + 1]; }
      lv[kMaxTopK - 1] = -INFINITY;
      li[kMaxTopK - 1] = 0x7fffffff;
    }
    if (lane == 0) { sv[wave * K + r] = bv; si[wave * K + r] = bi; }
  }
  __syncthreads();
  if (wave == 0) {
    float v = lane < 4 * K ? sv[lane] : -INFINITY;
    int id = lane < 4 * K ? si[lane] : 0x7fffffff;
    wave_sort_desc(v, id);
    if (lane < K) {
      const int x = id;
      p.topk_id[static_cast<int64_t>(m) * K + lane] = x;
      p.topk_val[static_cast<int64_t>(m) * K + lane] =
          (x >= 0 && x < p.V) ? lg[x] / p.T : -INFINITY;
    }
    if (lane == 0) {
      const float S = red_s[0] + red_s[1] + red_s[2] + red_s[3];
      p.lse[m] = m_all / p.T + logf(S);
    }
  }
}

hipError_t launch_sample_children(const SampleParams& p, hipStream_t s) {
  if (p.rows <= 0) return hipSuccess;
  if (p.K < 1 || p.K > kMaxTopK || p.T <= 0.f) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sample_children_kernel, dim3(p.rows), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ============================================================================
// verification
// ============================================================================
__device__ __forceinline__ float wexp(float l, float m, float T) {
  return expf((l - m) / T);
}

// Statistics of one target row (max, first index of the max, sum of
// exp((l - max) / T) in double, non-finite flag) by one workgroup of 1024
// threads.  When the rows are whole 16-byte vectors (V a multiple of 4, the
// logits 16-byte aligned) and one row is at most 32768 long, every thread
// loads its 32 values at once -- one memory round trip -- and keeps them in
// registers for the sum; otherwise it strides over the row and reads it
// twice.
constexpr int kStatThreads = 1024;
constexpr int kStatVec = 8;   // 16-byte loads per thread in the one-round path

__device__ __forceinline__ void stat_take(float v, int i, float& bv, int& bi, bool& bad) {
  if (!isfinite(v)) bad = true;
  if (better(v, i, bv, bi)) { bv = v; bi = i; }
}

__global__ __launch_bounds__(kStatThreads) void row_stats_kernel(VerifyParams p) {
  constexpr int NW = kStatThreads / 64;
  __shared__ float sv[NW];
  __shared__ int si[NW];
  __shared__ double sd[NW];
  __shared__ int sbad;
  const int r = blockIdx.x, b = blockIdx.y;
  const int n = p.t_n[b];
  if (n < 0 || r > n) return;
  const int rows1 = p.N + 1;
  const int64_t o = static_cast<int64_t>(b) * rows1 + r;
  const float* lg = p.logits + o * p.V;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) sbad = 0;
  const bool one_round = p.V % 4 == 0 && p.V <= kStatThreads * 4 * kStatVec &&
                         (reinterpret_cast<uintptr_t>(p.logits) & 15) == 0;
  f32x4 x[kStatVec];
  float bv = -INFINITY;
  int bi = 0x7fffffff;
  bool bad = false;
  if (one_round) {
#pragma unroll
    for (int u = 0; u < kStatVec; ++u) {
      const int i = 4 * (tid + kStatThreads * u);
      x[u] = i < p.V ? *reinterpret_cast<const f32x4*>(lg + i)
                     : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int u = 0; u < kStatVec; ++u) {
      const int i = 4 * (tid + kStatThreads * u);
      if (i < p.V)
#pragma unroll
        for (int e = 0; e < 4; ++e) stat_take(x[u][e], i + e, bv, bi, bad);
    }
  } else {
    for (int i = tid; i < p.V; i += kStatThreads) stat_take(lg[i], i, bv, bi, bad);
  }
  // block argmax (value, then the smaller index)
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = shfl_xor(bv, m);
    const int oi = shfl_xor(bi, m);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  __syncthreads();
  if (bad) atomicOr(&sbad, 1);
  if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
  __syncthreads();
  float mx = sv[0];
  int arg = si[0];
#pragma unroll
  for (int w = 1; w < NW; ++w)
    if (better(sv[w], si[w], mx, arg)) { mx = sv[w]; arg = si[w]; }
  double acc = 0.0;
  if (p.T > 0.f) {
    if (one_round) {
#pragma unroll
      for (int u = 0; u < kStatVec; ++u) {
        const int i = 4 * (tid + kStatThreads * u);
        if (i < p.V)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc += static_cast<double>(wexp(x[u][e], mx, p.T));
      }
    } else {
      for (int i = tid; i < p.V; i += kStatThreads) acc += static_cast<double>(wexp(lg[i], mx, p.T));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0) sd[wave] = acc;
    __syncthreads();
  }
  if (tid == 0) {
    double S = 0.0;
    if (p.T > 0.f)
#pragma unroll
      for (int w = 0; w < NW; ++w) S += sd[w];
    p.row_max[o] = mx;
    p.row_arg[o] = arg;
    p.row_sum[o] = S;
    p.row_bad[o] = sbad;
  }
}

// Draw j of flattened row v of sequence b: the caller's uniforms when given
// (column j < K, or column K for the residual draw), else Philox.
__device__ __forceinline__ float draw_uniform(const VerifyParams& p, int b, int v, int j) {
  if (p.uniforms != nullptr) {
    const int col = j == kBonusDraw ? p.K : j;
    return p.uniforms[(static_cast<int64_t>(b) * (p.N + 1) + v) * (p.K + 1) + col];
  }
  return philox_uniform(p.seed, kStreamVerify, p.round, static_cast<uint64_t>(b),
                        static_cast<uint64_t>(v), static_cast<uint64_t>(j));
}

// Block-wide sum of one double per thread (s: 256 doubles of LDS); every
// thread gets the total.
__device__ __forceinline__ double block_sum_d(double v, double* s) {
  const int tid = threadIdx.x;
  __syncthreads();
  s[tid] = v;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (tid < w) s[tid] += s[tid + w];
    __syncthreads();
  }
  const double t = s[0];
  __syncthreads();
  return t;
}

// The walk of a tree with sampled children, by the whole workgroup
// (Algorithm 1 of the verification with per-child draft distributions: the
// children of a row were drawn from q = softmax(draft / T) without
// replacement, so the i-th child's distribution is q without the earlier
// children, renormalised).  With p = softmax(target / T), the residual after
// i rejections is (p(y) - C(y) q(y))+ / N_i, C(y) = C_i for tokens not yet
// drawn and frozen at C_j for the j-th drawn token, where C_0 = 0, N_0 = 1,
// C_i = C_(i-1) + N_(i-1) / R_i and R_i is the q mass not drawn before
// child i; child i is accepted when u_i < (p - C_(i-1) q)+(x_i) R_i /
// (N_(i-1) q(x_i)).  A residual of zero mass restarts from p.  Rows without
// children, and rows whose children were all rejected, emit a token drawn
// from the residual by inverse CDF over ascending ids.
__device__ void sampled_walk(const VerifyParams& p, int b, int* s_acc, int* s_a_out,
                             int* s_bonus_out, int* s_bad_out, double* s_red, int* s_pick) {
  __shared__ int s_v, s_fc, s_nc, s_stop, s_acc_n, s_bad, s_nd, s_take;
  __shared__ double s_C, s_N, s_R;
  __shared__ int s_dx[kMaxTopK];
  __shared__ double s_dc[kMaxTopK];
  __shared__ float s_mq;
  const int tid = threadIdx.x;
  const int rows1 = p.N + 1;
  const int64_t ob = static_cast<int64_t>(b) * rows1;
  const float T = p.T;
  if (tid == 0) { s_v = 0; s_acc_n = 0; s_bad = 0; s_stop = 0; }
  __syncthreads();
  while (true) {
    if (tid == 0) {
      const int v = s_v;
      const int fc = p.t_first[ob + v], nc = p.t_nchild[ob + v];
      if (p.row_bad[ob + v] || nc < 0 || nc > kMaxTopK ||
          (nc > 0 && (fc < 1 || fc + nc > rows1)))
        s_bad = 1;
      if (nc > 0) {
        const int e = v == 0 ? 0 : 1 + p.t_slot[ob + v];
        if (e < 0 || e >= p.NE) s_bad = 1;
        for (int j = 0; j < nc && !s_bad; ++j) {
          const int t = p.t_token[ob + fc + j];
          if (t < 0 || t >= p.V) s_bad = 1;
        }
      }
      s_fc = fc;
      s_nc = nc;
      s_C = 0.0; s_N = 1.0; s_R = 1.0; s_nd = 0;
    }
    __syncthreads();
    if (s_bad) break;
    const int v = s_v, fc = s_fc, nc = s_nc;
    const float* tl = p.logits + (ob + v) * p.V;
    const float mt = p.row_max[ob + v];
    const double St = p.row_sum[ob + v];
    const float* dl = nullptr;
    double Sq = 1.0;
    if (nc > 0) {
      const int e = v == 0 ? 0 : 1 + p.t_slot[ob + v];
      dl = p.draft_rows + (static_cast<int64_t>(b) * p.NE + e) * p.V;
      float mq = -INFINITY;
      for (int i = tid; i < p.V; i += 256) mq = fmaxf(mq, dl[i]);
      mq = wave_max(mq);
      if ((tid & 63) == 0) s_pick[tid >> 6] = __float_as_int(mq);
      __syncthreads();
      if (tid == 0) {
        float m = -INFINITY;
        for (int w = 0; w < 4; ++w) m = fmaxf(m, __int_as_float(s_pick[w]));
        s_mq = m;
      }
      __syncthreads();
      double part = 0.0;
      for (int i = tid; i < p.V; i += 256) part += static_cast<double>(wexp(dl[i], s_mq, T));
      Sq = block_sum_d(part, s_red);
    }
    const float mq = s_mq;
    auto pt = [&](int y) { return static_cast<double>(wexp(tl[y], mt, T)) / St; };
    auto qd = [&](int y) { return static_cast<double>(wexp(dl[y], mq, T)) / Sq; };
    int accepted = -1;
    for (int i = 0; i < nc; ++i) {
      if (tid == 0) {
        const int x = p.t_token[ob + fc + i];
        const double px = pt(x), qx = qd(x);
        const double num = fmax(0.0, px - s_C * qx) * s_R;
        const double den = s_N * qx;
        const double u = static_cast<double>(draw_uniform(p, b, v, i));
        s_take = (den <= 0.0) ? (num > 0.0) : (u * den < num);
        if (!s_take) {
          const double Cn = s_C + s_N / s_R;
          s_dx[s_nd] = x;
          s_dc[s_nd] = Cn;
          s_nd += 1;
          s_R -= qx;
          s_C = Cn;
        }
      }
      __syncthreads();
      if (s_take) { accepted = i; break; }
      // N_i: the bulk at the new C, then the tokens drawn before this one
      // at their frozen C
      const double C = s_C;
      double part = 0.0;
      for (int y = tid; y < p.V; y += 256) part += fmax(0.0, pt(y) - C * qd(y));
      const double bulk = block_sum_d(part, s_red);
      if (tid == 0) {
        double Nn = bulk;
        for (int j = 0; j + 1 < s_nd; ++j) {
          const int y = s_dx[j];
          Nn += fmax(0.0, pt(y) - s_dc[j] * qd(y)) - fmax(0.0, pt(y) - C * qd(y));
        }
        if (Nn > 0.0) {
          s_N = Nn;
        } else {  // zero-mass residual: start again from p
          s_C = 0.0;
          s_N = 1.0;
          s_nd = 0;
        }
      }
      __syncthreads();
    }
    if (accepted >= 0) {
      if (tid == 0) {
        if (s_acc_n >= p.D || s_acc_n >= kMaxPath) {
          s_bad = 1;
        } else {
          s_acc[s_acc_n++] = fc + accepted;
          s_v = fc + accepted;
        }
      }
      __syncthreads();
      if (s_bad) break;
      continue;
    }
    // ---- emitted token: inverse CDF of the residual over ascending ids ----
    const double C = s_C;
    const int nd = s_nd;
    auto wres = [&](int y) {
      if (dl == nullptr) return pt(y);
      double c = C;
      for (int j = 0; j < nd; ++j)
        if (s_dx[j] == y) c = s_dc[j];
      return fmax(0.0, pt(y) - c * qd(y));
    };
    const int per = (p.V + 255) / 256;
    const int lo = tid * per, hi = min(p.V, lo + per);
    double mine = 0.0;
    for (int y = lo; y < hi; ++y) mine += wres(y);
    __syncthreads();
    s_red[tid] = mine;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const double t = tid >= off ? s_red[tid - off] : 0.0;
      __syncthreads();
      s_red[tid] += t;
      __syncthreads();
    }
    const double total = s_red[255];
    const double excl = s_red[tid] - mine;
    const double thr = static_cast<double>(draw_uniform(p, b, v, kBonusDraw)) * total;
    int pick = -1, lastnz = -1;
    double cum = excl;
    for (int y = lo; y < hi; ++y) {
      const double w = wres(y);
      if (w > 0.0) lastnz = y;
      if (pick < 0 && w > 0.0 && thr >= excl) {
        cum += w;
        if (cum > thr) pick = y;
      }
    }
    __syncthreads();
    s_pick[tid] = pick;
    s_pick[256 + tid] = lastnz;
    __syncthreads();
    if (tid == 0) {
      int best = -1, last = -1;
      for (int t = 0; t < 256 && best < 0; ++t) best = s_pick[t];
      for (int t = 0; t < 256; ++t) last = max(last, s_pick[256 + t]);
      *s_bonus_out = best >= 0 ? best : last;
      if (*s_bonus_out < 0) s_bad = 1;
    }
    __syncthreads();
    break;
  }
  if (tid == 0) {
    *s_a_out = s_acc_n;
    *s_bad_out = s_bad;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void walk_kernel(VerifyParams p) {
  __shared__ int s_kids[kMaxTopK];
  __shared__ int s_nk, s_row, s_need_res, s_bad, s_a, s_bonus;
  __shared__ int s_acc[kMaxPath];
  __shared__ double s_part[256];
  __shared__ int s_pick[512];
  __shared__ int s_kept[kMaxPath];
  __shared__ int s_nkept;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int rows1 = p.N + 1;
  const int64_t ob = static_cast<int64_t>(b) * rows1;
  const int n = p.t_n[b];
  if (n < 0) {
    if (tid == 0) {
      p.accept_len[b] = -1;
      for (int i = 0; i < p.D; ++i) p.accepted_rows[b * p.D + i] = -1;
      for (int i = 0; i <= p.D; ++i) p.out_tokens[b * (p.D + 1) + i] = -1;
      p.seed_len[b] = 0;
      for (int i = 0; i < p.S; ++i) p.seed_rows[b * p.S + i] = p.seed_tokens[b * p.S + i] = -1;
    }
    return;
  }

  if (p.draft_rows != nullptr) {
    sampled_walk(p, b, s_acc, &s_a, &s_bonus, &s_bad, s_part, s_pick);
    __syncthreads();
  } else {
    if (tid == 0) {
      int v = 0, a = 0, bad = 0, need = 0, bonus = -1;
      while (true) {
        if (p.row_bad[ob + v]) { bad = 1; break; }
        const int fc = p.t_first[ob + v], nc = p.t_nchild[ob + v];
        if (nc < 0 || nc > kMaxTopK || (nc > 0 && (fc < 1 || fc + nc > rows1))) {
          bad = 1;
          break;
        }
        const float* lg = p.logits + (ob + v) * p.V;
        int nxt = -1;
        if (p.T == 0.f) {
          const int x = p.row_arg[ob + v];
          for (int j = 0; j < nc; ++j)
            if (p.t_token[ob + fc + j] == x) nxt = fc + j;
          if (nxt < 0) { bonus = x; break; }
        } else {
          double S = p.row_sum[ob + v];
          const float mx = p.row_max[ob + v];
          for (int j = 0; j < nc; ++j) {
            const int tok = p.t_token[ob + fc + j];
            if (tok < 0 || tok >= p.V) { bad = 1; break; }
            s_kids[j] = tok;
            const double w = static_cast<double>(wexp(lg[tok], mx, p.T));
            const float u = draw_uniform(p, b, v, j);
            if (static_cast<double>(u) * S < w) { nxt = fc + j; break; }
            S -= w;
          }
          if (bad) break;
          if (nxt < 0) {
            need = 1;
            s_nk = nc;
            break;
          }
        }
        if (a >= p.D || a >= kMaxPath) { bad = 1; break; }  // malformed tree
        s_acc[a++] = nxt;
        v = nxt;
      }
      s_row = v;
      s_need_res = need;
      s_bad = bad;
      s_a = a;
      s_bonus = bonus;
    }
    __syncthreads();

    if (s_need_res && !s_bad) {
      // residual draw at row v: children's tokens removed, inverse CDF
      const int v = s_row;
      const float* lg = p.logits + (ob + v) * p.V;
      const float mx = p.row_max[ob + v];
      const int nk = s_nk;
      const int per = (p.V + 255) / 256;
      const int lo = tid * per, hi = min(p.V, lo + per);
      double part = 0.0;
      for (int i = lo; i < hi; ++i) {
        bool kid = false;
        for (int j = 0; j < nk; ++j) kid |= s_kids[j] == i;
        if (!kid) part += static_cast<double>(wexp(lg[i], mx, p.T));
      }
      s_part[tid] = part;
      __syncthreads();
      for (int off = 1; off < 256; off <<= 1) {
        const double t = tid >= off ? s_part[tid - off] : 0.0;
        __syncthreads();
        s_part[tid] += t;
        __syncthreads();
      }
      const double total = s_part[255];
      const double excl = s_part[tid] - part;
      const double u = static_cast<double>(draw_uniform(p, b, v, kBonusDraw));
      const double thr = u * total;
      int pick = -1;
      if (total > 0.0) {
        if (thr >= excl && thr < excl + part) {
          double cum = excl;
          for (int i = lo; i < hi && pick < 0; ++i) {
            bool kid = false;
            for (int j = 0; j < nk; ++j) kid |= s_kids[j] == i;
            if (kid) continue;
            cum += static_cast<double>(wexp(lg[i], mx, p.T));
            if (cum > thr) pick = i;
          }
        }
        s_pick[tid] = pick;
        __syncthreads();
        if (tid == 0) {
          int best = -1;
          for (int t = 0; t < 256 && best < 0; ++t) best = s_pick[t];
          s_bonus = best;
        }
        __syncthreads();
        if (s_bonus < 0) {  // rounding put the threshold past the last mass
          int lastnz = -1;
          for (int i = lo; i < hi; ++i) {
            bool kid = false;
            for (int j = 0; j < nk; ++j) kid |= s_kids[j] == i;
            if (!kid && wexp(lg[i], mx, p.T) > 0.f) lastnz = i;
          }
          s_pick[tid] = lastnz;
          __syncthreads();
          if (tid == 0) {
            int best = -1;
            for (int t = 0; t < 256; ++t) best = max(best, s_pick[t]);
            s_bonus = best;
          }
        }
      } else {
        // the children held all the mass: best remaining token
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        for (int i = lo; i < hi; ++i) {
          bool kid = false;
          for (int j = 0; j < nk; ++j) kid |= s_kids[j] == i;
          if (!kid && better(lg[i], i, bv, bi)) { bv = lg[i]; bi = i; }
        }
        s_part[tid] = bv;
        s_pick[tid] = bi;
        __syncthreads();
        if (tid == 0) {
          float best = -INFINITY;
          int bid = 0x7fffffff;
          for (int t = 0; t < 256; ++t)
            if (better(static_cast<float>(s_part[t]), s_pick[t], best, bid)) {
              best = static_cast<float>(s_part[t]);
              bid = s_pick[t];
            }
          s_bonus = bid;
        }
      }
      __syncthreads();
    }
  }

  // ---- outputs, next seed, commit ----
  const int a = s_a;
  const bool bad = s_bad;
  const int p_root = p.t_pos[ob];
  const int len_out = p_root + 1;
  if (tid == 0) {
    int* srow = p.seed_rows + b * p.S;
    int* stok = p.seed_tokens + b * p.S;
    for (int i = 0; i < p.S; ++i) srow[i] = stok[i] = -1;
    if (bad) {
      atomicOr(p.status, 1 << 5);
      p.accept_len[b] = -1;
      for (int i = 0; i < p.D; ++i) p.accepted_rows[b * p.D + i] = -1;
      for (int i = 0; i <= p.D; ++i) p.out_tokens[b * (p.D + 1) + i] = -1;
      p.seed_len[b] = 0;
      s_nkept = 0;
    } else {
      const int bonus = s_bonus;
      p.accept_len[b] = a;
      for (int i = 0; i < p.D; ++i) p.accepted_rows[b * p.D + i] = i < a ? s_acc[i] : -1;
      for (int i = 0; i <= p.D; ++i) {
        int t = -1;
        if (i < a) t = p.t_token[ob + s_acc[i]];
        else if (i == a) t = bonus;
        p.out_tokens[b * (p.D + 1) + i] = t;
      }
      int nk = 0;
      if (p.commit_mode == 1) {
        // full reseed: every verified row's feature joins the next token
        p.seed_len[b] = a + 1;
        for (int i = 0; i <= a; ++i) {
          srow[i] = i == 0 ? 0 : s_acc[i - 1];
          stok[i] = i < a ? p.t_token[ob + s_acc[i]] : bonus;
        }
      } else if (a == 0) {
        p.seed_len[b] = 1;
        srow[0] = 0;
        stok[0] = bonus;
      } else if (p.t_slot[ob + s_acc[a - 1]] >= 0) {
        for (int i = 0; i < a; ++i) s_kept[nk++] = s_acc[i];
        p.seed_len[b] = 1;
        srow[0] = s_acc[a - 1];
        stok[0] = bonus;
      } else {
        for (int i = 0; i < a - 1; ++i) s_kept[nk++] = s_acc[i];
        p.seed_len[b] = 2;
        srow[0] = a >= 2 ? s_acc[a - 2] : 0;
        stok[0] = p.t_token[ob + s_acc[a - 1]];
        srow[1] = s_acc[a - 1];
        stok[1] = bonus;
      }
      s_nkept = nk;
    }
  }
  __syncthreads();
  if (p.kc == nullptr) return;
  const int nk = s_nkept;
  if (tid == 0) p.kv_len[b] = len_out + nk;
  if (nk == 0) return;
  // gather every kept row first, then scatter: destinations can overlap
  // sources of other kept rows.  K rows are [cap, hd]; V is stored
  // transposed ([hd, cap]), so a V "row" is a column.
  extern __shared__ __attribute__((aligned(16))) uint16_t s_rows[];
  const int n16 = p.hd * p.elem_bytes / 2;  // 16-bit units per row
  const int u16 = p.elem_bytes / 2;         // 16-bit units per element
  for (int kvh = 0; kvh < p.nkv; ++kvh) {
    const int64_t bk = static_cast<int64_t>(b) * p.nkv + kvh;
    for (int which = 0; which < 2; ++which) {
      uint16_t* cache = static_cast<uint16_t*>(which ? p.vc : p.kc);
      auto at = [&](int row, int off) -> int64_t {
        if (which == 0) return (bk * p.cap + row) * n16 + off;
        const int d = off / u16, w = off % u16;
        return ((bk * p.hd + d) * p.cap + row) * u16 + w;
      };
      for (int e = tid; e < nk * n16; e += 256) {
        const int i = e / n16, off = e % n16;
        const int src = len_out + p.t_slot[ob + s_kept[i]];
        s_rows[e] = (src >= 0 && src < p.cap) ? cache[at(src, off)] : 0;
      }
      __syncthreads();
      for (int e = tid; e < nk * n16; e += 256) {
        const int i = e / n16, off = e % n16;
        const int dst = p_root + p.t_depth[ob + s_kept[i]];
        if (dst >= 0 && dst < p.cap) cache[at(dst, off)] = s_rows[e];
      }
      __syncthreads();
    }
  }
}

hipError_t launch_verify(const VerifyParams& p, hipStream_t s) {
  hipLaunchKernelGGL(row_stats_kernel, dim3(p.N + 1, p.batch), dim3(kStatThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = static_cast<size_t>(p.D) * p.hd * p.elem_bytes;
  hipLaunchKernelGGL(walk_kernel, dim3(p.batch), dim3(256), lds, s, p);
  return hipGetLastError();
}

__global__ void uniforms_kernel(uint64_t seed, uint64_t stream, uint64_t rnd, int rows,
                                int draws, float* out) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  const int r = blockIdx.y, b = blockIdx.z;
  if (j >= draws) return;
  out[(static_cast<int64_t>(b) * rows + r) * draws + j] =
      philox_uniform(seed, stream, rnd, static_cast<uint64_t>(b), static_cast<uint64_t>(r),
                     static_cast<uint64_t>(j));
}

hipError_t launch_uniforms(uint64_t seed, uint64_t stream, uint64_t rnd, int batch, int rows,
                           int draws, float* out, hipStream_t s) {
  if (batch <= 0 || rows <= 0 || draws <= 0) return hipSuccess;
  hipLaunchKernelGGL(uniforms_kernel, dim3((draws + 255) / 256, rows, batch), dim3(256), 0, s,
                     seed, stream, rnd, rows, draws, out);
  return hipGetLastError();
}

// ============================================================================
// target tree layer set-up: row r of sequence b is tree row r, written to
// cache row len_in[b] + r, seeing the prefix [0, len_in) and the tree rows of
// its ancestor mask (bit j = cache row len_in + j); rows past n_nodes (or of
// a sequence whose rows do not fit the cache) are padding
// ============================================================================
__global__ void target_rows_kernel(TargetRowsParams p) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.batch * p.n1) return;
  const int b = idx / p.n1, r = idx - b * p.n1;
  const int len = p.len_in[b];
  const int n = p.n_nodes[b];
  const bool ok = n >= 0 && n < p.n1 && len >= 0 &&
                  static_cast<int64_t>(len) + p.n1 <= p.cap;
  if (!ok && r == 0 && p.status != nullptr) atomicOr(p.status, 1 << 4);
  const bool valid = ok && r <= n;
  p.tok[idx] = valid ? p.token[idx] : -1;
  p.pos[idx] = valid ? p.position[idx] : 0;
  p.dest[idx] = ok ? len + r : 0;
  p.plen[idx] = ok ? len : 0;
  p.rmask[idx] = valid ? p.mask[static_cast<int64_t>(idx) * p.mask_words] : 0ull;
  if (r == 0) p.sbase[b] = ok ? len : 0;
}

hipError_t launch_target_rows(const TargetRowsParams& p, hipStream_t s) {
  const int n = p.batch * p.n1;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(target_rows_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p);
  return hipGetLastError();
}

// x[row] = E[tok[row]] as fp32 (zero for padding rows) and the sums of
// squares of its 16-column tiles, which the next GEMM's RMSNorm reads
template <typename T>
__global__ __launch_bounds__(64) void embed_rows_kernel(const T* embed, int vocab,
                                                        const int32_t* tok, int H, float* x,
                                                        float* ss) {
  const int row = blockIdx.x;
  const int t = tok[row];
  const bool ok = t >= 0 && t < vocab;
  const int ntile = H / 16;
  for (int tile = threadIdx.x; tile < ntile; tile += 64) {
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float v = ok ? Elem<T>::to_f(embed[static_cast<int64_t>(t) * H + tile * 16 + i]) : 0.f;
      x[static_cast<int64_t>(row) * H + tile * 16 + i] = v;
      q += v * v;
    }
    ss[static_cast<int64_t>(row) * ntile + tile] = q;
  }
}

template <typename T>
hipError_t launch_embed_rows(const T* embed, int vocab, const int32_t* tok, int rows, int H,
                             float* x, float* ss, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(embed_rows_kernel<T>, dim3(rows), dim3(64), 0, s, embed, vocab, tok, H,
                     x, ss);
  return hipGetLastError();
}
template hipError_t launch_embed_rows<uint16_t>(const uint16_t*, int, const int32_t*, int, int,
                                                float*, float*, hipStream_t);
template hipError_t launch_embed_rows<float>(const float*, int, const int32_t*, int, int, float*,
                                             float*, hipStream_t);

__global__ void fill_i32_kernel(int32_t* p, int32_t v, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                     dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

}  // namespace eagle
