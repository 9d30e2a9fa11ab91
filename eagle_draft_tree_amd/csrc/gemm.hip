// Streaming MFMA GEMM for the draft path: C[M, N] = A[M, K] * W[N, K]^T with
// M <= 64 rows per chunk (bs1 trees: M = 1..16).  At these shapes the op is
// a stream of the weights from HBM, so the kernel is organised around them:
//  * a workgroup owns 64 CT output columns (four waves of CT 16-column tiles)
//    and one slice of K (S slices split K across workgroups);
//  * its slice of A is normalised (RMSNorm factor and gain), split into
//    bf16 hi + lo parts and laid out in LDS in MFMA fragment order, one
//    piece of steps at a time, the next piece fetched into registers while
//    the current one is used -- every wave then reads its A fragments with
//    one 16-byte LDS load per MFMA;
//  * the weights are packed once (pack_weights) in MFMA fragment order: for
//    each 128-wide k step, 16-column tile and 32-wide sub-step e, the 64
//    lanes' 8-element fragments lie contiguously, so every weight load of a
//    wave reads 1 KB of contiguous memory (row-major tiles touch 16 rows per
//    load and stream at well under half the bandwidth).  Tiles are
//    interleaved per k step, so the waves that run together read neighbouring
//    blocks and spread over all HBM channels instead of queuing on a few.  Lane (g, c) of
//    sub-step e holds column c at k = step*128 + g*32 + e*8 .. +7; A is laid
//    out with the same k permutation, so each 16x16x32 MFMA sums the right
//    products.  kPF steps of loads stay in flight, with no branch in the
//    loop body: steps past the slice re-read valid weights against an
//    all-zero A block;
//  * with S K-splits the partial sums go to a workspace and the last
//    workgroup of a column group to arrive sums them in split order
//    (deterministic) and runs the fused epilogue;
//  * RMSNorm of the A operand: the producer leaves per-16-column sums of
//    squares, and each consumer workgroup derives the row factor itself.
#include "common.hpp"
#include "kernels.hpp"

namespace eagle {

namespace {

constexpr int kStep = 128;     // k elements per wave step (4 lane groups x 32)
constexpr int kPF = 4;         // weight steps in flight per wave
constexpr int kBlk = 2048;     // bytes of one (step, e, row tile) A block in LDS
constexpr int kLdsCap = 130 * 1024;  // dynamic LDS a launch may use
constexpr int kPackBlk = 512;  // elements of one packed (tile, step, e) block

// global output column and weight row of tile column c
__device__ __forceinline__ int tile_col(const GemmParams& p, int tile, int c) {
  if (p.colmap == MAP_QKV) {
    const int hpt = p.hd / 16;
    const int hh = tile / hpt, pp = tile % hpt;
    const int cin = c < 8 ? 8 * pp + c : p.hd / 2 + 8 * pp + (c - 8);
    return hh * p.hd + cin;
  }
  if (p.colmap == MAP_SWIGLU) return 8 * tile + (c & 7);  // gate/up row
  return tile * 16 + c;
}

template <typename T>
__device__ __forceinline__ const T* weight_row(const GemmParams& p, int tile, int c) {
  const int col = tile_col(p, tile, c);
  const int64_t K = p.K;
  if (p.colmap == MAP_QKV) {
    if (col < p.qkv_n0) return static_cast<const T*>(p.w0) + col * K;
    if (col < p.qkv_n0 + p.qkv_n1) return static_cast<const T*>(p.w1) + (col - p.qkv_n0) * K;
    return static_cast<const T*>(p.w2) + (col - p.qkv_n0 - p.qkv_n1) * K;
  }
  if (p.colmap == MAP_SWIGLU) return static_cast<const T*>(c < 8 ? p.w0 : p.w1) + col * K;
  return static_cast<const T*>(p.w0) + col * K;
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + expf(-x)); }

// 8 consecutive A elements of segment-local column kk of one row, as floats
template <typename T>
__device__ __forceinline__ void load8(const ASeg& sg, int64_t row, int kk, float (&v)[8]) {
  if (sg.f32) {
    const float* src = static_cast<const float*>(sg.base) + row * sg.ld + kk;
    const f32x4 a = *reinterpret_cast<const f32x4*>(src);
    const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
  } else {
    Frag8<T> w;
    w.load(static_cast<const T*>(sg.base) + row * sg.ld + kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = w.get(i);
  }
}

// RMSNorm factors of rows m0 .. m0 + 16 MT of segment 0 (the only one that
// may be normalised) from the producer's per-16-column sums of squares:
// 1 / sqrt(mean(y^2) + eps), one value per row into rn (1 when segment 0 is
// not normalised).
template <int MT>
__device__ __forceinline__ void row_factors(const GemmParams& p, float* rn, int m0) {
  const ASeg& sg = p.seg[0];
  if (!sg.f32 || sg.ss == nullptr) {
    for (int r = threadIdx.x; r < 16 * MT; r += 256) rn[r] = 1.f;
    return;
  }
  constexpr int TPR = 256 / (16 * MT);  // threads per row: 16, 8, 4
  constexpr int kU = 16;                 // 16-byte loads in flight per thread
  const int r = threadIdx.x / TPR, part = threadIdx.x % TPR;
  const int row = m0 + r;
  float q = 0.f;
  if (row < p.M) {
    const float* src = sg.ss + static_cast<int64_t>(row) * sg.ss_tiles;
    if ((sg.ss_tiles & 3) == 0) {
      // four partial sums per load, kU loads issued before any is added
      const int n4 = sg.ss_tiles >> 2;
      for (int t0 = part; t0 < n4; t0 += TPR * kU) {
        f32x4 x[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u)
          x[u] = *reinterpret_cast<const f32x4*>(src + 4 * min(t0 + u * TPR, n4 - 1));
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (t0 + u * TPR < n4) q += (x[u][0] + x[u][1]) + (x[u][2] + x[u][3]);
      }
    } else {
      for (int t = part; t < sg.ss_tiles; t += TPR) q += src[t];
    }
  }
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) q += shfl_xor(q, o);
  if (part == 0) rn[r] = 1.f / sqrtf(q / static_cast<float>(sg.width) + p.eps);
}

// Value of A[row m0 + m][k .. k+7] as the GEMM multiplies it: the row of the
// segment holding k (gathered through its row index), times the RMSNorm
// factor and gain when segment 0 is normalised; zero past M, K or a gather
// out of range.
template <typename T>
__device__ __forceinline__ void a_values(const GemmParams& p, const float* rn, int m,
                                         int row, int k, int kend, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  if (row >= p.M || k >= kend) return;
  // the segment holding k; its fields are picked lane by lane from the
  // three (uniform) descriptors -- indexing the descriptor array by a
  // per-lane segment would read the kernel arguments through vector loads,
  // each one waiting for every load in flight, weights included
  const ASeg &s0 = p.seg[0], &s1 = p.seg[1], &s2 = p.seg[2];
  const int w0 = s0.width, w01 = s0.width + s1.width;
  const int si = (p.nseg > 1 && k >= w0) ? ((p.nseg > 2 && k >= w01) ? 2 : 1) : 0;
  const int kk = k - (si == 0 ? 0 : (si == 1 ? w0 : w01));
  const void* base = si == 0 ? s0.base : (si == 1 ? s1.base : s2.base);
  const int64_t ld = si == 0 ? s0.ld : (si == 1 ? s1.ld : s2.ld);
  const int32_t* rowidx = si == 0 ? s0.rowidx : (si == 1 ? s1.rowidx : s2.rowidx);
  const int rowlimit = si == 0 ? s0.rowlimit : (si == 1 ? s1.rowlimit : s2.rowlimit);
  const int f32 = si == 0 ? s0.f32 : (si == 1 ? s1.f32 : s2.f32);
  int r = row;
  if (rowidx != nullptr) {
    r = rowidx[row];
    if (r < 0 || r >= rowlimit) return;
  }
  if (f32) {
    const float* src = static_cast<const float*>(base) + r * ld + kk;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = x0[i]; v[4 + i] = x1[i]; }
  } else {
    Frag8<T> w;
    w.load(static_cast<const T*>(base) + r * ld + kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = w.get(i);
  }
  // RMSNorm (segment 0 only): row factor and gain
  if (si == 0 && s0.f32 && s0.ss != nullptr) {
    const float f = rn[m];
    Frag8<T> gv;
    gv.load(static_cast<const T*>(s0.gain) + kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * f * gv.get(i);
  }
}

// A[row][k .. k+7] as stored (gathered through the segment's row index),
// before any RMSNorm; zero past M, kend or a gather out of range
template <typename T>
__device__ __forceinline__ void a_raw_values(const GemmParams& p, int row, int k, int kend,
                                             float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.f;
  if (row >= p.M || k >= kend) return;
  const ASeg &s0 = p.seg[0], &s1 = p.seg[1], &s2 = p.seg[2];
  const int w0 = s0.width, w01 = s0.width + s1.width;
  const int si = (p.nseg > 1 && k >= w0) ? ((p.nseg > 2 && k >= w01) ? 2 : 1) : 0;
  const int kk = k - (si == 0 ? 0 : (si == 1 ? w0 : w01));
  const void* base = si == 0 ? s0.base : (si == 1 ? s1.base : s2.base);
  const int64_t ld = si == 0 ? s0.ld : (si == 1 ? s1.ld : s2.ld);
  const int32_t* rowidx = si == 0 ? s0.rowidx : (si == 1 ? s1.rowidx : s2.rowidx);
  const int rowlimit = si == 0 ? s0.rowlimit : (si == 1 ? s1.rowlimit : s2.rowlimit);
  const int f32 = si == 0 ? s0.f32 : (si == 1 ? s1.f32 : s2.f32);
  int r = row;
  if (rowidx != nullptr) {
    r = rowidx[row];
    if (r < 0 || r >= rowlimit) return;
  }
  if (f32) {
    const float* src = static_cast<const float*>(base) + r * ld + kk;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(src);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = x0[i]; v[4 + i] = x1[i]; }
  } else {
    Frag8<T> w;
    w.load(static_cast<const T*>(base) + r * ld + kk);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = w.get(i);
  }
}

// bf16 hi + lo parts of 8 fp32 values (hi = nearest bf16, lo = the rest)
__device__ __forceinline__ void split_hi_lo(const float (&v)[8], u32x4& hi_out, u32x4& lo_out) {
  Frag8<uint16_t> hi, lo;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hi.set_pair(j, v[2 * j], v[2 * j + 1]);
    lo.set_pair(j, v[2 * j] - hi.get(2 * j), v[2 * j + 1] - hi.get(2 * j + 1));
  }
  hi_out = hi.v;
  lo_out = lo.v;
}

// Stage rows [m0, m0 + 16 MT) x k in [k0, kend) of A in LDS, fragment order:
// block ((s * 4 + e) * MT + mt) holds, for each lane (g, c), the 8 values of
// row mt*16 + c at k = k0 + s*128 + g*32 + e*8.  bf16: hi at lane*16 and lo
// at 1024 + lane*16; fp32: values at lane*32.  The block after the last
// (index nsteps * 4 * MT) is all zero.
template <typename T, int MT>
__device__ __forceinline__ void fill_a(const GemmParams& p, unsigned char* lds, const float* rn,
                                       int m0, int k0, int kend, int nsteps) {
  const int k8n = nsteps * 16;
  const int total = MT * 16 * k8n;
  for (int idx = threadIdx.x; idx < total; idx += 256) {
    const int m = idx / k8n, k8 = idx - m * k8n;
    float v[8];
    a_values<T>(p, rn, m, m0 + m, k0 + 8 * k8, kend, v);
    const int s = k8 >> 4, rem = k8 & 15;
    const int g = rem >> 2, e = rem & 3;
    const int mt = m >> 4, c = m & 15;
    const int lane = g * 16 + c;
    unsigned char* blk = lds + static_cast<size_t>((s * 4 + e) * MT + mt) * kBlk;
    if constexpr (sizeof(T) == 2) {
      u32x4 hi, lo;
      split_hi_lo(v, hi, lo);
      *reinterpret_cast<u32x4*>(blk + lane * 16) = hi;
      *reinterpret_cast<u32x4*>(blk + 1024 + lane * 16) = lo;
    } else {
      *reinterpret_cast<f32x4*>(blk + lane * 32) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(blk + lane * 32 + 16) = f32x4{v[4], v[5], v[6], v[7]};
    }
  }
  // the zero block read by padding steps
  unsigned char* zb = lds + static_cast<size_t>(nsteps * 4 * MT) * kBlk;
  for (int i = threadIdx.x; i < kBlk / 16; i += 256)
    *reinterpret_cast<u32x4*>(zb + i * 16) = u32x4{0u, 0u, 0u, 0u};
}

}  // namespace

// One element of the QKV epilogue: RoPE on q and k columns (partner column
// value `other`, frequency inv), then q to the q buffer, k to cache row
// dest[m] and v to column dest[m] of the transposed V cache.
template <typename T>
__device__ __forceinline__ void qkv_element(const GemmParams& p, int m, int col, int c, float x,
                                         float other, double inv) {
  if (m >= p.M || p.tok[m] < 0) return;
  const int hh = col / p.hd, cin = col % p.hd;
  float y = x;
  if (hh < p.nq + p.nkv) {
    // the angle in double (at positions in the thousands a float product is
    // off by 1e-3 rad and more), reduced there to [-pi, pi]; its sine and
    // cosine then in float, within a few 1e-7 of the exact ones
    const double a = static_cast<double>(p.pos[m]) * inv;
    const double red = a - rint(a * 0.15915494309189535) * 6.283185307179586;
    float sn, cs;
    sincosf(static_cast<float>(red), &sn, &cs);
    y = (c < 8) ? (x * cs - other * sn) : (x * cs + other * sn);
  }
  const T v = Elem<T>::from_f(y);
  if (hh < p.nq) {
    static_cast<T*>(p.out)[m * p.ldo + col] = v;
    return;
  }
  const int b = m / p.rows_per_seq;
  const int d = p.dest[m];
  if (b >= p.batch || d < 0 || d >= p.cap) {
    if (p.status != nullptr) atomicOr(p.status, 1 << 4);
    return;
  }
  const bool isk = hh < p.nq + p.nkv;
  const int kvh = isk ? hh - p.nq : hh - p.nq - p.nkv;
  const int64_t bk = static_cast<int64_t>(b) * p.nkv + kvh;
  // K rows [cap, hd]; V stored transposed, [hd, cap]
  if (isk) static_cast<T*>(p.kc)[(bk * p.cap + d) * p.hd + cin] = v;
  else static_cast<T*>(p.vc)[(bk * p.hd + cin) * p.cap + d] = v;
}

// Fused epilogue on the accumulators of one workgroup tile (column group
// `group`, rows m0 .. m0 + 16 MT), lane layout of the 16x16 MFMA: lane
// (g, c) of tile (mt, ct) holds rows mt*16 + 4g + j, column c.
template <typename T, int MT, int CT>
__device__ __forceinline__ void epilogue(const GemmParams& p, f32x4 (&acc)[MT][CT],
                                         unsigned char* lds, int group, int m0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int ntiles = p.N / 16;
  // ---- epilogues -------------------------------------------------------------
  if (p.epi == EPI_LMHEAD) {
    // the workgroup holds 64 CT consecutive vocabulary columns: stage them in
    // LDS, store each row's logits, and emit per row and 64-column tile the
    // (max, sum of exp) that the merge's log-sum-exp and its choice of tiles
    // need (the merge reads the top-k candidates from the stored logits)
    __syncthreads();
    float* lm = reinterpret_cast<float*>(lds);  // [16 MT rows][64 CT cols]
    constexpr int W = 64 * CT;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          lm[(mt * 16 + 4 * g + j) * W + (wave * CT + ct) * 16 + c] = acc[mt][ct][j];
    __syncthreads();
    const int rows = min(16 * MT, p.M - m0);
    const int64_t ldl = static_cast<int64_t>(p.ntile_lm) * 64;
    if constexpr (MT == 4) {
      // many rows: the logits go out in coalesced row runs, and one thread
      // per (row, tile) pair takes the pair's max and sum of exp from LDS
      // (starting at its own offset, so a wave's reads hit distinct banks)
      for (int idx = threadIdx.x; idx < rows * W; idx += 256) {
        const int r = idx / W, cw = idx % W;
        const int col = group * W + cw;
        if (col >= 64 * p.ntile_lm) continue;
        float v = col < p.N ? lm[r * W + cw] : -INFINITY;
        if (v != v) v = -INFINITY;
        p.lm_logits[(m0 + r) * ldl + col] = v;
      }
      for (int pr = threadIdx.x; pr < 64 * CT; pr += 256) {
        const int r = pr / CT, ch = pr % CT;
        const int lt = group * CT + ch;
        if (r >= rows || lt >= p.ntile_lm) continue;
        const float* rowp = lm + r * W + ch * 64;
        float mx = -INFINITY;
        for (int jj = 0; jj < 64; ++jj) {
          const int j = (jj + pr) & 63;
          float v = lt * 64 + j < p.N ? rowp[j] : -INFINITY;
          if (v != v) v = -INFINITY;
          mx = fmaxf(mx, v);
        }
        float se = 0.f;
        for (int jj = 0; jj < 64; ++jj) {
          const int j = (jj + pr) & 63;
          float v = lt * 64 + j < p.N ? rowp[j] : -INFINITY;
          if (v != v) v = -INFINITY;
          se += v == -INFINITY ? 0.f : expf(v - mx);
        }
        const int64_t o = static_cast<int64_t>(m0 + r) * p.ntile_lm + lt;
        p.stat[o * 2] = mx;
        p.stat[o * 2 + 1] = se;
      }
      return;
    }
    for (int r = wave; r < rows; r += 4) {
#pragma unroll
      for (int ch = 0; ch < CT; ++ch) {
        const int lt = group * CT + ch;   // 64-column LM tile
        if (lt >= p.ntile_lm) continue;
        const int col = lt * 64 + lane;
        const int m = m0 + r;
        float v = col < p.N ? lm[r * W + ch * 64 + lane] : -INFINITY;
        if (v != v) v = -INFINITY;
        p.lm_logits[m * ldl + col] = v;
        const float mx = wave_max(v);
        const float se = wave_sum(v == -INFINITY ? 0.f : expf(v - mx));
        if (lane == 0) {
          const int64_t o = static_cast<int64_t>(m) * p.ntile_lm + lt;
          p.stat[o * 2] = mx;
          p.stat[o * 2 + 1] = se;
        }
      }
    }
    return;
  }

  if (p.epi == EPI_QKV) {
    // values and RoPE partners first, in a loop small enough to unroll;
    // then the element work, whose calls (pow, sincos) would keep a loop
    // over the accumulators from unrolling (and put them in scratch)
    float xs[CT][4 * MT], os[CT][4 * MT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xs[ct][mt * 4 + j] = acc[mt][ct][j];
          os[ct][mt * 4 + j] = shfl_xor(acc[mt][ct][j], 8);
        }
    for (int ct = 0; ct < CT; ++ct) {
      const int tile = (group * 4 + wave) * CT + ct;
      if (tile >= ntiles) continue;
      const int col = tile_col(p, tile, c);
      const int fi = (col % p.hd) % (p.hd / 2);
      const double inv = pow(static_cast<double>(p.theta),
                             -2.0 * static_cast<double>(fi) / static_cast<double>(p.hd));
      for (int i = 0; i < 4 * MT; ++i)
        qkv_element<T>(p, m0 + (i >> 2) * 16 + 4 * g + (i & 3), col, c, xs[ct][i], os[ct][i], inv);
    }
    return;
  }

#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int tile = (group * 4 + wave) * CT + ct;
    if (tile >= ntiles) continue;
    if (p.epi == EPI_STORE || p.epi == EPI_RESID) {
      float* out = static_cast<float*>(p.out);
      const int col = tile * 16 + c;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + mt * 16 + 4 * g + j;
          float y = acc[mt][ct][j];
          if (m < p.M && p.epi == EPI_RESID) y += p.resid[m * p.ldr + col];
          if (m < p.M) {
            const int64_t orow = p.out_row != nullptr ? p.out_row[m] : m;
            if (orow >= 0) out[orow * p.ldo + col] = y;
          }
          if (p.ss != nullptr) {
            float q = (m < p.M) ? y * y : 0.f;
            q += shfl_xor(q, 1);
            q += shfl_xor(q, 2);
            q += shfl_xor(q, 4);
            q += shfl_xor(q, 8);
            if (c == 0 && m < p.M) p.ss[m * ntiles + tile] = q;
          }
        }
    } else if (p.epi == EPI_SWIGLU) {
      float* out = static_cast<float*>(p.out);
      const int f = 8 * tile + (c & 7);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + mt * 16 + 4 * g + j;
          const float other = shfl_xor(acc[mt][ct][j], 8);
          if (c < 8 && m < p.M) out[m * p.ldo + f] = silu(acc[mt][ct][j]) * other;
        }
    }
  }
}

// ---- split-K: the last workgroup of a tile to arrive sums ---------------
// Partial tiles are written and read with agent-scope atomic (relaxed)
// stores and loads, which the memory model maps to accesses coherent at
// device scope (sc1: written through, read past the XCD's L2), and the
// stores have completed (vmcnt 0) before the arrival counter moves.  A
// device-scope release fence would do the same by writing back the whole
// L2 of the XCD, which costs more than the GEMM.  Returns true in the
// workgroup that arrived last, with acc holding the sum over splits in
// split order; ctr is that tile's arrival counter (left at zero).  lds
// holds at least the 16 MT x 64 CT tile in fp32.
template <int MT, int CT>
__device__ __forceinline__ bool splitk_last(const GemmParams& p, f32x4 (&acc)[MT][CT],
                                            unsigned char* lds, int group, int m0, int split,
                                            int* ctr) {
  __shared__ int last;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int ntiles = p.N / 16;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int tile = (group * 4 + wave) * CT + ct;
    if (tile >= ntiles) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + mt * 16 + 4 * g + j;
        if (m < p.M)
          __hip_atomic_store(p.part + (static_cast<int64_t>(split) * p.Mtot + m) * p.N +
                                 tile * 16 + c,
                             acc[mt][ct][j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == p.S - 1;
    if (last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return false;
  // The last workgroup sums the partials of its 16 MT x 64 CT tile in
  // split order: each thread takes kCh tile elements and reads their
  // partials kSB splits at a time, every load of a batch issued before any
  // is added (addresses clamped into the buffer, so no load sits behind a
  // branch that would make it wait on its own) -- one memory round trip per
  // batch; the sums are staged in LDS and each lane then takes its
  // accumulators back in fragment layout.
  constexpr int kCh = MT >= 4 ? 16 : 4, kSB = 4;
  constexpr int rows = 16 * MT, cols = 64 * CT;
  float* red = reinterpret_cast<float*>(lds);
  const int64_t split_stride = static_cast<int64_t>(p.Mtot) * p.N;
  for (int e0 = threadIdx.x; e0 < rows * cols; e0 += 256 * kCh) {
    float sum[kCh];
    int64_t off[kCh];
    bool ok[kCh];
#pragma unroll
    for (int i = 0; i < kCh; ++i) {
      const int e = e0 + i * 256;
      const int m = m0 + e / cols, col = group * cols + e % cols;
      ok[i] = e < rows * cols && m < p.M && col < p.N;
      off[i] = ok[i] ? static_cast<int64_t>(m) * p.N + col : 0;
      sum[i] = 0.f;
    }
    for (int sp0 = 0; sp0 < p.S; sp0 += kSB) {
      float part[kCh][kSB];
#pragma unroll
      for (int i = 0; i < kCh; ++i)
#pragma unroll
        for (int j = 0; j < kSB; ++j) {
          const int sp = min(sp0 + j, p.S - 1);
          part[i][j] = __hip_atomic_load(p.part + sp * split_stride + off[i], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
      for (int i = 0; i < kCh; ++i)
#pragma unroll
        for (int j = 0; j < kSB; ++j)
          if (sp0 + j < p.S) sum[i] += part[i][j];
    }
#pragma unroll
    for (int i = 0; i < kCh; ++i)
      if (e0 + i * 256 < rows * cols) red[e0 + i * 256] = ok[i] ? sum[i] : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[mt][ct][j] = red[(mt * 16 + 4 * g + j) * cols + (wave * CT + ct) * 16 + c];
  return true;
}

// ---- pipelined A staging (bf16, up to 32 rows) --------------------------
// A piece (PS steps of 128 k for 16 MT rows) is fetched into registers one
// piece ahead: its loads are issued before the weight loads of the piece
// being multiplied, so waiting for them (in-order completion) leaves that
// piece's weight stream in flight.  Each thread always handles the same
// rows.  The segment descriptors and the gathered source row of every
// (row, segment) sit in LDS, where lanes index them freely (indexing the
// kernel arguments or a register array by a per-lane segment would put
// them in memory).
// 16 bytes through a pointer that was read from LDS, as a global load: the
// compiler cannot tell such a pointer's address space and would emit a flat
// load, which also counts against the LDS counter, so that every later wait
// for an LDS read would wait for it and for the weight loads issued before it
__device__ __forceinline__ u32x4 load_global16(const void* ptr) {
  typedef const __attribute__((address_space(1))) u32x4 global_u32x4;
  return *(const global_u32x4*)ptr;
}

// A thread stages the same 8 columns of A (k8 = thread % (16 PS)) in rows
// thread / (16 PS) + j * 256 / (16 PS), j < NG: one gain load serves all rows.
template <int NG>
struct APipe {
  uint32_t raw[NG][8];   // fp32 values, or bf16 pairs in raw[0..3]
  u32x4 gain;            // RMSNorm gain (bf16) of the 8 columns, or ones
};

// What lanes with nothing to stage load instead: 32 zero bytes (values) and
// eight bf16 ones (the gain of columns that are not normalised), so that
// staging needs no masks.
__device__ __attribute__((aligned(64))) uint32_t g_stage_fill[12] = {
    0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};

struct ASegLds {
  const void* base[3];
  int64_t ld[3];
  int f32[3];
  int row[32][3];        // source row per (row of the chunk, segment), -1 = zero
};

template <int MT>
__device__ __forceinline__ void a_tables(const GemmParams& p, ASegLds& t, int m0) {
  const int tid = threadIdx.x;
  if (tid < 3) {
    const ASeg& sg = p.seg[tid < p.nseg ? tid : 0];
    t.base[tid] = sg.base;
    t.ld[tid] = sg.ld;
    t.f32[tid] = sg.f32;
  }
  if (tid < 16 * MT * 3) {
    const int m = tid / 3, si = tid % 3;
    const int row = m0 + m;
    int r = -1;
    if (row < p.M && si < p.nseg) {
      const ASeg& sg = si == 0 ? p.seg[0] : (si == 1 ? p.seg[1] : p.seg[2]);
      r = row;
      if (sg.rowidx != nullptr) {
        r = sg.rowidx[row];
        if (r < 0 || r >= sg.rowlimit) r = -1;
      }
    }
    t.row[m][si] = r;
  }
}

// Every lane issues the same loads whatever its rows, segment or bounds
// (two per row group and the gain; lanes with nothing to load read
// g_stage_fill): with loads under branches the compiler can only count the
// smallest number issued, and the wait for the next weight step would then
// also wait for the A loads issued after it -- draining the weight stream at
// every piece.
template <typename T, int MT, int PS, int NG>
__device__ __forceinline__ void a_fetch(const GemmParams& p, const ASegLds& t, APipe<NG>& ap,
                                        int k0, int kend) {
  constexpr int K8N = PS * 16;
  static_assert(256 % K8N == 0, "a thread keeps its columns across row groups");
  const int tid = threadIdx.x;
  const int w0 = p.seg[0].width, w01 = p.seg[0].width + p.seg[1].width;
  const bool norm0 = p.seg[0].f32 && p.seg[0].ss != nullptr;
  const T* gain0 = static_cast<const T*>(p.seg[0].gain);
  const char* zeros = reinterpret_cast<const char*>(g_stage_fill);
  const int k = k0 + 8 * (tid % K8N);
  const int si = (p.nseg > 1 && k >= w0) ? ((p.nseg > 2 && k >= w01) ? 2 : 1) : 0;
  const int kk = k - (si == 0 ? 0 : (si == 1 ? w0 : w01));
  const bool kin = k < kend;
  const int f32 = t.f32[si];
  const char* base = static_cast<const char*>(t.base[si]);
  const int64_t ld = t.ld[si];
  const int esz = f32 ? 4 : static_cast<int>(sizeof(T));
  const bool gok = kin && si == 0 && norm0;
  ap.gain = load_global16(gok ? static_cast<const void*>(gain0 + kk)
                              : static_cast<const void*>(g_stage_fill + 8));
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int m = tid / K8N + j * (256 / K8N);
    const int r = t.row[m][si];
    const bool ok = kin && r >= 0;
    const char* src = ok ? base + (static_cast<int64_t>(r) * ld + kk) * esz : zeros;
    // bf16 rows hold their 8 values in 16 bytes: the second load repeats it
    const u32x4 x0 = load_global16(src);
    const u32x4 x1 = load_global16(ok && f32 ? src + 16 : src);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ap.raw[j][i] = x0[i];
      ap.raw[j][4 + i] = x1[i];
    }
  }
}

// Stage the fetched piece in LDS: mask, RMSNorm factor and gain, bf16 hi + lo
// split, fragment order.  Selects only, no per-value branches.  Groups past
// the slice hold zeros (their loads were masked), so the padding steps of a
// last, partial piece read zero blocks.  Rows past M are skipped: their
// blocks were zeroed once, before the first piece, with the block after the
// piece (index PS * 4 * MT).  A wave stages one row (PS >= 4), so the skip is
// uniform across it.
template <typename T, int MT, int PS, int NG>
__device__ __forceinline__ void a_store(const GemmParams& p, const ASegLds& t,
                                        const APipe<NG>& ap, unsigned char* lds,
                                        const float* rn, int m0, int k0) {
  constexpr int K8N = PS * 16;
  static_assert(NG * 256 == 16 * MT * K8N, "the groups cover the piece exactly");
  const int tid = threadIdx.x;
  const int w0 = p.seg[0].width, w01 = p.seg[0].width + p.seg[1].width;
  const int k8 = tid % K8N;
  const int st = k8 >> 4, rem = k8 & 15;
  const int g = rem >> 2, e = rem & 3;
  const int k = k0 + 8 * k8;
  const int si = (p.nseg > 1 && k >= w0) ? ((p.nseg > 2 && k >= w01) ? 2 : 1) : 0;
  const bool f32 = t.f32[si] != 0;
  float gn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t gw = ap.gain[i >> 1];
    gn[i] = __uint_as_float((i & 1) ? (gw & 0xffff0000u) : (gw << 16));
  }
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int m = tid / K8N + j * (256 / K8N);
    if (m0 + m >= p.M) continue;
    // the row factor applies to segment 0 only (it is 1 when that segment
    // is not normalised); masked values are zeros, masked gains ones
    const float f = si == 0 ? rn[m] : 1.f;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t w = ap.raw[j][i >> 1];
      const float vb = __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
      v[i] = (f32 ? __uint_as_float(ap.raw[j][i]) : vb) * f * gn[i];
    }
    const int mt = m >> 4, c = m & 15;
    const int lane = g * 16 + c;
    unsigned char* blk = lds + static_cast<size_t>((st * 4 + e) * MT + mt) * kBlk;
    u32x4 hi, lo;
    split_hi_lo(v, hi, lo);
    *reinterpret_cast<u32x4*>(blk + lane * 16) = hi;
    *reinterpret_cast<u32x4*>(blk + 1024 + lane * 16) = lo;
  }
}

template <typename T, int MT, int CT, int PS>
__global__ __launch_bounds__(256) void stream_gemm_kernel(GemmParams p) {
  // weight steps in flight per wave; a piece of PS steps is fully unrolled,
  // so buffer (s % PF) always holds step s of the piece
  constexpr int PF = PS < kPF ? PS : kPF;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ntiles = p.N / 16;
  const int group = blockIdx.x / p.S;
  const int split = blockIdx.x % p.S;
  const int m0 = blockIdx.z * (16 * MT);
  const int ksteps = (p.K + kStep - 1) / kStep;
  const int st0 = split * (p.KS / kStep);
  const int nsteps = min(p.KS / kStep, ksteps - st0);
  const int kend = min(p.K, st0 * kStep + p.KS);

  // ---- per-lane weight fragments in the packed layout (inactive tiles read
  // tile 0 and are dropped) ----
  const T* wtile[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int tile = (group * 4 + wave) * CT + ct;
    wtile[ct] = static_cast<const T*>(p.wpack) +
                static_cast<int64_t>(tile < ntiles ? tile : 0) * 4 * kPackBlk + lane * 8;
  }
  // weight fragments of step st (clamped into the slice): one fully
  // coalesced 1 KB (bf16) load per wave and fragment
  const int64_t step_stride = static_cast<int64_t>(ntiles) * 4 * kPackBlk;
  auto load_w = [&](int st, Frag8<T>(&wf)[CT][4]) {
    const int sc = min(st, st0 + nsteps - 1);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e) wf[ct][e].load_nt(wtile[ct] + sc * step_stride + e * kPackBlk);
  };

  // order of the first loads: the row factors and the gathered rows, then
  // the first piece of A, then the first PF steps of weights -- waiting for
  // the A loads when staging them (in-order completion) leaves the weights
  // in flight
  __shared__ float rn[16 * MT];
  row_factors<MT>(p, rn, m0);
  constexpr bool kPipe = sizeof(T) == 2 && MT <= 2;
  constexpr int NG = kPipe ? (MT * 16 * PS * 16 + 255) / 256 : 1;
  APipe<NG> ap;
  __shared__ ASegLds at;
  if constexpr (kPipe) {
    a_tables<MT>(p, at, m0);
    // every block zero once: rows past M are never staged, and the block
    // after the piece is the one padding steps read
    for (int i = threadIdx.x; i < (PS * 4 * MT + 1) * kBlk / 16; i += 256)
      *reinterpret_cast<u32x4*>(lds + i * 16) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    a_fetch<T, MT, PS, NG>(p, at, ap, st0 * kStep, kend);
  }
  __syncthreads();

  Frag8<T> wb[PF][CT][4];
#pragma unroll
  for (int i = 0; i < PF; ++i) load_w(st0 + i, wb[i]);
  __builtin_amdgcn_sched_barrier(0);

  f32x4 acc[MT][CT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ps0 = 0; ps0 < nsteps; ps0 += PS) {
    const int np = min(PS, nsteps - ps0);
    if (ps0 > 0) __syncthreads();  // every wave is done with the last piece
    if constexpr (kPipe) {
      a_store<T, MT, PS, NG>(p, at, ap, lds, rn, m0, (st0 + ps0) * kStep);
      __syncthreads();
      // the next piece's A, ahead of this piece's weight refills; issued
      // after the last piece too (every lane then reads the dummy address),
      // so that the number of loads in flight is the same on every path and
      // the waits for the weights below count past these loads
      a_fetch<T, MT, PS, NG>(p, at, ap, (st0 + ps0 + PS) * kStep, kend);
      __builtin_amdgcn_sched_barrier(0);
    } else {
      fill_a<T, MT>(p, lds, rn, m0, (st0 + ps0) * kStep, kend, np);
      __syncthreads();
    }
    const int zero_blk = (kPipe ? PS : np) * 4 * MT;
#pragma unroll
    for (int s = 0; s < PS; ++s) {
      const int i = s % PF;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int blk = s < np ? (s * 4 + e) * MT + mt : zero_blk;
          const unsigned char* ap = lds + static_cast<size_t>(blk) * kBlk;
          if constexpr (sizeof(T) == 2) {
            Frag8<uint16_t> ah, al;
            ah.v = *reinterpret_cast<const u32x4*>(ap + lane * 16);
            al.v = *reinterpret_cast<const u32x4*>(ap + 1024 + lane * 16);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              acc[mt][ct] = mfma16(ah, wb[i][ct][e], acc[mt][ct]);
              acc[mt][ct] = mfma16(al, wb[i][ct][e], acc[mt][ct]);
            }
          } else {
            Frag8<float> af;
            af.a = *reinterpret_cast<const f32x4*>(ap + lane * 32);
            af.b = *reinterpret_cast<const f32x4*>(ap + lane * 32 + 16);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
              acc[mt][ct] = mfma16(af, wb[i][ct][e], acc[mt][ct]);
          }
        }
      }
      // refill this buffer right after its last use: keep the compiler from
      // sinking the loads, which would shorten the stream in flight
      __builtin_amdgcn_sched_barrier(0);
      load_w(st0 + ps0 + s + PF, wb[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (p.S > 1) {
    const int ngroups = (ntiles + 4 * CT - 1) / (4 * CT);
    if (!splitk_last<MT, CT>(p, acc, lds, group, m0, split,
                             p.cnt + blockIdx.z * ngroups + group))
      return;
  }
  epilogue<T, MT, CT>(p, acc, lds, group, m0);
}

// ============================================================================
// Dense path: more than 64 rows (a batch of trees) makes the product a dense
// contraction, bound by the matrix cores.  A is normalised and split into
// bf16 hi/lo fragments once per launch (pack_a_kernel); then each workgroup
// computes a 64-row x 256-column tile: its four waves share the A tile,
// double-buffered in LDS one 128-wide k step at a time, and each wave reads
// its own 64 columns of packed weights straight into registers, the next
// step's fragments loaded as the current ones retire.  Workgroups that share
// a column block are numbered so that they land on the same XCD (dispatch
// goes round-robin over the 8 XCDs) and reuse its L2 copy of the weights.
// ============================================================================
constexpr int kDenseABytes = 16 * kBlk;  // A bytes of one step of a 64-row block

// One 128-wide k step of a 64-row block per workgroup: each thread takes
// four 8-element groups (rows tid / 16 + 16 i, columns 8 (tid % 16)).  The
// values and the gain are requested first, the row factors (from the
// producer's partial sums of squares) meanwhile, so a workgroup waits for
// memory about once.
template <typename T>
__global__ __launch_bounds__(256) void pack_a_kernel(GemmParams p) {
  __shared__ float rn[64];
  const int m0 = blockIdx.x * 64;
  const int ksteps = (p.K + kStep - 1) / kStep;
  const int s = blockIdx.y;
  const int k8 = threadIdx.x & 15;
  const int g = k8 >> 2, e = k8 & 3;
  const int k = (s * 16 + k8) * 8;
  const ASeg& s0 = p.seg[0];
  const bool norm = s0.f32 && s0.ss != nullptr && k < s0.width && k < p.K;
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = (threadIdx.x >> 4) + 16 * i;
    a_raw_values<T>(p, m0 + m, k, p.K, v[i]);
  }
  Frag8<T> gv;
  if (norm) gv.load(static_cast<const T*>(s0.gain) + k);
  row_factors<4>(p, rn, m0);
  __syncthreads();
  unsigned char* out = static_cast<unsigned char*>(p.apack);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = (threadIdx.x >> 4) + 16 * i;
    if (norm) {
      const float f = rn[m];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = v[i][j] * f * gv.get(j);
    }
    const int rt = (m0 >> 4) + (m >> 4), c = m & 15;
    unsigned char* blk = out + ((static_cast<int64_t>(rt) * ksteps + s) * 4 + e) * kBlk;
    u32x4 hi, lo;
    split_hi_lo(v[i], hi, lo);
    *reinterpret_cast<u32x4*>(blk + (g * 16 + c) * 16) = hi;
    *reinterpret_cast<u32x4*>(blk + 1024 + (g * 16 + c) * 16) = lo;
  }
}

template <typename T, int CT>
__global__ __launch_bounds__(256) void dense_gemm_kernel(GemmParams p) {
  constexpr int MT = 4;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ntiles = p.N / 16;
  const int ngroups = (ntiles + 4 * CT - 1) / (4 * CT);
  const int RB = (p.M + 63) / 64;
  const int ntask = RB * ngroups * p.S;
  const int per_xcd = (ntask + 7) / 8;
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= ntask) return;
  const int rb = t % RB;
  const int split = (t / RB) % p.S;
  const int group = t / (RB * p.S);
  const int m0 = rb * 64;
  const int ksteps = (p.K + kStep - 1) / kStep;
  const int st0 = split * (p.KS / kStep);
  const int nsteps = min(p.KS / kStep, ksteps - st0);

  const T* wtile[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int tile = (group * 4 + wave) * CT + ct;
    wtile[ct] = static_cast<const T*>(p.wpack) +
                static_cast<int64_t>(tile < ntiles ? tile : 0) * 4 * kPackBlk + lane * 8;
  }
  const int64_t step_stride = static_cast<int64_t>(ntiles) * 4 * kPackBlk;
  // the block's four row tiles lie ksteps * 8 KB apart in the packed A
  const unsigned char* abase = static_cast<const unsigned char*>(p.apack) +
                               static_cast<int64_t>(rb) * 4 * ksteps * (4 * kBlk);
  u32x4 ar[8];
  auto load_a = [&](int st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = (i * 256 + static_cast<int>(threadIdx.x)) * 16;
      const int rt = o >> 13, w = o & 8191;
      ar[i] = *reinterpret_cast<const u32x4*>(
          abase + (static_cast<int64_t>(rt) * ksteps + st) * (4 * kBlk) + w);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int o = (i * 256 + static_cast<int>(threadIdx.x)) * 16;
      const int rt = o >> 13, w = o & 8191;
      const int e = w >> 11, inb = w & 2047;
      *reinterpret_cast<u32x4*>(lds + buf * kDenseABytes + ((e * 4 + rt) << 11) + inb) = ar[i];
    }
  };

  Frag8<T> wb[CT][4];
  load_a(st0);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) wb[ct][e].load(wtile[ct] + st0 * step_stride + e * kPackBlk);
  f32x4 acc[MT][CT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[mt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  store_a(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    const int nst = st0 + (more ? s + 1 : s);
    if (more) load_a(nst);
    const unsigned char* ab = lds + (s & 1) * kDenseABytes;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Frag8<uint16_t> ah, al;
        ah.v = *reinterpret_cast<const u32x4*>(ab + ((e * 4 + mt) << 11) + lane * 16);
        al.v = *reinterpret_cast<const u32x4*>(ab + ((e * 4 + mt) << 11) + 1024 + lane * 16);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          acc[mt][ct] = mfma16(ah, wb[ct][e], acc[mt][ct]);
          acc[mt][ct] = mfma16(al, wb[ct][e], acc[mt][ct]);
        }
      }
      // the next step's fragments of sub-step e replace the retired ones
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) wb[ct][e].load(wtile[ct] + nst * step_stride + e * kPackBlk);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (more) store_a((s + 1) & 1);
    __syncthreads();
  }

  if (p.S > 1 &&
      !splitk_last<MT, CT>(p, acc, lds, group, m0, split, p.cnt + rb * ngroups + group))
    return;
  epilogue<T, MT, CT>(p, acc, lds, group, m0);
}

template <typename T>
__global__ __launch_bounds__(256) void pack_weights_kernel(GemmParams p, T* dst) {
  const int ksteps = (p.K + kStep - 1) / kStep;
  const int tile = blockIdx.x / ksteps, st = blockIdx.x % ksteps;
  const int e = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int g = lane >> 4, c = lane & 15;
  const int k = st * kStep + g * 32 + e * 8;
  Frag8<T> v;
  if (k < p.K) v.load(weight_row<T>(p, tile, c) + k); else v.zero();
  const int ntiles = p.N / 16;
  T* out = dst + ((static_cast<int64_t>(st) * ntiles + tile) * 4 + e) * kPackBlk + lane * 8;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<u32x4*>(out) = v.v;
  } else {
    *reinterpret_cast<f32x4*>(out) = v.a;
    *reinterpret_cast<f32x4*>(out + 4) = v.b;
  }
}

int64_t packed_elems(int N, int K) {
  return static_cast<int64_t>(N) * ((K + kStep - 1) / kStep) * kStep;
}

template <typename T>
hipError_t launch_pack(const GemmParams& p, void* dst, hipStream_t s) {
  if (p.N % 16 || p.K % 8 || p.K < 8) return hipErrorInvalidValue;
  const int64_t blocks = static_cast<int64_t>(p.N / 16) * ((p.K + kStep - 1) / kStep);
  hipLaunchKernelGGL(pack_weights_kernel<T>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     p, static_cast<T*>(dst));
  return hipGetLastError();
}
template hipError_t launch_pack<uint16_t>(const GemmParams&, void*, hipStream_t);
template hipError_t launch_pack<float>(const GemmParams&, void*, hipStream_t);

namespace {

size_t lds_bytes(int MT, int steps) { return static_cast<size_t>(steps * 4 * MT + 1) * kBlk; }
// most k steps of A one LDS piece holds (34 KB, 66 KB and 130 KB of LDS for
// 1, 2 and 4 row tiles): longer pieces measured slower at one row tile
constexpr int kMaxPiece = 4;

}  // namespace

void plan_gemm(GemmParams& p, int num_cus, bool fp32) {
  const int ntiles = p.N / 16;
  p.dense = !fp32 && p.M > 64 && p.apack != nullptr && p.M <= p.apack_rows;
  if (p.dense) {
    // 64 x 256 tiles (four 16-column tiles per wave).  K is split only when
    // it is long (64 steps and more; a split costs a round of partial sums
    // through memory, more than a few steps of the main loop): into as many
    // splits of at least 8 steps as keep the grid within two tiles per CU and
    // the partial sums within their buffer.  Shorter K is not split, and
    // takes 64 x 128 tiles when 64 x 256 ones would not give every CU two
    // workgroups (measured: 64 x 256 tiles with split K do better for long K,
    // worse for short K, where the split's partial sums weigh more)
    const int RB = (p.M + 63) / 64;
    const int ksteps = (p.K + kStep - 1) / kStep;
    const bool longk = ksteps >= 64;
    p.MT = 4;
    p.CT = (!longk && RB * ((ntiles + 15) / 16) < 2 * num_cus) ? 2 : 4;
    const int ngroups = (ntiles + 4 * p.CT - 1) / (4 * p.CT);
    int S = 1;
    if (longk)
      while (ksteps / (S + 1) >= 8 && RB * ngroups * (S + 1) <= 2 * num_cus && S < 16 &&
             static_cast<int64_t>(S + 1) * p.Mtot * p.N <= p.part_elems)
        ++S;
    const int steps = (ksteps + S - 1) / S;
    p.KS = steps * kStep;
    p.S = (ksteps + steps - 1) / steps;
    p.piece_steps = 2;
    return;
  }
  const int rows = p.M < 64 ? p.M : 64;
  p.MT = rows <= 16 ? 1 : (rows <= 32 ? 2 : 4);
  const int chunks = (p.M + 16 * p.MT - 1) / (16 * p.MT);
  // one 16-column tile per wave; two (bf16 only: fp32 fragments take twice
  // the registers) when there are far more tiles than the chip holds, and
  // for the wide gate/up product at one row tile: at 8B (1792 tiles) it
  // streams 5% faster as 224 workgroups of two tiles per wave than as 448 of
  // one.  Measured no gain for the LM head (2000 tiles), and a 20% loss for
  // the narrower products, which then need more K splits.
  p.CT = (!fp32 && (ntiles >= 16 * num_cus ||
                    (p.M <= 16 && ntiles >= 4 * num_cus && p.epi == EPI_SWIGLU)))
             ? 2 : 1;
  const int ngroups = (ntiles + 4 * p.CT - 1) / (4 * p.CT);
  const int ksteps = (p.K + kStep - 1) / kStep;
  // no K split when the column groups alone cover every CU; else split K
  // until the grid holds about one workgroup per CU (each split's partial
  // sums cost a round trip through memory, so fewer, longer splits do
  // better than more workgroups), each split keeping at least two steps
  int S = 1;
  if (ngroups * chunks < num_cus)
    while (ngroups * chunks * S < num_cus && (ksteps + S) / (S + 1) >= 2 && S < 16) ++S;
  // a grid a little over one workgroup per CU keeps most CUs idle while the
  // excess runs: one split fewer when that still covers 3/4 of the CUs
  const int tiles_s = ngroups * chunks;
  if (S > 1 && tiles_s * S > num_cus && 4 * tiles_s * (S - 1) >= 3 * num_cus) --S;
  // the partial sums must fit the workspace
  while (S > 1 && static_cast<int64_t>(S) * p.Mtot * p.N > p.part_elems) --S;
  // a split longer than 4 steps is rounded up to whole pieces (fewer,
  // longer splits): steps past the slice still stream their weights, against
  // zero A, so a ragged piece costs bandwidth
  int steps = (ksteps + S - 1) / S;
  if (steps > kMaxPiece) steps = (steps + kMaxPiece - 1) / kMaxPiece * kMaxPiece;
  p.KS = steps * kStep;
  p.S = (ksteps + steps - 1) / steps;
  // smallest unrolled piece that holds the slice (several pieces otherwise)
  p.piece_steps = steps <= 2 ? 2 : kMaxPiece;
}

namespace {

template <typename T, int MT, int CT, int PS>
hipError_t launch_one(const GemmParams& p, hipStream_t s) {
  const int ntiles = p.N / 16;
  const int ngroups = (ntiles + 4 * CT - 1) / (4 * CT);
  const int chunks = (p.M + 16 * MT - 1) / (16 * MT);
  size_t lds = lds_bytes(MT, PS);
  const size_t tile_bytes = static_cast<size_t>(16 * MT) * 64 * CT * 4;
  if (lds < tile_bytes) lds = tile_bytes;
  if (lds > static_cast<size_t>(kLdsCap)) return hipErrorInvalidValue;
  auto kern = stream_gemm_kernel<T, MT, CT, PS>;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, kLdsCap);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(ngroups * p.S, 1, chunks), dim3(256), lds, s, p);
  return hipGetLastError();
}

template <typename T, int MT, int CT>
hipError_t launch_ps(const GemmParams& p, hipStream_t s) {
  switch (p.piece_steps) {
    case 2: return launch_one<T, MT, CT, 2>(p, s);
    case kMaxPiece: return launch_one<T, MT, CT, kMaxPiece>(p, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int MT>
hipError_t launch_mt(const GemmParams& p, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (p.CT == 2) return launch_ps<T, MT, 2>(p, s);
  }
  return launch_ps<T, MT, 1>(p, s);
}

}  // namespace

template <typename T, int CT>
hipError_t launch_dense_ct(const GemmParams& p, hipStream_t s) {
  const int RB = (p.M + 63) / 64;
  const int ngroups = (p.N / 16 + 4 * CT - 1) / (4 * CT);
  const int ntask = RB * ngroups * p.S;
  auto kern = dense_gemm_kernel<T, CT>;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             2 * kDenseABytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((ntask + 7) / 8 * 8), dim3(256), 2 * kDenseABytes, s, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dense(const GemmParams& p, hipStream_t s) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorInvalidValue;
  } else {
    const int RB = (p.M + 63) / 64;
    const int ksteps = (p.K + kStep - 1) / kStep;
    hipLaunchKernelGGL(pack_a_kernel<T>, dim3(RB, ksteps), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return p.CT == 2 ? launch_dense_ct<T, 2>(p, s) : launch_dense_ct<T, 4>(p, s);
  }
}

template <typename T>
hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  if (p.dense) {
    if (p.N % 16 || p.K % 8 || p.K < 8 || p.KS % kStep || p.S < 1 || p.MT != 4 ||
        (p.CT != 4 && p.CT != 2) || static_cast<int64_t>(p.S) * p.KS < p.K ||
        p.M > p.apack_rows ||
        (p.S > 1 && (p.part == nullptr || p.cnt == nullptr ||
                     static_cast<int64_t>(p.S) * p.Mtot * p.N > p.part_elems)) ||
        p.wpack == nullptr || p.apack == nullptr)
      return hipErrorInvalidValue;
    return launch_dense<T>(p, s);
  }
  if (p.N % 16 || p.K % 8 || p.K < 8 || p.KS % kStep || p.S < 1 ||
      static_cast<int64_t>(p.S) * p.KS < p.K ||
      (p.S > 1 && (p.part == nullptr || p.cnt == nullptr)) ||
      (p.CT == 2 && sizeof(T) != 2) || p.wpack == nullptr)
    return hipErrorInvalidValue;
  // a split either fits one piece or spans whole pieces of kMaxPiece steps
  if (p.KS / kStep > p.piece_steps && p.piece_steps < 4) return hipErrorInvalidValue;
  switch (p.MT) {
    case 1: return launch_mt<T, 1>(p, s);
    case 2: return launch_mt<T, 2>(p, s);
    default: return launch_mt<T, 4>(p, s);
  }
}

template hipError_t launch_gemm<uint16_t>(const GemmParams&, hipStream_t);
template hipError_t launch_gemm<float>(const GemmParams&, hipStream_t);

}  // namespace eagle
