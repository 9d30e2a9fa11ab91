// Skinny MFMA GEMM for the draft path: C[M, N] = A[M, K] * W[N, K]^T with
// M <= 64 rows per grid.z chunk (bs1 trees: M = 1..16).  At these shapes the
// op is a weight stream from HBM, so the kernel is organised around the
// weight reads:
//  * each wave owns 16 output columns; every lane reads 64 contiguous bytes
//    of one weight row per 128-wide k step (4 x 16-byte loads), and the k
//    order inside a step is permuted identically for A and W so each 16x16x32
//    MFMA consumes exactly what the lane loaded;
//  * the next step's loads are issued before the current step's MFMAs;
//  * waves of a workgroup split K (WK) or N (WN), and S workgroups split K
//    further; partial sums go to a workspace and the last-arriving workgroup
//    of a column group sums them in a fixed order (deterministic) and runs the
//    fused epilogue;
//  * the RMSNorm of the A operand is applied on load (factor per row computed
//    by the producing GEMM's last workgroup), so no separate norm kernel runs.
#include "common.hpp"
#include "kernels.hpp"

namespace eagle {

namespace {

constexpr int kStep = 128;  // k elements per wave step (4 lane groups x 32)

struct ARow {
  const void* ptr[3];
  float r[3];
};

// A fragment for k in [k, k+8): float activation segments are normalised on
// load (RMSNorm factor r and gain) and split for bf16 weights; weight-type
// segments (embedding rows, target taps) load as they are.
template <typename TW>
__device__ __forceinline__ void load_a(const GemmParams& p, const ARow& ar,
                                       int k, AFrag<TW>& f) {
  int s = 0, base = 0;
  if (p.nseg > 1 && k >= p.seg[0].width) {
    base = p.seg[0].width;
    s = 1;
    if (p.nseg > 2 && k >= base + p.seg[1].width) {
      base += p.seg[1].width;
      s = 2;
    }
  }
  const ASeg& sg = s == 0 ? p.seg[0] : (s == 1 ? p.seg[1] : p.seg[2]);
  const void* rp = s == 0 ? ar.ptr[0] : (s == 1 ? ar.ptr[1] : ar.ptr[2]);
  if (rp == nullptr) {
    f.zero();
    return;
  }
  const int kk = k - base;
  if (sg.f32) {
    Frag8<float> x;
    x.load(static_cast<const float*>(rp) + kk);
    if (sg.rnorm != nullptr) {
      Frag8<TW> gf;
      gf.load(static_cast<const TW*>(sg.gain) + kk);
      const float r = s == 0 ? ar.r[0] : (s == 1 ? ar.r[1] : ar.r[2]);
#pragma unroll
      for (int i = 0; i < 8; ++i) x.set(i, x.get(i) * r * gf.get(i));
    }
    f.from_float(x);
  } else {
    Frag8<TW> w;
    w.load(static_cast<const TW*>(rp) + kk);
    f.from_raw(w);
  }
}

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
__device__ __forceinline__ const T* weight_row(const GemmParams& p, int tile,
                                               int c) {
  const int col = tile_col(p, tile, c);
  const int64_t K = p.K;
  if (p.colmap == MAP_QKV) {
    if (col < p.qkv_n0) return static_cast<const T*>(p.w0) + col * K;
    if (col < p.qkv_n0 + p.qkv_n1)
      return static_cast<const T*>(p.w1) + (col - p.qkv_n0) * K;
    return static_cast<const T*>(p.w2) + (col - p.qkv_n0 - p.qkv_n1) * K;
  }
  if (p.colmap == MAP_SWIGLU)
    return static_cast<const T*>(c < 8 ? p.w0 : p.w1) + col * K;
  return static_cast<const T*>(p.w0) + col * K;
}

__device__ __forceinline__ float silu(float x) { return x / (1.f + expf(-x)); }

}  // namespace

template <typename T, int MT>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(GemmParams p) {
  __shared__ float red[4 * 4 * 64 * 4];   // WK partial tiles / LM-head tile
  __shared__ int flag;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int wn = wave % p.WN, wk = wave / p.WN;
  const int ntiles = p.N / 16;
  const int ngroups = (ntiles + p.WN - 1) / p.WN;
  const int group = blockIdx.x / p.S;
  const int split = blockIdx.x % p.S;
  const int tile = group * p.WN + wn;
  const bool active = tile < ntiles;
  const int m0 = blockIdx.z * 64;

  // ---- per-lane A rows and W row -------------------------------------------
  ARow ar[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + mt * 16 + c;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
      ar[mt].ptr[s] = nullptr;
      ar[mt].r[s] = 1.f;
      if (s < p.nseg && m < p.M) {
        const ASeg& sg = p.seg[s];
        int row = m;
        if (sg.rowidx != nullptr) {
          row = sg.rowidx[m];
          if (row < 0 || row >= sg.rowlimit) row = -1;
        }
        if (row >= 0) {
          const int64_t off = static_cast<int64_t>(row) * sg.ld;
          ar[mt].ptr[s] = sg.f32 ? static_cast<const void*>(static_cast<const float*>(sg.base) + off)
                                 : static_cast<const void*>(static_cast<const T*>(sg.base) + off);
          if (sg.rnorm != nullptr) ar[mt].r[s] = sg.rnorm[m];
        }
      }
    }
  }
  const T* wrow = active ? weight_row<T>(p, tile, c) : nullptr;

  // ---- K loop ----------------------------------------------------------------
  const int steps = (p.K + kStep - 1) / kStep;
  const int nworkers = p.S * p.WK;
  const int worker = split * p.WK + wk;
  const int st0 = static_cast<int>((static_cast<int64_t>(worker) * steps) / nworkers);
  const int st1 = static_cast<int>((static_cast<int64_t>(worker + 1) * steps) / nworkers);

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weights are double-buffered (the HBM stream); activation fragments come
  // from L2 and are loaded per step
  Frag8<T> wa[4], wb[4];
  auto load_w = [&](int st, Frag8<T>(&wf)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = st * kStep + g * 32 + e * 8;
      if (active && k < p.K) wf[e].load(wrow + k); else wf[e].zero();
    }
  };
  auto step = [&](int st, const Frag8<T>(&wf)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k = st * kStep + g * 32 + e * 8;
      const bool ok = active && k < p.K;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        AFrag<T> af;
        if (ok) load_a<T>(p, ar[mt], k, af); else af.zero();
        acc[mt] = mfma16(af.hi, wf[e], acc[mt]);
        if constexpr (sizeof(T) == 2) {
          if (p.a_lo) acc[mt] = mfma16(af.lo, wf[e], acc[mt]);
        }
      }
    }
  };

  if (st0 < st1) load_w(st0, wa);
  for (int st = st0; st < st1; st += 2) {
    if (st + 1 < st1) load_w(st + 1, wb);
    step(st, wa);
    if (st + 2 < st1) load_w(st + 2, wa);
    if (st + 1 < st1) step(st + 1, wb);
  }

  // ---- reduce the WK waves of this workgroup ---------------------------------
  if (p.WK > 1) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        red[(((wk * p.WN + wn) * MT + mt) * 64 + lane) * 4 + j] = acc[mt][j];
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float s = 0.f;
          for (int w = 0; w < p.WK; ++w)
            s += red[(((w * p.WN + wn) * MT + mt) * 64 + lane) * 4 + j];
          acc[mt][j] = s;
        }
    }
    __syncthreads();
  }

  // ---- split-K across workgroups: last arrival finishes -----------------------
  if (p.S > 1) {
    if (wk == 0 && active) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + mt * 16 + 4 * g + j;
          if (m < p.M)
            p.part[(static_cast<int64_t>(split) * p.Mtot + m) * p.N + tile * 16 + c] =
                acc[mt][j];
        }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      int* ctr = p.cnt + blockIdx.z * ngroups + group;
      const int prev = atomicAdd(ctr, 1);
      flag = (prev == p.S - 1);
      if (flag) atomicExch(ctr, 0);
    }
    __syncthreads();
    if (!flag) return;
    __threadfence();
    if (wk == 0 && active) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + mt * 16 + 4 * g + j;
          float s = 0.f;
          if (m < p.M) {
            for (int sp = 0; sp < p.S; ++sp)
              s += __builtin_nontemporal_load(
                  p.part + (static_cast<int64_t>(sp) * p.Mtot + m) * p.N + tile * 16 + c);
          }
          acc[mt][j] = s;
        }
    }
  }

  // ---- epilogues ---------------------------------------------------------------
  if (p.epi == EPI_LMHEAD) {
    // WN == 4, WK == 1: the workgroup holds 64 consecutive vocabulary columns
    float* lm = red;  // [64 rows][64 cols]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        lm[(mt * 16 + 4 * g + j) * 64 + wn * 16 + c] = acc[mt][j];
    __syncthreads();
    const int rows = min(64, p.M - m0);
    const int col = group * 64 + lane;
    for (int r = wave; r < rows; r += 4) {
      float v = col < p.N ? lm[r * 64 + lane] : -INFINITY;
      if (v != v) v = -INFINITY;
      int id = col < p.N ? col : 0x7fffffff;
      const float mx = wave_max(v);
      const float se = wave_sum(v == -INFINITY ? 0.f : expf(v - mx));
      wave_sort_desc(v, id);
      const int m = m0 + r;
      const int64_t o = static_cast<int64_t>(m) * p.ntile_lm + group;
      if (lane < p.topk) {
        p.cand_val[o * p.topk + lane] = v;
        p.cand_id[o * p.topk + lane] = id;
      }
      if (lane == 0) {
        p.stat[o * 2] = mx;
        p.stat[o * 2 + 1] = se;
      }
    }
    return;
  }

  if (wk == 0 && active) {
    if (p.epi == EPI_STORE || p.epi == EPI_RESID) {
      float* out = static_cast<float*>(p.out);
      const int col = tile * 16 + c;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + mt * 16 + 4 * g + j;
          float y = acc[mt][j];
          if (m < p.M && p.epi == EPI_RESID) y += p.resid[m * p.ldr + col];
          if (m < p.M) out[m * p.ldo + col] = y;
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
          const float other = shfl_xor(acc[mt][j], 8);
          if (c < 8 && m < p.M)
            out[m * p.ldo + f] = silu(acc[mt][j]) * other;
        }
    } else if (p.epi == EPI_QKV) {
      const int col = tile_col(p, tile, c);
      const int hh = col / p.hd, cin = col % p.hd;
      const int half = p.hd / 2;
      const bool rot = hh < p.nq + p.nkv;
      const int fi = cin % half;
      const double inv = pow(static_cast<double>(p.theta),
                             -2.0 * static_cast<double>(fi) / static_cast<double>(p.hd));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int m = m0 + mt * 16 + 4 * g + j;
          const float x = acc[mt][j];
          const float other = shfl_xor(x, 8);
          if (m >= p.M || p.tok[m] < 0) continue;
          float y = x;
          if (rot) {
            double sd, cd;
            sincos(static_cast<double>(p.pos[m]) * inv, &sd, &cd);
            const float cs = static_cast<float>(cd), sn = static_cast<float>(sd);
            y = (c < 8) ? (x * cs - other * sn) : (x * cs + other * sn);
          }
          const T v = Elem<T>::from_f(y);
          if (hh < p.nq) {
            static_cast<T*>(p.out)[m * p.ldo + col] = v;
          } else {
            const int b = m / p.rows_per_seq;
            const int d = p.dest[m];
            if (b >= p.batch || d < 0 || d >= p.cap) {
              if (p.status != nullptr) atomicOr(p.status, 1 << 4);
              continue;
            }
            const bool isk = hh < p.nq + p.nkv;
            const int kvh = isk ? hh - p.nq : hh - p.nq - p.nkv;
            T* cache = static_cast<T*>(isk ? p.kc : p.vc);
            cache[((static_cast<int64_t>(b) * p.nkv + kvh) * p.cap + d) * p.hd + cin] = v;
          }
        }
    }
  }

  // ---- last finishing group of the chunk computes the RMSNorm factors ------
  if (p.ss != nullptr && p.rnorm_out != nullptr) {
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const int prev = atomicAdd(p.done + blockIdx.z, 1);
      flag = (prev == ngroups - 1);
      if (flag) atomicExch(p.done + blockIdx.z, 0);
    }
    __syncthreads();
    if (!flag) return;
    __threadfence();
    const int rows = min(64, p.M - m0);
    for (int r = wave; r < rows; r += 4) {
      const int m = m0 + r;
      float s = 0.f;
      for (int t = lane; t < ntiles; t += 64)
        s += __builtin_nontemporal_load(p.ss + m * ntiles + t);
      s = wave_sum(s);
      if (lane == 0) p.rnorm_out[m] = 1.f / sqrtf(s / static_cast<float>(p.N) + p.eps);
    }
  }
}

void plan_gemm(GemmParams& p, int num_cus) {
  const int ntiles = p.N / 16;
  const int chunks = (p.M + 63) / 64;
  if (p.epi == EPI_LMHEAD) {
    p.WN = 4;
    p.WK = 1;
    p.S = 1;
    return;
  }
  p.WN = 1;
  p.WK = 4;
  const int steps = (p.K + kStep - 1) / kStep;
  const int want_waves = 16 * num_cus;
  int S = want_waves / (ntiles * p.WK * chunks);
  S = S < 1 ? 1 : (S > 8 ? 8 : S);
  while (S > 1 && S * p.WK > steps) --S;
  while (S > 1 && S * p.N > p.part_cols) --S;
  if (p.WK > steps) p.WK = steps < 1 ? 1 : (steps >= 4 ? 4 : (steps >= 2 ? 2 : 1));
  p.S = S;
}

template <typename T>
hipError_t launch_gemm(const GemmParams& p, hipStream_t s) {
  const int ntiles = p.N / 16;
  const int ngroups = (ntiles + p.WN - 1) / p.WN;
  const int chunks = (p.M + 63) / 64;
  const int mt = chunks > 1 ? 4 : (p.M + 15) / 16;
  dim3 grid(ngroups * p.S, 1, chunks);
  dim3 block(256);
  switch (mt) {
    case 1: hipLaunchKernelGGL((skinny_gemm_kernel<T, 1>), grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL((skinny_gemm_kernel<T, 2>), grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL((skinny_gemm_kernel<T, 3>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((skinny_gemm_kernel<T, 4>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

template hipError_t launch_gemm<uint16_t>(const GemmParams&, hipStream_t);
template hipError_t launch_gemm<float>(const GemmParams&, hipStream_t);

}  // namespace eagle
