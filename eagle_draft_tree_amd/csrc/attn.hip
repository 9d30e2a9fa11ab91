// Tree attention of the draft layer (split-KV, "flash decoding" style).
//
// The query vectors of a sequence that share a kv head (rows_per_seq rows x
// G grouped heads, at most 128) are the MFMA columns.  Every wave owns one
// key range (a split) and up to QBW blocks of 16 query vectors, and runs the
// online softmax over its keys with the state in registers:
//  * S^T = K Q^T: K rows are read straight from the cache as MFMA A
//    fragments (lane (g, c): key c, 32 contiguous dims), Q as B fragments
//    with the same dim permutation; lane (g, c) ends up holding keys
//    4g + i of query column c;
//  * O^T += V^T P^T: the V cache is stored transposed ([hd, cap] per head),
//    so lane (g, c) reads its 8 keys of dim c as two 4-key runs -- exactly
//    the keys whose probabilities it already holds, which makes them the B
//    fragment with no data movement.  In bf16, P is carried as hi + lo bf16
//    parts, so o keeps float precision;
//  * visibility: cache rows [0, prefix_len) of the query's row (prefix
//    splits) and scratch rows scratch_base + j for the set bits j of the
//    row's 64-bit ancestor mask (the last split).
// Keys are visited 32 at a time, which keeps a wave within 256 registers.
// Each wave writes its (max, sum, O) per query vector; a second kernel
// merges the splits in split order.  No workgroup waits on another.
#include "common.hpp"
#include "kernels.hpp"

namespace eagle {

namespace {

constexpr int QBW = kAttnQBlocks;   // 16-query blocks per wave

// 4 consecutive elements of T into half of a fragment
template <typename T>
__device__ __forceinline__ void load4(const T* p, Frag8<T>& f, int half);
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, Frag8<uint16_t>& f, int half) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  f.v[2 * half] = v.x;
  f.v[2 * half + 1] = v.y;
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, Frag8<float>& f, int half) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  if (half == 0) f.a = v; else f.b = v;
}

}  // namespace

template <typename T, int HD>
__global__ __launch_bounds__(256, 2) void tree_attn_kernel(AttnParams p) {
  constexpr int NE = HD / 32;   // 8-element fragments per lane per query / key
  constexpr int NB = HD / 16;   // 16-dim blocks of O^T
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.nq / p.nkv;
  const int QG = p.rows_per_seq * G;
  const int nqb = (QG + 15) / 16;
  const int nqg = (nqb + QBW - 1) / QBW;
  const int NS = p.nsplit + 1;
  const int item = blockIdx.x * 4 + wave;
  if (item >= NS * nqg) return;
  const int split = item / nqg, qgrp = item % nqg;
  const bool scratch = split == p.nsplit;
  const int row0 = b * p.rows_per_seq;
  const int64_t bk = static_cast<int64_t>(b) * p.nkv + kvh;
  const T* kc = static_cast<const T*>(p.kc) + bk * p.cap * HD;
  const T* vt = static_cast<const T*>(p.vc) + bk * HD * p.cap;

  // Fragments of a prefix step at t0: K rows as MFMA A fragments (lane
  // (g, c) = key kb*16 + c) and V^T fragments (dim nb*16 + c, keys {4g + i}
  // in elements 0..3 and {16 + 4g + i} in 4..7, as two 4-key runs --
  // contiguous and 8-byte aligned, cap being a multiple of 8).  Rows past
  // the cache read its last row / run; nothing here depends on which keys
  // are live (dead keys' scores are masked and their V zeroed when the step
  // is used), so the loads can go out before the rows' lengths are known,
  // and every lane issues the same loads.
  auto load_prefix = [&](int t0, Frag8<T> (&kf)[2][NE], Frag8<T> (&vf)[NB]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int ci = min(t0 + kb * 16 + c, p.cap - 1);
#pragma unroll
      for (int e = 0; e < NE; ++e)
        kf[kb][e].load_nt(kc + static_cast<int64_t>(ci) * HD + g * (HD / 4) + 8 * e);
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int vo = min(t0 + 16 * half + 4 * g, p.cap - 4);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        load4<T>(vt + static_cast<int64_t>(nb * 16 + c) * p.cap + vo, vf[nb], half);
    }
  };

  // keys any row of this sequence may see: lane i reads row i, then a wave
  // reduction (rows_per_seq <= 64)
  int kmax = 0;
  uint64_t umask = 0;
  {
    // loaded together (row clamped), then selected
    const int lr = row0 + min(lane, p.rows_per_seq - 1);
    const int tk = p.tok[lr], pl = p.plen[lr];
    const uint64_t sm = p.smask[lr];
    const bool live = lane < p.rows_per_seq && tk >= 0;
    kmax = live ? min(pl, p.cap) : 0;
    umask = live ? sm : 0ull;
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    kmax = max(kmax, shfl_xor(kmax, o));
    const uint32_t lo = static_cast<uint32_t>(umask), hi = static_cast<uint32_t>(umask >> 32);
    const uint32_t olo = static_cast<uint32_t>(shfl_xor(static_cast<int>(lo), o));
    const uint32_t ohi = static_cast<uint32_t>(shfl_xor(static_cast<int>(hi), o));
    umask |= (static_cast<uint64_t>(ohi) << 32) | olo;
  }
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  umask = (static_cast<uint64_t>(static_cast<uint32_t>(
               __builtin_amdgcn_readfirstlane(static_cast<int>(umask >> 32)))) << 32) |
          static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(umask)));
  const int sbase = p.sbase[b];
  int kbeg, kend;
  if (scratch) {
    // the two 32-slot halves of the 64-bit ancestor mask
    kbeg = (umask & 0xffffffffull) ? 0 : 32;
    kend = umask ? ((umask >> 32) ? 64 : 32) : 0;
  } else {
    kbeg = split * p.split_keys;
    kend = min(kbeg + p.split_keys, kmax);
  }

  // per-column state; queries past the sequence's live rows are zero
  f32x4 oacc[QBW][NB];
  float mrun[QBW], lrun[QBW];
  bool qok[QBW];
  int plen_c[QBW];
  uint64_t mask_c[QBW];
#pragma unroll
  for (int u = 0; u < QBW; ++u) {
    const int mb = qgrp * QBW + u;
    const int m = mb * 16 + c;
    const int row = row0 + min(m / G, p.rows_per_seq - 1);
    const int tk = p.tok[row], pl = p.plen[row];
    const uint64_t sm = p.smask[row];
    qok[u] = mb < nqb && m < QG && tk >= 0;
    plen_c[u] = qok[u] ? min(pl, p.cap) : 0;
    mask_c[u] = qok[u] ? sm : 0ull;
    mrun[u] = -INFINITY;
    lrun[u] = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[u][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // the query fragments (rows clamped into the sequence; the scores of
  // queries past its live rows are masked), then a prefix split's first two
  // steps
  Frag8<T> qf[QBW][NE];
#pragma unroll
  for (int u = 0; u < QBW; ++u) {
    const int m = (qgrp * QBW + u) * 16 + c;
    const int row = row0 + min(m / G, p.rows_per_seq - 1);
    const int head = kvh * G + m % G;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      qf[u][e].load(static_cast<const T*>(p.q) + (static_cast<int64_t>(row) * p.nq + head) * HD +
                    g * (HD / 4) + 8 * e);
  }
  Frag8<T> ka[2][NE], va[NB], kb2[2][NE], vb2[NB];
  if (!scratch && kbeg < kend) {
    load_prefix(kbeg, ka, va);
    load_prefix(kbeg + 32, kb2, vb2);
  }

  // cache index of key j (0..31) of the step at t0, and whether any query
  // may see it
  auto key_index = [&](int t0, int j) { return scratch ? sbase + t0 + j : t0 + j; };
  auto key_live = [&](int t0, int j) {
    if (scratch) return ((umask >> (t0 + j)) & 1ull) != 0 && sbase + t0 + j < p.cap;
    return t0 + j < kend;
  };

  // Fragments of a scratch step (the tree's own rows: slots start at an
  // arbitrary row, so V is read element by element; dead keys read zero)
  auto load_scratch = [&](int t0, Frag8<T> (&kf)[2][NE], Frag8<T> (&vf)[NB]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int j = kb * 16 + c;
      const int ci = key_live(t0, j) ? key_index(t0, j) : 0;
#pragma unroll
      for (int e = 0; e < NE; ++e)
        kf[kb][e].load_nt(kc + static_cast<int64_t>(ci) * HD + g * (HD / 4) + 8 * e);
    }
    for (int nb = 0; nb < NB; ++nb) {
      const int d = nb * 16 + c;
      for (int e8 = 0; e8 < 8; ++e8) {
        const int j = 16 * (e8 >> 2) + 4 * g + (e8 & 3);
        const float x = key_live(t0, j)
                            ? Elem<T>::to_f(vt[static_cast<int64_t>(d) * p.cap + key_index(t0, j)])
                            : 0.f;
        vf[nb].set(e8, x);
      }
    }
  };

  // The online-softmax update of every query block with the step at t0.
  auto compute = [&](int t0, const Frag8<T> (&kf)[2][NE], Frag8<T> (&vf)[NB]) {
    // dead keys' V is zero (their probabilities are zero, and the rows they
    // were read from may hold anything)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8)
        if (!key_live(t0, 16 * (e8 >> 2) + 4 * g + (e8 & 3))) vf[nb].set(e8, 0.f);
#pragma unroll
    for (int u = 0; u < QBW; ++u) {
      if (qgrp * QBW + u >= nqb) continue;
      // S^T block: 32 keys x 16 query columns
      f32x4 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < NE; ++e) sc[kb] = mfma16(kf[kb][e], qf[u][e], sc[kb]);
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = kb * 16 + 4 * g + i;
          bool vis;
          if (scratch) vis = ((mask_c[u] >> (t0 + j)) & 1ull) != 0 && sbase + t0 + j < p.cap;
          else vis = t0 + j < plen_c[u] && t0 + j < kend;
          vis = vis && qok[u];
          const float v = vis ? sc[kb][i] * p.scale : -INFINITY;
          sc[kb][i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrun[u], tmax);
      float alpha = 1.f, psum = 0.f;
      if (mnew != -INFINITY) {
        alpha = (mrun[u] == -INFINITY) ? 0.f : expf(mrun[u] - mnew);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = (sc[kb][i] == -INFINITY) ? 0.f : expf(sc[kb][i] - mnew);
            sc[kb][i] = pv;
            psum += pv;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      psum += shfl_xor(psum, 16);
      psum += shfl_xor(psum, 32);
      lrun[u] = lrun[u] * alpha + psum;
      mrun[u] = mnew;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[u][nb] *= alpha;
      // P^T fragment: the lane's own probabilities, keys {4g + i} (elements
      // 0..3) and {16 + 4g + i} (elements 4..7)
      Frag8<T> ph, pl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = sc[0][i], p1 = sc[1][i];
        ph.set(i, p0);
        ph.set(4 + i, p1);
        if constexpr (sizeof(T) == 2) {
          pl.set(i, p0 - ph.get(i));
          pl.set(4 + i, p1 - ph.get(4 + i));
        }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        oacc[u][nb] = mfma16(vf[nb], ph, oacc[u][nb]);
        if constexpr (sizeof(T) == 2) oacc[u][nb] = mfma16(vf[nb], pl, oacc[u][nb]);
      }
    }
  };

  if (!scratch) {
    // prefix keys: each step's successor is in flight while it is used (two
    // register sets); loads past the range re-read the cache's last rows, so
    // every wait counts the same loads behind it
    for (int t0 = kbeg; t0 < kend; t0 += 64) {
      compute(t0, ka, va);
      if (t0 + 32 >= kend) break;
      load_prefix(t0 + 64, ka, va);
      compute(t0 + 32, kb2, vb2);
      if (t0 + 64 >= kend) break;
      load_prefix(t0 + 96, kb2, vb2);
    }
  } else {
    for (int t0 = kbeg; t0 < kend; t0 += 32) {
      Frag8<T> kf[2][NE], vf[NB];
      load_scratch(t0, kf, vf);
      compute(t0, kf, vf);
    }
  }

  // ---- this split's partial (max, sum, O) per query vector ----
  const int NSP = p.nsplit + 1;
#pragma unroll
  for (int u = 0; u < QBW; ++u) {
    const int mb = qgrp * QBW + u;
    const int m = mb * 16 + c;
    if (mb >= nqb || m >= QG) continue;
    const int64_t base = (bk * NSP + split) * QG + m;
    if (g == 0) {
      p.part_ml[base * 2] = mrun[u];
      p.part_ml[base * 2 + 1] = lrun[u];
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) p.part_o[base * HD + nb * 16 + 4 * g + i] = oacc[u][nb][i];
  }
}

// Merge of the splits: one workgroup per (query vector, kv head, sequence),
// one thread per dim.  The splits' (max, sum) pairs are read by one thread
// each and reduced across the workgroup, so their loads overlap instead of
// waiting on each other; the per-split weights go through LDS and every
// thread then sums its dim over the splits in split order (deterministic).
constexpr int kMergeThreads = 128;

__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(AttnParams p) {
  __shared__ float w_s[kMergeThreads];
  __shared__ float red_m[kMergeThreads / 64], red_l[kMergeThreads / 64];
  const int m = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int G = p.nq / p.nkv;
  const int QG = p.rows_per_seq * G;
  const int row = b * p.rows_per_seq + m / G;
  if (m >= QG || p.tok[row] < 0) return;
  const int NSP = p.nsplit + 1;   // <= kMergeThreads (checked at launch)
  const int64_t bk = static_cast<int64_t>(b) * p.nkv + kvh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float ms = -INFINITY, ls = 0.f;
  if (tid < NSP) {
    const int64_t base = (bk * NSP + tid) * QG + m;
    ms = p.part_ml[base * 2];
    ls = p.part_ml[base * 2 + 1];
  }
  float M = wave_max(ms);
  if (lane == 0) red_m[wave] = M;
  __syncthreads();
  M = red_m[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red_m[w]);
  const float wt = (ms == -INFINITY || M == -INFINITY) ? 0.f : expf(ms - M);
  w_s[tid] = wt;
  const float L = wave_sum(wt * ls);
  if (lane == 0) red_l[wave] = L;
  __syncthreads();
  float Ltot = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeThreads / 64; ++w) Ltot += red_l[w];
  const int head = kvh * G + m % G;
  for (int d = tid; d < p.hd; d += kMergeThreads) {
    float O = 0.f;
    const float* po = p.part_o + ((bk * NSP) * QG + m) * p.hd + d;
    const int64_t stride = static_cast<int64_t>(QG) * p.hd;
    int sp = 0;
    for (; sp + 4 <= NSP; sp += 4) {
      const float o0 = po[(sp + 0) * stride], o1 = po[(sp + 1) * stride];
      const float o2 = po[(sp + 2) * stride], o3 = po[(sp + 3) * stride];
      O += w_s[sp] * o0;
      O += w_s[sp + 1] * o1;
      O += w_s[sp + 2] * o2;
      O += w_s[sp + 3] * o3;
    }
    for (; sp < NSP; ++sp) O += w_s[sp] * po[sp * stride];
    p.o[(static_cast<int64_t>(row) * p.nq + head) * p.hd + d] = Ltot > 0.f ? O / Ltot : 0.f;
  }
}

template <typename T>
hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  const int G = p.nq / p.nkv;
  const int QG = p.rows_per_seq * G;
  if (p.rows_per_seq > 64 || QG > 1024 || p.split_keys % 64 || p.split_keys < 64 ||
      p.nsplit + 1 > kMergeThreads)
    return hipErrorInvalidValue;
  const int nqb = (QG + 15) / 16;
  const int nqg = (nqb + QBW - 1) / QBW;
  const int items = (p.nsplit + 1) * nqg;
  dim3 grid((items + 3) / 4, p.nkv, p.batch);
  if constexpr (sizeof(T) == 2) {
    if (p.hd == 128)
      hipLaunchKernelGGL((tree_attn_kernel<T, 128>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((tree_attn_kernel<T, 64>), grid, dim3(256), 0, s, p);
  } else {
    // fp32 storage is supported with head_dim 64 only
    if (p.hd != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL((tree_attn_kernel<T, 64>), grid, dim3(256), 0, s, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_merge_kernel, dim3(QG, p.nkv, p.batch), dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_attention<uint16_t>(const AttnParams&, hipStream_t);
template hipError_t launch_attention<float>(const AttnParams&, hipStream_t);

}  // namespace eagle
