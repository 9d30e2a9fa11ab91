// Tree attention of the draft layer (split-KV, "flash decoding" style).
//
// One workgroup per (key range = split, kv head, sequence, round of four
// 16-query blocks).  The query vectors of a sequence that share a kv head
// (rows_per_seq rows x G grouped heads) are the MFMA columns; each of the
// four waves owns one block of 16 of them and runs the online softmax over
// the split's keys with its state in registers.  The keys are visited 32 at
// a time: the workgroup stages each step's K rows and V^T columns in LDS
// (double-buffered, the loads of the step after next in flight in
// registers), so every K/V byte is read from memory once per workgroup and
// shared by its query blocks.
//  * S^T = K Q^T: lane (g, c) reads key c's 8-dim fragments from the staged
//    K tile as the MFMA A operand, Q as the B operand with the same dim
//    permutation; it ends up holding keys 4g + i of query column c;
//  * O^T += V^T P^T: the V cache is stored transposed ([hd, cap] per head),
//    so lane (g, c) reads its 8 keys of dim c as two 4-key runs -- exactly
//    the keys whose probabilities it already holds, which makes them the B
//    fragment with no data movement.  In bf16, P is carried as hi + lo bf16
//    parts, so o keeps float precision;
//  * visibility: cache rows [0, prefix_len) of the query's row (prefix
//    splits) and scratch rows scratch_base + j for the set bits j of the
//    row's 64-bit ancestor mask (the last split).
// Each wave writes its (max, sum, O) per query vector; a second kernel
// merges the splits in split order.  No workgroup waits on another.
#include "common.hpp"
#include "kernels.hpp"

namespace eagle {

namespace {

// 16 bytes of LDS as 8 (bf16) or 4 (fp32) elements into a fragment
template <typename T>
__device__ __forceinline__ void lds_frag8(const unsigned char* p, Frag8<T>& f);
template <>
__device__ __forceinline__ void lds_frag8<uint16_t>(const unsigned char* p, Frag8<uint16_t>& f) {
  f.v = *reinterpret_cast<const u32x4*>(p);
}
template <>
__device__ __forceinline__ void lds_frag8<float>(const unsigned char* p, Frag8<float>& f) {
  f.a = *reinterpret_cast<const f32x4*>(p);
  f.b = *reinterpret_cast<const f32x4*>(p + 16);
}
// 4 consecutive elements of LDS into half of a fragment
template <typename T>
__device__ __forceinline__ void lds_half4(const unsigned char* p, Frag8<T>& f, int half);
template <>
__device__ __forceinline__ void lds_half4<uint16_t>(const unsigned char* p, Frag8<uint16_t>& f,
                                                    int half) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  f.v[2 * half] = v.x;
  f.v[2 * half + 1] = v.y;
}
template <>
__device__ __forceinline__ void lds_half4<float>(const unsigned char* p, Frag8<float>& f, int half) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  if (half == 0) f.a = v; else f.b = v;
}

}  // namespace

// LDS layout of one staged step: K tile [32 keys][HD] then V^T tile
// [HD][32 keys], rows padded (16 and 8/16 bytes) so that the 16 lanes
// reading 16 keys (K) or 16 dims (V^T) hit distinct banks.
template <typename T, int HD>
struct AttnTile {
  static constexpr int E = 16 / sizeof(T);                  // elements per 16 B
  static constexpr int KSTR = HD * sizeof(T) + 16;
  static constexpr int VSTR = 32 * sizeof(T) + (sizeof(T) == 2 ? 8 : 16);
  static constexpr int KCH = HD * sizeof(T) / 16;           // 16-byte chunks per K row
  static constexpr int VCH = 32 * sizeof(T) / 16;           // per V^T row
  static constexpr int NKC = 32 * KCH;                      // K chunks per step
  static constexpr int NCH = NKC + HD * VCH;                // all chunks per step
  static constexpr int CPT = NCH / 256;                     // chunks per thread
  static constexpr int BUF = 32 * KSTR + HD * VSTR;         // bytes per buffer
  static_assert(NKC % 256 == 0 && NCH % 256 == 0, "chunks split evenly over 256 threads");
};

// Three workgroups per CU (the second launch bound): at most 168 registers per
// lane, which the fragment order in `compute` below meets without spilling.
template <typename T, int HD>
__global__ __launch_bounds__(256, 3) void tree_attn_kernel(AttnParams p) {
  using L = AttnTile<T, HD>;
  constexpr int NE = HD / 32;   // 8-element fragments per lane per query / key
  constexpr int NB = HD / 16;   // 16-dim blocks of O^T
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * L::BUF];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int G = p.nq / p.nkv;
  const int QG = p.rows_per_seq * G;
  const int nqb = (QG + 15) / 16;
  const int nrounds = (nqb + 3) / 4;
  const int split = blockIdx.x, kvh = blockIdx.y;
  const int b = blockIdx.z / nrounds, round = blockIdx.z % nrounds;
  const int qb = round * 4 + wave;   // this wave's query block (none past nqb)
  const bool active = qb < nqb;
  const bool scratch = split == p.nsplit;
  const int row0 = b * p.rows_per_seq;
  const int64_t bk = static_cast<int64_t>(b) * p.nkv + kvh;
  const T* kc = static_cast<const T*>(p.kc) + bk * p.cap * HD;
  const T* vt = static_cast<const T*>(p.vc) + bk * HD * p.cap;

  // keys any row of this sequence may see (the same in every wave): lane i
  // reads row i, then a wave reduction (rows_per_seq <= 64)
  int kmax = 0;
  uint64_t umask = 0;
  {
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

  // this wave's query column: row, head, visibility, online-softmax state
  const int m = qb * 16 + c;
  const int qrow = row0 + min(m / G, p.rows_per_seq - 1);
  bool qok;
  int plen_c;
  uint64_t mask_c;
  {
    const int tk = p.tok[qrow], pl = p.plen[qrow];
    const uint64_t sm = p.smask[qrow];
    qok = active && m < QG && tk >= 0;
    plen_c = qok ? min(pl, p.cap) : 0;
    mask_c = qok ? sm : 0ull;
  }
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 oacc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) oacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  Frag8<T> qf[NE];
  {
    const int head = kvh * G + m % G;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      qf[e].load(static_cast<const T*>(p.q) + (static_cast<int64_t>(qrow) * p.nq + head) * HD +
                 g * (HD / 4) + 8 * e);
  }

  // cache index of key j (0..31) of the step at t0, and whether any query
  // may see it
  auto key_index = [&](int t0, int j) { return scratch ? sbase + t0 + j : t0 + j; };
  auto key_live = [&](int t0, int j) {
    if (scratch) return ((umask >> (t0 + j)) & 1ull) != 0 && sbase + t0 + j < p.cap;
    return t0 + j < kend;
  };

  // ---- staging: thread t moves 16-byte chunks t + 256 i of a step ----
  // request the chunks of the step at t0 (rows past the cache read its last
  // rows; dead keys are masked when the step is used)
  auto fetch = [&](int t0, u32x4 (&stg)[L::CPT]) {
#pragma unroll
    for (int i = 0; i < L::CPT; ++i) {
      const int q = tid + 256 * i;
      if (i < L::NKC / 256) {
        const int key = q / L::KCH, cc = q % L::KCH;
        const int row = min(key_index(t0, key), p.cap - 1);
        stg[i] = *reinterpret_cast<const u32x4*>(kc + static_cast<int64_t>(row) * HD + cc * L::E);
      } else {
        const int qq = q - L::NKC;
        const int d = qq / L::VCH, cv = qq % L::VCH;
        const T* vrow = vt + static_cast<int64_t>(d) * p.cap;
        if (!scratch) {
          // prefix keys: a 16-byte run (cap is a multiple of 8)
          const int k0 = min(t0 + cv * L::E, p.cap - L::E);
          stg[i] = *reinterpret_cast<const u32x4*>(vrow + k0);
        } else {
          // scratch slots start at an arbitrary row: element by element
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if constexpr (sizeof(T) == 2) {
              const int k = sbase + t0 + cv * L::E + 2 * e;
              const uint32_t lo = vrow[min(k, p.cap - 1)], hi = vrow[min(k + 1, p.cap - 1)];
              w[e] = lo | (hi << 16);
            } else {
              w[e] = __float_as_uint(vrow[min(sbase + t0 + cv * L::E + e, p.cap - 1)]);
            }
          }
          stg[i] = w;
        }
      }
    }
  };
  auto put = [&](const u32x4 (&stg)[L::CPT], int buf) {
    unsigned char* base = lds + buf * L::BUF;
#pragma unroll
    for (int i = 0; i < L::CPT; ++i) {
      const int q = tid + 256 * i;
      unsigned char* dst;
      if (i < L::NKC / 256) {
        dst = base + (q / L::KCH) * L::KSTR + (q % L::KCH) * 16;
      } else {
        const int qq = q - L::NKC;
        dst = base + 32 * L::KSTR + (qq / L::VCH) * L::VSTR + (qq % L::VCH) * 16;
      }
      // V^T rows are 8-byte aligned only
      reinterpret_cast<uint2*>(dst)[0] = uint2{stg[i][0], stg[i][1]};
      reinterpret_cast<uint2*>(dst)[1] = uint2{stg[i][2], stg[i][3]};
    }
  };

  // The online-softmax update of this wave's query block with the staged
  // step at t0 in buffer buf.
  auto compute = [&](int t0, int buf) {
    const unsigned char* kt = lds + buf * L::BUF;
    const unsigned char* vtt = kt + 32 * L::KSTR;
    // S^T block: 32 keys x 16 query columns, one 16-key half at a time
    f32x4 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      Frag8<T> kf[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e)
        lds_frag8<T>(kt + (kb * 16 + c) * L::KSTR + (g * (HD / 4) + 8 * e) * sizeof(T), kf[e]);
      sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < NE; ++e) sc[kb] = mfma16(kf[e], qf[e], sc[kb]);
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = kb * 16 + 4 * g + i;
        bool vis;
        if (scratch) vis = ((mask_c >> (t0 + j)) & 1ull) != 0 && sbase + t0 + j < p.cap;
        else vis = t0 + j < plen_c && t0 + j < kend;
        vis = vis && qok;
        const float v = vis ? sc[kb][i] * p.scale : -INFINITY;
        sc[kb][i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, shfl_xor(tmax, 32));
    const float mnew = fmaxf(mrun, tmax);
    float alpha = 1.f, psum = 0.f;
    if (mnew != -INFINITY) {
      alpha = (mrun == -INFINITY) ? 0.f : expf(mrun - mnew);
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
    lrun = lrun * alpha + psum;
    mrun = mnew;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) oacc[nb] *= alpha;
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
    // O^T += V^T P^T, half of the 16-dim blocks at a time (the V^T
    // fragments are read only now, and half of them at once: fewer registers
    // live, three waves per SIMD).  Dead keys' V is zero (their
    // probabilities are zero, and the rows they were read from may hold
    // anything); a step of live prefix keys skips that.
    const bool all_live = t0 + 32 <= kend && !scratch;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      Frag8<T> vf[NB / 2];
#pragma unroll
      for (int i = 0; i < NB / 2; ++i) {
        const unsigned char* vr = vtt + ((h * NB / 2 + i) * 16 + c) * L::VSTR;
        lds_half4<T>(vr + 4 * g * sizeof(T), vf[i], 0);
        lds_half4<T>(vr + (16 + 4 * g) * sizeof(T), vf[i], 1);
      }
      if (!all_live) {
#pragma unroll
        for (int i = 0; i < NB / 2; ++i)
#pragma unroll
          for (int e8 = 0; e8 < 8; ++e8)
            if (!key_live(t0, 16 * (e8 >> 2) + 4 * g + (e8 & 3))) vf[i].set(e8, 0.f);
      }
#pragma unroll
      for (int i = 0; i < NB / 2; ++i) {
        const int nb = h * NB / 2 + i;
        oacc[nb] = mfma16(vf[i], ph, oacc[nb]);
        if constexpr (sizeof(T) == 2) oacc[nb] = mfma16(vf[i], pl, oacc[nb]);
      }
    }
  };

  // ---- the steps ----
  const int nst = kbeg < kend ? (kend - kbeg + 31) / 32 : 0;
  if (nst > 0 && !scratch) {
    // prefix keys: step s + 1 is staged from registers while step s is used,
    // the loads of steps s + 2 and s + 3 in flight meanwhile (two register
    // sets).  Every fetch is issued, past the range re-reading the last
    // step, so that each wait counts the same loads behind it.
    u32x4 r0[L::CPT], r1[L::CPT];
    auto step_t0 = [&](int st) { return kbeg + 32 * min(st, nst - 1); };
    fetch(step_t0(0), r0);
    put(r0, 0);
    fetch(step_t0(1), r0);
    fetch(step_t0(2), r1);
    __syncthreads();
    for (int st = 0; st < nst; st += 2) {
      put(r0, 1);                        // step st + 1
      fetch(step_t0(st + 3), r0);
      if (active) compute(kbeg + 32 * st, 0);
      __syncthreads();
      if (st + 1 >= nst) break;
      put(r1, 0);                        // step st + 2
      fetch(step_t0(st + 4), r1);
      if (active) compute(kbeg + 32 * (st + 1), 1);
      __syncthreads();
    }
  } else if (nst > 0) {
    // the tree's own rows (at most two steps): one register set
    u32x4 r0[L::CPT];
    fetch(kbeg, r0);
    put(r0, 0);
    if (nst > 1) fetch(kbeg + 32, r0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
      if (st + 1 < nst) put(r0, (st + 1) & 1);
      if (active) compute(kbeg + 32 * st, st & 1);
      __syncthreads();
    }
  }

  // ---- this split's partial (max, sum, O) per query vector ----
  if (!active || m >= QG) return;
  const int NSP = p.nsplit + 1;
  const int64_t base = (bk * NSP + split) * QG + m;
  if (g == 0) {
    p.part_ml[base * 2] = mrun;
    p.part_ml[base * 2 + 1] = lrun;
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    *reinterpret_cast<f32x4*>(p.part_o + base * HD + nb * 16 + 4 * g) = oacc[nb];
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
      p.nsplit + 1 > kMergeThreads || p.cap % 8 || p.cap < 32)
    return hipErrorInvalidValue;
  const int nrounds = ((QG + 15) / 16 + 3) / 4;
  dim3 grid(p.nsplit + 1, p.nkv, p.batch * nrounds);
  if constexpr (sizeof(T) == 2) {
    if (p.hd == 128)
      hipLaunchKernelGGL((tree_attn_kernel<T, 128>), grid, dim3(256), 0, s, p);
    else if (p.hd == 64)
      hipLaunchKernelGGL((tree_attn_kernel<T, 64>), grid, dim3(256), 0, s, p);
    else
      return hipErrorInvalidValue;
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
