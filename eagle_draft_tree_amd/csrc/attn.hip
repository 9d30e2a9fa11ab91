// Tree attention of the draft layer.
//
// One workgroup per (split, kv head, sequence).  The query vectors of a
// sequence that share a kv head (rows_per_seq rows x G grouped heads, at most
// 128) form the MFMA columns; 64-key tiles of K and V are staged in LDS
// (V transposed) and shared by the four waves.  Scores are S^T = K Q^T, so
// each lane ends up owning one query column, which is also the column layout
// of O^T = V^T P^T: the online-softmax state never leaves the lane group.
// Visibility per query row: cache rows [0, prefix_len) (prefix splits) and
// the scratch rows scratch_base + j whose bit j is set in the row's 64-bit
// ancestor mask (one extra split).  Partial (max, sum, O) per split go to the
// workspace; the last split of a (sequence, kv head) to finish merges them.
#include "common.hpp"
#include "kernels.hpp"

namespace eagle {

namespace {

template <typename T> struct Vec16;
template <> struct Vec16<uint16_t> { static constexpr int n = 8; };
template <> struct Vec16<float> { static constexpr int n = 4; };

template <typename T>
__device__ __forceinline__ void load4(const T* p, Frag8<T>& f, int half);
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, Frag8<uint16_t>& f,
                                                int half) {
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
__global__ __launch_bounds__(256) void tree_attn_kernel(AttnParams p) {
  constexpr int KS = HD + 8;   // padded K row (elements)
  constexpr int VS = 64 + 8;   // padded V^T row (elements)
  constexpr int NE = HD / 32;  // frag8 per lane per query vector
  constexpr int NHB = HD / 16; // 16-row blocks of O^T
  __shared__ __attribute__((aligned(16))) T Ks[64 * KS];
  __shared__ __attribute__((aligned(16))) T Vt[HD * VS];
  __shared__ int s_kmax;
  __shared__ uint64_t s_umask;
  __shared__ int s_last;

  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int G = p.nq / p.nkv;
  const int QG = p.rows_per_seq * G;
  const int nmb = (QG + 15) / 16;
  const int NS = p.nsplit + 1;
  const bool scratch = split == p.nsplit;
  const int row0 = b * p.rows_per_seq;

  if (threadIdx.x == 0) {
    int km = 0;
    uint64_t um = 0;
    for (int i = 0; i < p.rows_per_seq; ++i) {
      if (p.tok[row0 + i] < 0) continue;
      km = max(km, min(p.plen[row0 + i], p.cap));
      um |= p.smask[row0 + i];
    }
    s_kmax = km;
    s_umask = um;
  }
  __syncthreads();
  const int kmax = s_kmax;
  const uint64_t umask = s_umask;
  const int sbase = p.sbase[b];

  int kbeg, kend;
  if (scratch) {
    kbeg = 0;
    kend = umask ? 64 : 0;
  } else {
    kbeg = split * p.chunk;
    kend = min(kbeg + p.chunk, kmax);
  }

  // per-wave query blocks (at most 2: QG <= 128)
  Frag8<T> qf[2][NE];
  f32x4 oacc[2][NHB];
  float mrun[2], lrun[2];
  int qrow[2], qhead[2];
  bool qok[2];
  int plen_c[2];
  uint64_t mask_c[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int mb = wave + 4 * u;
    const int m = mb * 16 + c;
    const int i = m / G;
    qok[u] = mb < nmb && m < QG && p.tok[row0 + min(i, p.rows_per_seq - 1)] >= 0;
    qrow[u] = row0 + (qok[u] ? i : 0);
    qhead[u] = kvh * G + m % G;
    plen_c[u] = qok[u] ? min(p.plen[qrow[u]], p.cap) : 0;
    mask_c[u] = qok[u] ? p.smask[qrow[u]] : 0ull;
    mrun[u] = -INFINITY;
    lrun[u] = 0.f;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) oacc[u][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      if (qok[u]) {
        const T* qp = static_cast<const T*>(p.q) +
                      (static_cast<int64_t>(qrow[u]) * p.nq + qhead[u]) * HD +
                      g * (HD / 4) + 8 * e;
        qf[u][e].load(qp);
      } else {
        qf[u][e].zero();
      }
    }
  }

  const T* kc = static_cast<const T*>(p.kc) +
                (static_cast<int64_t>(b) * p.nkv + kvh) * p.cap * HD;
  const T* vc = static_cast<const T*>(p.vc) +
                (static_cast<int64_t>(b) * p.nkv + kvh) * p.cap * HD;
  constexpr int VN = Vec16<T>::n;
  constexpr int CPR = HD / VN;  // 16-byte chunks per row

  for (int t0 = kbeg; t0 < kend; t0 += 64) {
    // ---- stage K and V^T tiles ----
    for (int ch = threadIdx.x; ch < 64 * CPR; ch += 256) {
      const int key = ch / CPR, h = (ch % CPR) * VN;
      const int ci = scratch ? sbase + key : t0 + key;
      const bool ok = scratch ? (((umask >> key) & 1ull) && ci >= 0 && ci < p.cap)
                              : (t0 + key < kend);
      Frag8<T> kv;  // used as a 16-byte carrier
      if constexpr (sizeof(T) == 2) {
        u32x4 kk = u32x4{0u, 0u, 0u, 0u}, vv = kk;
        if (ok) {
          kk = *reinterpret_cast<const u32x4*>(kc + static_cast<int64_t>(ci) * HD + h);
          vv = *reinterpret_cast<const u32x4*>(vc + static_cast<int64_t>(ci) * HD + h);
        }
        *reinterpret_cast<u32x4*>(&Ks[key * KS + h]) = kk;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          Vt[(h + e) * VS + key] =
              static_cast<T>((e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xffffu));
      } else {
        f32x4 kk = f32x4{0.f, 0.f, 0.f, 0.f}, vv = kk;
        if (ok) {
          kk = *reinterpret_cast<const f32x4*>(kc + static_cast<int64_t>(ci) * HD + h);
          vv = *reinterpret_cast<const f32x4*>(vc + static_cast<int64_t>(ci) * HD + h);
        }
        *reinterpret_cast<f32x4*>(&Ks[key * KS + h]) = kk;
#pragma unroll
        for (int e = 0; e < 4; ++e) Vt[(h + e) * VS + key] = vv[e];
      }
      (void)kv;
    }
    __syncthreads();

#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int mb = wave + 4 * u;
      if (mb >= nmb) continue;
      // S^T block: keys x query columns
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          Frag8<T> kf;
          kf.load(&Ks[(kb * 16 + c) * KS + g * (HD / 4) + 8 * e]);
          s[kb] = mfma16(kf, qf[u][e], s[kb]);
        }
      }
      // mask + scale, tile max
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kl = kb * 16 + 4 * g + j;
          bool vis;
          if (scratch) vis = ((mask_c[u] >> kl) & 1ull) != 0;
          else vis = (t0 + kl) < plen_c[u] && (t0 + kl) < kend;
          vis = vis && qok[u];
          const float v = vis ? s[kb][j] * p.scale : -INFINITY;
          s[kb][j] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, shfl_xor(tmax, 16));
      tmax = fmaxf(tmax, shfl_xor(tmax, 32));
      const float mnew = fmaxf(mrun[u], tmax);
      float alpha = 1.f, psum = 0.f;
      if (mnew != -INFINITY) {
        alpha = (mrun[u] == -INFINITY) ? 0.f : expf(mrun[u] - mnew);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float pv = (s[kb][j] == -INFINITY) ? 0.f : expf(s[kb][j] - mnew);
            s[kb][j] = pv;
            psum += pv;
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      psum += shfl_xor(psum, 16);
      psum += shfl_xor(psum, 32);
      lrun[u] = lrun[u] * alpha + psum;
      mrun[u] = mnew;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) oacc[u][hb] *= alpha;
      // O^T += V^T P^T over two 32-key halves
      // In bf16, P is carried as hi + lo bf16 parts (2^-17 relative), so the
      // only roundings of o are fp32 accumulation and its final storage.
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        Frag8<T> pf, pl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = s[2 * h2][j], p1 = s[2 * h2 + 1][j];
          pf.set(j, p0);
          pf.set(4 + j, p1);
          if constexpr (sizeof(T) == 2) {
            pl.set(j, p0 - pf.get(j));
            pl.set(4 + j, p1 - pf.get(4 + j));
          }
        }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          Frag8<T> vf;
          const T* vrow = &Vt[(hb * 16 + c) * VS];
          load4<T>(vrow + (2 * h2) * 16 + 4 * g, vf, 0);
          load4<T>(vrow + (2 * h2 + 1) * 16 + 4 * g, vf, 1);
          oacc[u][hb] = mfma16(vf, pf, oacc[u][hb]);
          if constexpr (sizeof(T) == 2) oacc[u][hb] = mfma16(vf, pl, oacc[u][hb]);
        }
      }
    }
    __syncthreads();
  }

  // ---- write this split's partial ----
  const int bk = b * p.nkv + kvh;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int mb = wave + 4 * u;
    const int m = mb * 16 + c;
    if (mb >= nmb || m >= QG) continue;
    const int64_t base = (static_cast<int64_t>(bk) * NS + split) * QG + m;
    if (g == 0) {
      p.part_ml[base * 2] = mrun[u];
      p.part_ml[base * 2 + 1] = lrun[u];
    }
    if (mrun[u] != -INFINITY) {
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          p.part_o[base * HD + hb * 16 + 4 * g + j] = oacc[u][hb][j];
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(p.cnt + bk, 1);
    s_last = prev == NS - 1;
    if (s_last) atomicExch(p.cnt + bk, 0);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // ---- merge all splits ----
  for (int idx = threadIdx.x; idx < QG * HD; idx += 256) {
    const int m = idx / HD, h = idx % HD;
    const int i = m / G;
    const int row = row0 + i;
    if (p.tok[row] < 0) continue;
    float M = -INFINITY;
    for (int sp = 0; sp < NS; ++sp) {
      const int64_t base = (static_cast<int64_t>(bk) * NS + sp) * QG + m;
      M = fmaxf(M, __builtin_nontemporal_load(p.part_ml + base * 2));
    }
    float L = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int sp = 0; sp < NS; ++sp) {
        const int64_t base = (static_cast<int64_t>(bk) * NS + sp) * QG + m;
        const float ms = __builtin_nontemporal_load(p.part_ml + base * 2);
        if (ms == -INFINITY) continue;
        const float w = expf(ms - M);
        L += w * __builtin_nontemporal_load(p.part_ml + base * 2 + 1);
        O += w * __builtin_nontemporal_load(p.part_o + base * HD + h);
      }
    }
    const float y = L > 0.f ? O / L : 0.f;
    const int head = kvh * G + m % G;
    p.o[(static_cast<int64_t>(row) * p.nq + head) * HD + h] = y;
  }
}

template <typename T>
hipError_t launch_attention(const AttnParams& p, hipStream_t s) {
  dim3 grid(p.nsplit + 1, p.nkv, p.batch);
  if (p.hd == 128)
    hipLaunchKernelGGL((tree_attn_kernel<T, 128>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((tree_attn_kernel<T, 64>), grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

template hipError_t launch_attention<uint16_t>(const AttnParams&, hipStream_t);
template hipError_t launch_attention<float>(const AttnParams&, hipStream_t);

}  // namespace eagle
