// Shared device helpers for the gfx950 kernels: element types, bf16
// conversion, 8-element fragments and the 16x16x32 MFMA step, wave shuffles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eagle {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kWave = 64;
constexpr int kMaxTopK = 16;
constexpr float kLogEps = -27.631021115928547f;  // log(1e-12) in float32

// ----------------------------------------------------------------------------
// bf16 <-> fp32
// ----------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
// Round to nearest even through the hardware conversion (v_cvt_pk_bf16_f32,
// NaN stays NaN).  A bit-level rounding in software costs a divergent branch
// per value for the NaN case, which made staging fp32 activations as bf16
// pairs a large part of the streaming GEMM's time.
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
// two values in one 32-bit word: a in the low half, b in the high half
__device__ __forceinline__ uint32_t f2bf_pair(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Element traits.  T is the storage type: uint16_t (bf16 bits) or float.
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float to_f(uint16_t v) { return bf2f(v); }
  static __device__ __forceinline__ uint16_t from_f(float v) { return f2bf(v); }
  // value after storage rounding
  static __device__ __forceinline__ float round(float v) { return bf2f(f2bf(v)); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
  static __device__ __forceinline__ float round(float v) { return v; }
};

// ----------------------------------------------------------------------------
// 8-element fragments (one lane's share of a 16x16x32 MFMA operand)
// ----------------------------------------------------------------------------
template <typename T> struct Frag8;
template <> struct Frag8<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void load(const uint16_t* p) {
    v = *reinterpret_cast<const u32x4*>(p);
  }
  // streamed once: non-temporal loads keep HBM reads off the cache paths
  // that cap ordinary loads at well under half the bandwidth
  __device__ __forceinline__ void load_nt(const uint16_t* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ float get(int i) const {
    uint32_t w = v[i >> 1];
    return bf2f(static_cast<uint16_t>((i & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  __device__ __forceinline__ void set_pair(int j, float lo, float hi) { v[j] = f2bf_pair(lo, hi); }
  __device__ __forceinline__ void set(int i, float x) {
    uint32_t w = v[i >> 1];
    uint32_t b = f2bf(x);
    w = (i & 1) ? ((w & 0xffffu) | (b << 16)) : ((w & 0xffff0000u) | b);
    v[i >> 1] = w;
  }
};
template <> struct Frag8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void zero() {
    a = f32x4{0.f, 0.f, 0.f, 0.f};
    b = a;
  }
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4*>(p);
    b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  __device__ __forceinline__ void load_nt(const float* p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  }
  __device__ __forceinline__ float get(int i) const { return i < 4 ? a[i] : b[i - 4]; }
  __device__ __forceinline__ void set(int i, float x) {
    if (i < 4) a[i] = x; else b[i - 4] = x;
  }
};

// A operand of a weight-type MFMA built from float activations.  For bf16
// weights the activation is carried as hi + lo bf16 parts (2^-17 relative),
// so the product is accurate to float precision at twice the MFMA count.
template <typename TW> struct AFrag;
template <> struct AFrag<uint16_t> {
  Frag8<uint16_t> hi, lo;
  __device__ __forceinline__ void zero() { hi.zero(); lo.zero(); }
  __device__ __forceinline__ void from_float(const Frag8<float>& x) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = x.get(2 * j), b = x.get(2 * j + 1);
      hi.set_pair(j, a, b);
      lo.set_pair(j, a - hi.get(2 * j), b - hi.get(2 * j + 1));
    }
  }
  __device__ __forceinline__ void from_raw(const Frag8<uint16_t>& w) { hi = w; lo.zero(); }
};
template <> struct AFrag<float> {
  Frag8<float> hi;
  __device__ __forceinline__ void zero() { hi.zero(); }
  __device__ __forceinline__ void from_float(const Frag8<float>& x) { hi = x; }
  __device__ __forceinline__ void from_raw(const Frag8<float>& w) { hi = w; }
};

// acc[16x16] += A[16 x 32] * B[32 x 16] where lane l holds row/col (l % 16)
// and the 8 k-values of lane group (l / 16).  Any k-permutation shared by A
// and B gives the same sum, which the callers use to load wide contiguous
// runs per lane.
__device__ __forceinline__ f32x4 mfma16(const Frag8<uint16_t>& a,
                                        const Frag8<uint16_t>& b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8_t, a.v), __builtin_bit_cast(bf16x8_t, b.v),
      acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const Frag8<float>& a,
                                        const Frag8<float>& b, f32x4 acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a[i], b.a[i], acc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b[i], b.b[i], acc, 0, 0, 0);
  return acc;
}

// ----------------------------------------------------------------------------
// wave helpers
// ----------------------------------------------------------------------------
// Lane i gets the value of lane i ^ m.  Masks 1 and 2 are DPP quad
// permutations and 8 a DPP rotation by 8 within each 16-lane row (both plain
// VALU moves); 4 and 16 are ds_swizzle in bit mode (within 32 lanes, no LDS
// access); 32 and anything else go through ds_bpermute.  The callers' loops
// are unrolled, so m is a constant and the choice folds away.
__device__ __forceinline__ int shfl_xor(int v, int m) {
  switch (m) {
    case 1: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    case 8: return __builtin_amdgcn_mov_dpp(v, 0x128, 0xF, 0xF, false);  // row_ror:8
    case 4: return __builtin_amdgcn_ds_swizzle(v, (4 << 10) | 0x1F);
    case 16: return __builtin_amdgcn_ds_swizzle(v, (16 << 10) | 0x1F);
    default: return __shfl_xor(v, m, kWave);
  }
}
__device__ __forceinline__ float shfl_xor(float v, int m) {
  return __int_as_float(shfl_xor(__float_as_int(v), m));
}
// Wave-wide max / sum, the same value in every lane: a butterfly within each
// 32-lane half, then the two halves' results combined (half 0 first).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m <= 16; m <<= 1) v = fmaxf(v, shfl_xor(v, m));
  return fmaxf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)),
               __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32)));
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m <= 16; m <<= 1) v += shfl_xor(v, m);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0)) +
         __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
}

// (value, id) order used by every top-k: larger value first, then lower id
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// Bitonic sort of one (value, id) pair per lane across the wave; afterwards
// lane i holds the i-th best pair.
__device__ __forceinline__ void wave_sort_desc(float& v, int& id) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j >= 1; j >>= 1) {
      float ov = shfl_xor(v, j);
      int oi = shfl_xor(id, j);
      bool lower = (lane & j) == 0;           // lane is the lower of the pair
      bool desc = (lane & k) == 0;            // this block sorts best-first
      bool o_better = better(ov, oi, v, id);
      bool take = desc ? (lower ? o_better : !o_better)
                       : (lower ? !o_better : o_better);
      if (ov == v && oi == id) take = false;
      if (take) { v = ov; id = oi; }
    }
  }
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// ----------------------------------------------------------------------------
// Philox4x64-10 counter-based generator (Salmon, Moraes, Dror, Shaw, SC 2011):
// ten rounds of two 64x64->128-bit multiplications over a 4-word counter,
// key bumped by two Weyl constants between rounds.
// ----------------------------------------------------------------------------
constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;
constexpr uint64_t kStreamVerify = 0;   // key word 1 of verification draws
constexpr uint64_t kStreamDraft = 1;    // key word 1 of drafting draws

// the four output words of the block at counter (c0, c1, c2, c3), key (k0, k1)
__device__ __forceinline__ void philox4x64(uint64_t c0, uint64_t c1, uint64_t c2, uint64_t c3,
                                           uint64_t k0, uint64_t k1, uint64_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kPhiloxM0, c0), lo0 = kPhiloxM0 * c0;
    const uint64_t hi1 = __umul64hi(kPhiloxM1, c2), lo1 = kPhiloxM1 * c2;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// first output word of the block at counter (c0, c1, c2, c3), key (k0, k1)
__device__ __forceinline__ uint64_t philox4x64_w0(uint64_t c0, uint64_t c1, uint64_t c2,
                                                  uint64_t c3, uint64_t k0, uint64_t k1) {
  uint64_t w[4];
  philox4x64(c0, c1, c2, c3, k0, k1, w);
  return w[0];
}

// U[0,1) float: counter (draw, row, sequence, round), key (seed, stream);
// the top 24 bits of the first output word times 2^-24 (exact in float)
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint64_t stream, uint64_t rnd,
                                                uint64_t b, uint64_t row, uint64_t draw) {
  const uint64_t x = philox4x64_w0(draw, row, b, rnd, seed, stream);
  return static_cast<float>(x >> 40) * 5.9604644775390625e-08f;
}

}  // namespace eagle
