// Shared device helpers for the MTP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

constexpr int kWG = 256;   // threads per workgroup in every kernel here (4 waves)
constexpr int kWave = 64;

// Workspace status word bits (the first int32 of every workspace).
constexpr int kFlagCapacity = 1;
constexpr int kFlagToken = 2;

// ----------------------------------------------------------------------------------------------
// element types: a 16-byte vector of weights holds VE elements
// ----------------------------------------------------------------------------------------------
struct BF16 {
  using T = uint16_t;
  static constexpr int VE = 8;
  __device__ __forceinline__ static void cvt(const uint4 v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ __forceinline__ static float get(const T* p, long i) { return __uint_as_float(uint32_t(p[i]) << 16); }
  // the first k elements of a vector, the rest zero
  __device__ __forceinline__ static uint4 keep_first(uint4 v, int k) {
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (e >= k) w[e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  // round-to-nearest-even float -> bf16 (finite inputs; NaN stays NaN)
  __device__ __forceinline__ static T put(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u) return T((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return T(u >> 16);
  }
};

struct F32 {
  using T = float;
  static constexpr int VE = 4;
  __device__ __forceinline__ static uint4 keep_first(uint4 v, int k) {
    return make_uint4(k > 0 ? v.x : 0u, k > 1 ? v.y : 0u, k > 2 ? v.z : 0u, k > 3 ? v.w : 0u);
  }
  __device__ __forceinline__ static void cvt(const uint4 v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static float get(const T* p, long i) { return p[i]; }
  __device__ __forceinline__ static T put(float f) { return f; }
};

// streaming 16-byte load (weights are read once per step: do not keep them in cache)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld_stream(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float4 ld_stream_f4(const float* p) {
  const uint4 v = ld_stream(p);
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// (value, index) order used by every argmax: larger value first, lower index on ties.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, kWave);
    int oi = __shfl_xor(i, o, kWave);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
}

// Sum of `n` per-thread values across the 256-thread workgroup; every thread gets the totals.
// red: __shared__ float[4 * n] scratch.  Contains two barriers.
template <int N>
__device__ __forceinline__ void wg_sum(float (&v)[N], float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < N; ++k) {
    float s = wave_sum(v[k]);
    if (lane == 0) red[wid * N + k] = s;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = red[k] + red[N + k] + red[2 * N + k] + red[3 * N + k];
  __syncthreads();
}

// Number of valid rows of a sequence: the prefix of non-negative tokens that are inside the
// vocabulary and still fit in the cache.  Also returns the flags that stopped the prefix.
// count_tokens8 judges the first min(rps, 8) tokens already in registers (t[e] for e < 8; the
// caller resolves rps > 8 with count_rows); count_rows reads eight tokens at a time, every load
// of a group issued unconditionally (clamped to the row) so that short rows cost one memory
// round trip.
__device__ __forceinline__ int count_tokens8(const int (&t)[8], int rps, int V, int len, int max_len, int* flags) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e >= rps || t[e] < 0) {
      if (flags) *flags = 0;
      return e < rps ? e : rps;
    }
    if (t[e] >= V) {
      if (flags) *flags = kFlagToken;
      return e;
    }
    if (len + e >= max_len) {
      if (flags) *flags = kFlagCapacity;
      return e;
    }
  }
  if (flags) *flags = 0;
  return 8;
}

__device__ __forceinline__ int count_rows(const int32_t* tok, int rps, int V, int len, int max_len, int* flags) {
  for (int i0 = 0; i0 < rps; i0 += 8) {
    int t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = tok[min(i0 + e, rps - 1)];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int n = i0 + e;
      if (n >= rps || t[e] < 0) {
        if (flags) *flags = 0;
        return n < rps ? n : rps;
      }
      if (t[e] >= V) {
        if (flags) *flags = kFlagToken;
        return n;
      }
      if (len + n >= max_len) {
        if (flags) *flags = kFlagCapacity;
        return n;
      }
    }
  }
  if (flags) *flags = 0;
  return rps;
}

// ---- MFMA operands (v_mfma_f32_16x16x32_bf16)
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// float -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Eight floats as two bf16x8 operands hi = bf16(x), lo = bf16(x - hi): hi + lo carries x to
// about 2^-17 relative, so two MFMAs give a near-fp32 product with a bf16 operand.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint16_t h0 = bf16_rne(x[2 * e]), h1 = bf16_rne(x[2 * e + 1]);
    const uint16_t l0 = bf16_rne(x[2 * e] - __uint_as_float(uint32_t(h0) << 16));
    const uint16_t l1 = bf16_rne(x[2 * e + 1] - __uint_as_float(uint32_t(h1) << 16));
    h[e] = uint32_t(h0) | (uint32_t(h1) << 16);
    l[e] = uint32_t(l0) | (uint32_t(l1) << 16);
  }
  hi = __builtin_bit_cast(bf16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8_t, make_uint4(l[0], l[1], l[2], l[3]));
}

}  // namespace mtp
