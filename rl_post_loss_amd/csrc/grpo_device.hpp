// Device-side building blocks shared by the libgrpo kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace grpo {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Start value of a running maximum.  Finite on purpose: kLog2e * kMaxInit
// stays finite, so fma(x, kLog2e, -mL) is never (-inf) - (-inf).
constexpr float kMaxInit = -1.0e30f;

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// bf16 -> f32 is exact: the bf16 bits are the top half of the f32 bits.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Two f32 -> packed bf16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return uint16_t(pack_bf16x2(x, 0.0f) & 0xffffu);
}

// IEEE binary16: -> f32 is exact (v_cvt_f32_f16); f32 -> f16 rounds to
// nearest even in the default rounding mode.
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f2 f16x2_to_f32(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(h2, w), f2);
}
__device__ __forceinline__ float f16_to_f32(uint16_t h) {
  return float(__builtin_bit_cast(_Float16, h));
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
}
__device__ __forceinline__ uint16_t f32_to_f16(float x) {
  return __builtin_bit_cast(uint16_t, _Float16(x));
}

// Raw 2^x (v_exp_f32).  Results below the normal range flush to zero; every
// caller only feeds it arguments whose tiny results do not matter.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Running log-sum-exp state of one thread, in base 2:
//   sum over seen x of 2^(x*log2e - mL),  m = max seen x,  mL = fl(m*log2e).
// mL is carried (not recomputed) so every rescale uses the same rounded value.
struct Lse {
  float m, mL, s;
};

__device__ __forceinline__ Lse lse_init() { return Lse{kMaxInit, kMaxInit * kLog2e, 0.0f}; }

// Commutative merge: the operand with the larger maximum is the base, so the
// result does not depend on which side of a butterfly computes it.
__device__ __forceinline__ Lse lse_merge(Lse a, Lse b) {
  if (b.m > a.m || (b.m == a.m && b.s > a.s)) {
    Lse t = a;
    a = b;
    b = t;
  }
  a.s = a.s + b.s * fast_exp2(b.mL - a.mL);
  return a;
}

__device__ __forceinline__ Lse shfl_xor_lse(Lse v, int mask) {
  return Lse{__shfl_xor(v.m, mask), __shfl_xor(v.mL, mask), __shfl_xor(v.s, mask)};
}

// Butterfly over `width` lanes (power of two <= 64); every lane ends with the
// same merged state, independent of lane order.
template <int width>
__device__ __forceinline__ Lse wave_lse(Lse v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v = lse_merge(v, shfl_xor_lse(v, off));
  return v;
}

template <int width>
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int width>
__device__ __forceinline__ long long wave_sum_i64(long long v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

template <int width>
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int off = width / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Block-wide sums in a fixed tree (butterfly in each wave, then the per-wave
// partials in wave order).  All threads of the block must call them.
template <int NT>
__device__ __forceinline__ double block_sum_f64(double v, double* sh) {
  constexpr int NW = NT / kWave;
  v = wave_sum_f64<kWave>(v);
  if constexpr (NW == 1) {
    return v;
  } else {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) sh[w] = v;
    __syncthreads();
    double t = 0.0;
    for (int k = 0; k < NW; ++k) t += sh[k];
    return t;
  }
}

template <int NT>
__device__ __forceinline__ long long block_sum_i64(long long v, long long* sh) {
  constexpr int NW = NT / kWave;
  v = wave_sum_i64<kWave>(v);
  if constexpr (NW == 1) {
    return v;
  } else {
    const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) sh[w] = v;
    __syncthreads();
    long long t = 0;
    for (int k = 0; k < NW; ++k) t += sh[k];
    return t;
  }
}

}  // namespace grpo
