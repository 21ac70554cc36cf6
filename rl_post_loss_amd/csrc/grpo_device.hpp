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

// --- launch order to work order across the XCDs ----------------------------
// The dispatcher hands a launch's blocks to the chip's 8 XCDs in turn (block
// b to XCD b mod 8), and each XCD has its own L2 and address translation
// caches.  xcd_runs() permutes [0, n) so that each XCD takes runs of C
// consecutive work items: the items are cut into spans of 8 C, and in span
// s the XCD's blocks take its run (x + s) mod 8 in order.  The rows (or
// sequences) an XCD has in flight are then neighbours in memory, not spread
// over eight times the address range, while every span is still shared
// evenly by the XCDs;
// the rotation keeps a span that is only partly busy (the end of a ragged
// sequence) from loading the same XCDs every time.  Items past the last
// whole span keep their place.  C = 0 keeps the launch order.
__device__ __forceinline__ uint32_t xcd_runs(uint32_t b, uint32_t n, uint32_t C) {
  if (C == 0u) return b;
  const uint32_t span = 8u * C;
  const uint32_t whole = n - n % span;
  if (b >= whole) return b;
  const uint32_t x = b % 8u, k = b / 8u, s = k / C;
  return s * span + ((x + s) % 8u) * C + k % C;
}

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

// --- wave64 reductions without LDS traffic -----------------------------------
// A wave-wide reduction runs six exchange steps; after step k every lane holds
// the combination of a group of 2^(k+1) lanes.  Steps 0-3 stay inside a row
// of 16 lanes and use DPP lane selection on a v_mov (quad permutation
// 1,0,3,2, quad permutation 2,3,0,1, the half-row mirror 7 - l, the row mirror
// 15 - l); steps 4 and 5 cross rows with gfx950's v_permlane16_swap (rows
// 0 <-> 1, 2 <-> 3) and v_permlane32_swap (lanes 0-31 <-> 32-63).  Each step
// pairs lanes symmetrically and combines the two values with a commutative
// operation, so both lanes of a pair, and at the end every lane, hold the
// same bits; the tree is fixed, so the result is the same from run to run.
// Every lane of the wave must be active.
struct Pair32 {
  uint32_t a, b;
};

template <int STEP>
__device__ __forceinline__ Pair32 wave_step_u32(uint32_t v) {
  static_assert(STEP >= 0 && STEP < 6, "six steps cover 64 lanes");
  if constexpr (STEP < 4) {
    constexpr int ctrl = STEP == 0 ? 0xB1 : (STEP == 1 ? 0x4E : (STEP == 2 ? 0x141 : 0x140));
    const uint32_t p = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), ctrl, 0xF, 0xF, true));
    return Pair32{v, p};
  } else if constexpr (STEP == 4) {
    // with both operands v, the pair comes back as (even row's value, odd
    // row's value) in every lane of the two rows: the same operands, in the
    // same order, on both sides
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return Pair32{r[0], r[1]};
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return Pair32{r[0], r[1]};
  }
}

template <int STEP>
__device__ __forceinline__ void wave_step_f32(float v, float& a, float& b) {
  const Pair32 p = wave_step_u32<STEP>(__float_as_uint(v));
  a = __uint_as_float(p.a);
  b = __uint_as_float(p.b);
}

template <int STEP>
__device__ __forceinline__ void wave_step_u64(uint64_t v, uint64_t& a, uint64_t& b) {
  const Pair32 lo = wave_step_u32<STEP>(uint32_t(v));
  const Pair32 hi = wave_step_u32<STEP>(uint32_t(v >> 32));
  a = uint64_t(lo.a) | (uint64_t(hi.a) << 32);
  b = uint64_t(lo.b) | (uint64_t(hi.b) << 32);
}

template <int STEP>
__device__ __forceinline__ Lse wave_step_lse(Lse v) {
  Lse a, b;
  wave_step_f32<STEP>(v.m, a.m, b.m);
  wave_step_f32<STEP>(v.mL, a.mL, b.mL);
  wave_step_f32<STEP>(v.s, a.s, b.s);
  return lse_merge(a, b);
}

template <int STEP>
__device__ __forceinline__ double wave_step_f64(double v) {
  uint64_t a, b;
  wave_step_u64<STEP>(uint64_t(__double_as_longlong(v)), a, b);
  return __longlong_as_double((long long)a) + __longlong_as_double((long long)b);
}

template <int STEP>
__device__ __forceinline__ long long wave_step_i64(long long v) {
  uint64_t a, b;
  wave_step_u64<STEP>(uint64_t(v), a, b);
  return (long long)(a + b);
}

template <int STEP>
__device__ __forceinline__ uint32_t wave_step_or(uint32_t v) {
  const Pair32 p = wave_step_u32<STEP>(v);
  return p.a | p.b;
}

template <int STEP>
__device__ __forceinline__ int wave_step_i32(int v) {
  const Pair32 p = wave_step_u32<STEP>(uint32_t(v));
  return int(p.a + p.b);
}

// Every lane ends with the merged state of the whole wave.
template <int width>
__device__ __forceinline__ Lse wave_lse(Lse v) {
  static_assert(width == kWave, "whole waves");
  v = wave_step_lse<0>(v);
  v = wave_step_lse<1>(v);
  v = wave_step_lse<2>(v);
  v = wave_step_lse<3>(v);
  v = wave_step_lse<4>(v);
  return wave_step_lse<5>(v);
}

template <int width>
__device__ __forceinline__ double wave_sum_f64(double v) {
  static_assert(width == kWave, "whole waves");
  v = wave_step_f64<0>(v);
  v = wave_step_f64<1>(v);
  v = wave_step_f64<2>(v);
  v = wave_step_f64<3>(v);
  v = wave_step_f64<4>(v);
  return wave_step_f64<5>(v);
}

template <int width>
__device__ __forceinline__ long long wave_sum_i64(long long v) {
  static_assert(width == kWave, "whole waves");
  v = wave_step_i64<0>(v);
  v = wave_step_i64<1>(v);
  v = wave_step_i64<2>(v);
  v = wave_step_i64<3>(v);
  v = wave_step_i64<4>(v);
  return wave_step_i64<5>(v);
}

template <int width>
__device__ __forceinline__ int wave_sum_i32(int v) {
  static_assert(width == kWave, "whole waves");
  v = wave_step_i32<0>(v);
  v = wave_step_i32<1>(v);
  v = wave_step_i32<2>(v);
  v = wave_step_i32<3>(v);
  v = wave_step_i32<4>(v);
  return wave_step_i32<5>(v);
}

template <int STEP>
__device__ __forceinline__ int wave_step_max(int v) {
  const Pair32 p = wave_step_u32<STEP>(uint32_t(v));
  return int(p.a) > int(p.b) ? int(p.a) : int(p.b);
}

__device__ __forceinline__ int wave_max_i32(int v) {
  v = wave_step_max<0>(v);
  v = wave_step_max<1>(v);
  v = wave_step_max<2>(v);
  v = wave_step_max<3>(v);
  v = wave_step_max<4>(v);
  return wave_step_max<5>(v);
}

__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
  v = wave_step_or<0>(v);
  v = wave_step_or<1>(v);
  v = wave_step_or<2>(v);
  v = wave_step_or<3>(v);
  v = wave_step_or<4>(v);
  return wave_step_or<5>(v);
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
