// In-place scaling of gradient rows by a device scalar.
//
// An autograd wrapper that writes d loss / d logits during its forward call
// ("GRPO Loss", Entry Point: the gradient lands in policy_logits, computed
// with an upstream gradient of 1) multiplies by the true upstream gradient in
// its backward.  The common upstream gradient 1 costs one scalar load per
// block: every block reads the scalar first and returns when it is 1.

#include <type_traits>

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_internal.hpp"

namespace grpo {

constexpr int kScaleThreads = 256;
constexpr int kScaleChunks = 4;  // 16-byte chunks per thread, loads issued together

template <typename TG>
__device__ __forceinline__ void scale_chunk(uint4& v, float s);

template <>
__device__ __forceinline__ void scale_chunk<float>(uint4& v, float s) {
  v.x = __float_as_uint(__uint_as_float(v.x) * s);
  v.y = __float_as_uint(__uint_as_float(v.y) * s);
  v.z = __float_as_uint(__uint_as_float(v.z) * s);
  v.w = __float_as_uint(__uint_as_float(v.w) * s);
}

template <>
__device__ __forceinline__ void scale_chunk<uint16_t>(uint4& v, float s) {
  v.x = pack_bf16x2(bf16lo(v.x) * s, bf16hi(v.x) * s);
  v.y = pack_bf16x2(bf16lo(v.y) * s, bf16hi(v.y) * s);
  v.z = pack_bf16x2(bf16lo(v.z) * s, bf16hi(v.z) * s);
  v.w = pack_bf16x2(bf16lo(v.w) * s, bf16hi(v.w) * s);
}

template <>
__device__ __forceinline__ void scale_chunk<_Float16>(uint4& v, float s) {
  uint32_t* w = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f2 f = f16x2_to_f32(w[k]);
    w[k] = pack_f16x2(f.x * s, f.y * s);
  }
}

// Rows of 16-byte chunks (every row start 16-byte aligned, V a whole number
// of chunks): a grid-stride walk over (row, chunk) pairs.
template <typename TG>
__global__ __launch_bounds__(kScaleThreads) void grpo_scale_vec_kernel(ScaleArgs a) {
  const float s = *a.scale;
  if (s == 1.0f) return;
  const int64_t per_row = a.V * int64_t(sizeof(TG)) / 16;
  const int64_t total = a.rows * per_row;
  const int64_t stride = int64_t(gridDim.x) * kScaleThreads * kScaleChunks;
  for (int64_t k0 = int64_t(blockIdx.x) * kScaleThreads * kScaleChunks + threadIdx.x; k0 < total;
       k0 += stride) {
    uint4 v[kScaleChunks];
    uint4* p[kScaleChunks];
#pragma unroll
    for (int u = 0; u < kScaleChunks; ++u) {
      const int64_t k = k0 + int64_t(u) * kScaleThreads;
      const int64_t row = k / per_row, c = k - row * per_row;
      p[u] = reinterpret_cast<uint4*>(static_cast<char*>(a.g) + row * a.ld * int64_t(sizeof(TG))) + c;
      if (k < total) v[u] = *p[u];
    }
#pragma unroll
    for (int u = 0; u < kScaleChunks; ++u) {
      if (k0 + int64_t(u) * kScaleThreads >= total) continue;
      scale_chunk<TG>(v[u], s);
      *p[u] = v[u];
    }
  }
}

// Any layout: one element per thread and step.
template <typename TG>
__global__ __launch_bounds__(kScaleThreads) void grpo_scale_any_kernel(ScaleArgs a) {
  const float s = *a.scale;
  if (s == 1.0f) return;
  const int64_t total = a.rows * a.V;
  for (int64_t k = int64_t(blockIdx.x) * kScaleThreads + threadIdx.x; k < total;
       k += int64_t(gridDim.x) * kScaleThreads) {
    const int64_t row = k / a.V, v = k - row * a.V;
    TG* p = reinterpret_cast<TG*>(static_cast<char*>(a.g) + row * a.ld * int64_t(sizeof(TG))) + v;
    if constexpr (sizeof(TG) == 4) {
      *p = *p * s;
    } else if constexpr (std::is_same<TG, uint16_t>::value) {
      *p = f32_to_bf16(bf16_to_f32(*p) * s);
    } else {
      // Left alone, the compiler fuses the multiply and the narrowing into
      // one f16-output mix FMA with a +0 addend, which rounds once and turns
      // a -0 product into +0.  The empty asm keeps the f32 product in a
      // register so that it rounds to f32 and then to f16, as the vector
      // path does.
      float prod = float(*p) * s;
      asm volatile("" : "+v"(prod));
      *p = _Float16(prod);
    }
  }
}

hipError_t launch_scale(const ScaleArgs& a, hipStream_t stream) {
  const int esize = a.dtype == GRPO_F32 ? 4 : 2;
  const bool vec = (reinterpret_cast<uintptr_t>(a.g) % 16) == 0 && (a.ld * esize) % 16 == 0 &&
                   (a.V * esize) % 16 == 0;
  // enough blocks to fill the chip several times over; the grid-stride loops
  // cover the rest
  const int64_t items = vec ? a.rows * (a.V * esize / 16) / kScaleChunks : a.rows * a.V;
  int64_t blocks = (items + kScaleThreads - 1) / kScaleThreads;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  const dim3 grid(static_cast<unsigned>(blocks)), block(kScaleThreads);
  if (vec) {
    if (a.dtype == GRPO_F32) hipLaunchKernelGGL(grpo_scale_vec_kernel<float>, grid, block, 0, stream, a);
    else if (a.dtype == GRPO_BF16) hipLaunchKernelGGL(grpo_scale_vec_kernel<uint16_t>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(grpo_scale_vec_kernel<_Float16>, grid, block, 0, stream, a);
  } else {
    if (a.dtype == GRPO_F32) hipLaunchKernelGGL(grpo_scale_any_kernel<float>, grid, block, 0, stream, a);
    else if (a.dtype == GRPO_BF16) hipLaunchKernelGGL(grpo_scale_any_kernel<uint16_t>, grid, block, 0, stream, a);
    else hipLaunchKernelGGL(grpo_scale_any_kernel<_Float16>, grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace grpo
