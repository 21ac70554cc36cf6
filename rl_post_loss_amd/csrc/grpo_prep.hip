// Mask counts, group-relative advantages and per-sequence token weights.
//
// Advantages follow the group normalisation of "GRPO Loss" (RL-Kernel docs,
// section Accuracy: population std, floored) and the leave-one-out baseline
// of the dockyard_rl design doc (section Advantage estimation).  Weights
// follow "GRPO Loss" (Normalizer semantics), the Relax REINFORCE++ page
// (PPO and KL reduction: mean within a response, then over responses) and
// the grpo.cpp README (The length-normalization detail: total weight
// L_i^alpha / B per response).
//
// Everything here is binary64 with contraction off, in the same sequential
// order as the defining formulas, so advantages and weights round to the
// same float32 bits as any other correct binary64 evaluation of that order.

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_internal.hpp"

namespace grpo {

constexpr int kPrepThreads = 256;

// Number of nonzero bytes in a 32-bit word.  For each byte b, bit 7 of
// ((b & 0x7f) + 0x7f) | b is set exactly when b != 0 (no carry crosses bytes).
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  uint32_t t = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
  return __popc(t);
}

__device__ double group_advantage(const float* __restrict__ r, int64_t s, int64_t e, int64_t i,
                                  bool leave_one_out, bool scale_by_std, double std_eps) {
#pragma clang fp contract(off)
  const int64_t n = e - s;
  double total = 0.0;
  for (int64_t j = s; j < e; ++j) total = total + double(r[j]);
  const double mean = total / double(n);
  double sq = 0.0;
  for (int64_t j = s; j < e; ++j) {
    const double dev = double(r[j]) - mean;
    sq = sq + dev * dev;
  }
  const double sd = sqrt(sq / double(n));
  const double denom = sd >= std_eps ? sd : std_eps;
  const double ri = double(r[i]);
  const double base = leave_one_out ? (total - ri) / double(n - 1) : mean;
  const double diff = ri - base;
  return scale_by_std ? diff / denom : diff;
}

__device__ double sequence_weight(int32_t reduction, double alpha, int64_t B, int64_t L,
                                  int64_t N) {
#pragma clang fp contract(off)
  if (reduction == GRPO_TOKEN_MEAN) return 1.0 / double(N > 0 ? N : 1);
  if (reduction == GRPO_SEQUENCE_MEAN) return 1.0 / (double(B) * double(L > 0 ? L : 1));
  if (L == 0) return 0.0;
  const double Lf = double(L);
  double num;
  if (alpha == 0.0) num = 1.0;
  else if (alpha == 0.5) num = sqrt(Lf);
  else if (alpha == 1.0) num = Lf;
  else num = pow(Lf, alpha);
  return num / (double(B) * Lf);
}

__global__ __launch_bounds__(kPrepThreads) void grpo_prep_kernel(PrepArgs a) {
  __shared__ long long sh_i64[kPrepThreads / kWave];
  __shared__ int sh_flag;
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;

  // L_i: active slots of sequence i
  long long cnt = 0;
  if (a.T > 0) {
    if (a.mask == nullptr) {
      cnt = (tid == 0) ? a.T : 0;
    } else {
      const uint8_t* row = a.mask + i * a.T;
      if ((a.T & 3) == 0 && (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0) {
        const uint32_t* w4 = reinterpret_cast<const uint32_t*>(row);
        for (int64_t k = tid; k < a.T / 4; k += kPrepThreads) cnt += nonzero_bytes(w4[k]);
      } else {
        for (int64_t k = tid; k < a.T; k += kPrepThreads) cnt += row[k] != 0;
      }
    }
  }
  const long long L = block_sum_i64<kPrepThreads>(cnt, sh_i64);

  if (tid == 0) {
    int64_t s, e;
    if (a.spp > 0) {
      s = (i / a.spp) * a.spp;
      e = s + a.spp;
    } else {
      int lo = 0, hi = a.num_groups;  // offsets[lo] <= i < offsets[hi]
      while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (a.offsets[mid] <= i) lo = mid; else hi = mid;
      }
      s = a.offsets[lo];
      e = a.offsets[lo + 1];
    }
    const double adv = group_advantage(a.rewards, s, e, i, a.leave_one_out != 0,
                                       a.scale_by_std != 0, a.std_eps);
    const float advf = float(adv);
    a.A[i] = advf;
    if (a.adv_out) a.adv_out[i] = advf;
    a.L[i] = int32_t(L);
    if (a.seq_tokens_out) a.seq_tokens_out[i] = int32_t(L);
  }
  if (!a.want_weights) return;

  if (last_block(&a.hdr->ticket_prep, unsigned(gridDim.x), &sh_flag)) {
    long long n = 0;
    for (int64_t k = tid; k < a.B; k += kPrepThreads) n += a.L[k];
    const long long N = block_sum_i64<kPrepThreads>(n, sh_i64);
    for (int64_t k = tid; k < a.B; k += kPrepThreads) {
      const double wk = sequence_weight(a.reduction, a.alpha, a.B, a.L[k], N);
      a.w[k] = wk;
      if (a.seq_weight_out) a.seq_weight_out[k] = float(wk);
    }
    if (tid == 0) {
      a.hdr->num_tokens = N;
      if (N == 0) atomicOr(&a.hdr->status, GRPO_FAULT_NO_TOKENS);
    }
  }
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(grpo_prep_kernel, dim3(unsigned(a.B)), dim3(kPrepThreads), 0, stream, a);
  return hipGetLastError();
}

// Workspace clearing (used once, before a workspace's first call).
__global__ void grpo_zero_kernel(uint4* p, size_t n16) {
  for (size_t k = size_t(blockIdx.x) * blockDim.x + threadIdx.x; k < n16;
       k += size_t(gridDim.x) * blockDim.x)
    p[k] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero(void* ws, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(grpo_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                     reinterpret_cast<uint4*>(ws), n16);
  return hipGetLastError();
}

}  // namespace grpo
