// Mask counts, group-relative advantages and per-sequence token weights.
//
// Advantages follow the group normalisation of "GRPO Loss" (RL-Kernel docs,
// section Accuracy: population std, floored) and the leave-one-out baseline
// of the dockyard_rl design doc (section Advantage estimation).  Weights
// follow "GRPO Loss" (Normalizer semantics), the Relax REINFORCE++ page
// (PPO and KL reduction: mean within a response, then over responses) and
// the grpo.cpp README (The length-normalization detail: total weight
// L_i^alpha / B per response); the fixed-constant normaliser divides by a
// declared constant ("GRPO Loss", Normalizer semantics).
//
// Everything here is binary64 with contraction off, in the same sequential
// order as the defining formulas, so advantages and weights round to the
// same float32 bits as any other correct binary64 evaluation of that order.
//
// Two kernels, so that no block ever waits on another: grpo_prep_kernel (one
// block per sequence: L_i and A_i) and grpo_weights_kernel (one block: N and
// every w_i).  The kernel boundary between them makes the counts visible.
// The log-prob token loss skips the second: its token kernel forms w_i itself.

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_groupadv.hpp"
#include "grpo_internal.hpp"
#include "grpo_objective.hpp"

namespace grpo {

constexpr int kPrepThreads = 256;
constexpr int kWeightThreads = 1024;


// One block per sequence i: L_i (active slots) and A_i.  The group's rewards
// are staged in LDS by all threads; one thread then forms the binary64 sums
// in index order.  Block 0 also clears the workspace fault word, which no
// other kernel of the call writes before this one has finished.
__global__ __launch_bounds__(kPrepThreads) void grpo_prep_kernel(PrepArgs a) {
#pragma clang fp contract(off)
  __shared__ long long sh_i64[kPrepThreads / kWave];
  __shared__ double sh_f64[kPrepThreads / kWave];
  __shared__ float sh_r[kRewardStage];
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  if (i == 0 && tid == 0 && a.want_weights) a.hdr->status = 0;

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

  // importance-weight statistic over the active tokens, in binary64 and a
  // fixed tree: the sum of (old - gen) for sequence masking, the sum of the
  // (truncated) token weights for the sequence ratio's mean weight
  if (a.iw_mode != kIwNone) {
    const int64_t base = i * a.T;
    double acc = 0.0;
    for (int64_t t = tid; t < a.T; t += kPrepThreads) {
      if (a.mask != nullptr && a.mask[base + t] == 0) continue;
      const float o = a.old[base + t], g = a.gen[base + t];
      if (a.iw_mode == kIwSeqMask) acc = acc + (double(o) - double(g));
      else acc = acc + double(token_is_weight(a.obj, o, g));
    }
    acc = block_sum_f64<kPrepThreads>(acc, sh_f64);
    if (tid == 0) {
      const double mean = acc / double(L > 0 ? L : 1);
      if (a.iw_mode == kIwSeqMask) {
        const double r = exp(mean);
        a.iwseq[i] = (r >= a.seq_lo && r <= a.seq_hi) ? 1.0 : 0.0;
      } else {
        a.iwseq[i] = mean;
      }
    }
  }
  if (tid == 0 && a.useq) a.useq[i] = 0.0f;

  if (a.rewards == nullptr) {
    // token advantages come from the caller: only the counts are needed
    if (tid == 0) {
      a.A[i] = 0.0f;
      a.L[i] = int32_t(L);
      if (a.seq_tokens_out) a.seq_tokens_out[i] = int32_t(L);
    }
    return;
  }

  GroupSpec g{};
  g.spp = a.spp;
  g.num_groups = a.num_groups;
  g.offsets = a.offsets;
  g.leave_one_out = a.leave_one_out;
  g.scale_by_std = a.scale_by_std;
  g.std_eps = a.std_eps;
  g.clip = a.clip;
  g.clip_lo = a.clip_lo;
  g.clip_hi = a.clip_hi;
  const float advf = group_advantage<kPrepThreads>(g, a.rewards, i, sh_r);
  if (tid == 0) {
    a.A[i] = advf;
    if (a.adv_out) a.adv_out[i] = advf;
    a.L[i] = int32_t(L);
    if (a.seq_tokens_out) a.seq_tokens_out[i] = int32_t(L);
  }
}

// One block: N = sum L_i, then every w_i.
__global__ __launch_bounds__(kWeightThreads) void grpo_weights_kernel(PrepArgs a) {
  __shared__ long long sh_i64[kWeightThreads / kWave];
  const int tid = threadIdx.x;
  long long n = 0, nc = 0;
  for (int64_t k = tid; k < a.B; k += kWeightThreads) {
    n += a.L[k];
    nc += reduction_count(a.reduction, a.L[k]);
  }
  const long long N = block_sum_i64<kWeightThreads>(n, sh_i64);
  // the reduction's own count (N again, or the live sequences)
  const long long C = a.reduction == GRPO_SEQUENCE_MEAN_LIVE ? block_sum_i64<kWeightThreads>(nc, sh_i64) : N;
  for (int64_t k = tid; k < a.B; k += kWeightThreads) {
    const double wk = sequence_weight(a.reduction, a.alpha, a.norm_constant, a.B, a.L[k], C);
    a.w[k] = wk;
    if (a.seq_weight_out) a.seq_weight_out[k] = float(wk);
  }
  if (tid == 0) {
    a.hdr->num_tokens = N;
    if (N == 0) a.hdr->status |= GRPO_FAULT_NO_TOKENS;
  }
}

hipError_t launch_prep(const PrepArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(grpo_prep_kernel, dim3(unsigned(a.B)), dim3(kPrepThreads), 0, stream, a);
  if (!a.want_weights || !a.weights_kernel) return hipGetLastError();
  hipLaunchKernelGGL(grpo_weights_kernel, dim3(1), dim3(kWeightThreads), 0, stream, a);
  return hipGetLastError();
}

// CSR group offsets reach the device as kernel arguments, kOffsetChunk
// values per launch: a call enqueues kernel launches only (no host-to-device
// copy), so calls with CSR groups can be captured in a HIP graph, and the
// host array is no longer read once the call returns.
constexpr int kOffsetChunk = 240;
struct OffsetChunk {
  int64_t v[kOffsetChunk];
  int32_t n;
};

__global__ __launch_bounds__(256) void grpo_offsets_kernel(OffsetChunk c, int64_t* dst) {
  if (int(threadIdx.x) < c.n) dst[threadIdx.x] = c.v[threadIdx.x];
}

hipError_t launch_copy_offsets(const int64_t* host, int64_t n, int64_t* dev, hipStream_t stream) {
  for (int64_t k0 = 0; k0 < n; k0 += kOffsetChunk) {
    OffsetChunk c;
    c.n = int32_t(n - k0 < kOffsetChunk ? n - k0 : kOffsetChunk);
    for (int32_t j = 0; j < c.n; ++j) c.v[j] = host[k0 + j];
    for (int32_t j = c.n; j < kOffsetChunk; ++j) c.v[j] = 0;
    hipLaunchKernelGGL(grpo_offsets_kernel, dim3(1), dim3(256), 0, stream, c, dev + k0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Workspace clearing (optional: every call initialises what it reads).
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
