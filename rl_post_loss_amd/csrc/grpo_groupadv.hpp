// Group-relative advantage of one sequence, shared by the prep kernel and the
// log-prob token kernel so that both give the same bits.
//
// The group normalisation of "GRPO Loss" (RL-Kernel docs, section Accuracy:
// population std, floored) with the leave-one-out baseline of the
// dockyard_rl design doc (section Advantage estimation) and its optional
// clamp.  Binary64 with contraction off, sums in index order, one rounding
// to float32 at the end.
#pragma once

#include <math.h>

#include "grpo_device.hpp"
#include "grpo_internal.hpp"

namespace grpo {

constexpr int kRewardStage = 1024;  // rewards of one group staged in LDS per round

// Group [s, e) of sequence i.
__device__ inline void group_bounds(const GroupSpec& g, int64_t i, int64_t* s, int64_t* e) {
  if (g.spp > 0) {
    *s = (i / g.spp) * g.spp;
    *e = *s + g.spp;
    return;
  }
  int lo = 0, hi = g.num_groups;  // offsets[lo] <= i < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) / 2;
    if (g.offsets[mid] <= i) lo = mid; else hi = mid;
  }
  *s = g.offsets[lo];
  *e = g.offsets[lo + 1];
}

// A_i from the group's sum S and sum of squared deviations (n values; r_i
// the sequence's own reward), rounded once to float32.
__device__ inline float advantage_value(const GroupSpec& g, double total, double sq, int64_t n,
                                        float r_i) {
#pragma clang fp contract(off)
  const double mean = total / double(n);
  const double sd = sqrt(sq / double(n));
  const double denom = sd >= g.std_eps ? sd : g.std_eps;
  const double ri = double(r_i);
  const double base = g.leave_one_out ? (total - ri) / double(n - 1) : mean;
  const double diff = ri - base;
  double adv = g.scale_by_std ? diff / denom : diff;
  // optional clamp before the one rounding; the comparisons keep a NaN
  if (g.clip) adv = adv < g.clip_lo ? g.clip_lo : (adv > g.clip_hi ? g.clip_hi : adv);
  return float(adv);
}

// A_i, rounded once to float32 (meaningful in thread 0 only).  Every thread of
// the block calls it: the group's rewards are staged in LDS (sh_r holds
// kRewardStage floats) by all threads, and thread 0 forms S = sum r, then
// var = sum (r - mean)^2 / n, sequentially; groups longer than the stage go
// through it in rounds, keeping that order.
template <int NT>
__device__ inline float group_advantage(const GroupSpec& g, const float* rewards, int64_t i,
                                        float* sh_r) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  int64_t s, e;
  group_bounds(g, i, &s, &e);
  const int64_t n = e - s;
  double total = 0.0;
  for (int64_t b = s; b < e; b += kRewardStage) {
    const int64_t m = (e - b) < kRewardStage ? (e - b) : kRewardStage;
    __syncthreads();
    for (int64_t k = tid; k < m; k += NT) sh_r[k] = rewards[b + k];
    __syncthreads();
    if (tid == 0)
      for (int64_t k = 0; k < m; ++k) total = total + double(sh_r[k]);
  }
  double sq = 0.0;
  if (n <= kRewardStage) {
    // the stage still holds the whole group
    if (tid == 0) {
      const double mean = total / double(n);
      for (int64_t k = 0; k < n; ++k) {
        const double dev = double(sh_r[k]) - mean;
        sq = sq + dev * dev;
      }
    }
  } else {
    const double mean_all = total / double(n);  // only thread 0's value is used
    for (int64_t b = s; b < e; b += kRewardStage) {
      const int64_t m = (e - b) < kRewardStage ? (e - b) : kRewardStage;
      __syncthreads();
      for (int64_t k = tid; k < m; k += NT) sh_r[k] = rewards[b + k];
      __syncthreads();
      if (tid == 0)
        for (int64_t k = 0; k < m; ++k) {
          const double dev = double(sh_r[k]) - mean_all;
          sq = sq + dev * dev;
        }
    }
  }
  return tid == 0 ? advantage_value(g, total, sq, n, rewards[i]) : 0.0f;
}

// Thread 0's part when the whole group (n values) already sits in sh_r and
// r_i = sh_r[i - s]: the same sums in the same order as group_advantage.
__device__ inline float group_advantage_staged(const GroupSpec& g, const float* sh_r, int64_t n,
                                               int64_t i_in_group) {
#pragma clang fp contract(off)
  double total = 0.0;
  for (int64_t k = 0; k < n; ++k) total = total + double(sh_r[k]);
  const double mean = total / double(n);
  double sq = 0.0;
  for (int64_t k = 0; k < n; ++k) {
    const double dev = double(sh_r[k]) - mean;
    sq = sq + dev * dev;
  }
  return advantage_value(g, total, sq, n, sh_r[i_in_group]);
}

// Number of nonzero bytes in a 32-bit word.  For each byte b, bit 7 of
// ((b & 0x7f) + 0x7f) | b is set exactly when b != 0 (no carry crosses bytes).
__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
  uint32_t t = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
  return __popc(t);
}

}  // namespace grpo
