// Token-level and multi-reward advantage estimators.
//
// REINFORCE++ and REINFORCE++-baseline follow the Relax docs page
// "REINFORCE++ and REINFORCE++-baseline" (sections REINFORCE++,
// REINFORCE++-baseline, Global masked normalization):
//   REINFORCE++  token reward r_t = m_t (-kl_coef (old_t - ref_t) + [t = T_i] R_i),
//                return A_t = m_t sum_{u >= t} gamma^(u - t) r_u;
//   baseline     A_t = m_t (R_i - mean of R over i's group, i included);
// then optionally A <- (A - mu) / sqrt(max(var, 1e-8)) with the population
// moments of every active slot of the batch.  GDPO follows the dockyard_rl
// design doc (GDPO multi-reward advantage): a per-component group baseline,
// summed over components, renormalised over the batch.
//
// Everything is binary64 with contraction off and rounded once to float32.
// The returns run as a tiled backward scan: a sequence's block walks tiles of
// kAdvTile slots from the right end; a tile's token rewards are staged in LDS
// with coalesced loads, thread j folds its kAdvChunk consecutive slots into
// an affine map x -> h + g x of the return after the chunk, a suffix scan of
// those maps (wave shuffles, then the waves in order) gives every chunk its
// carry and the carry into the next tile, every chunk replays its slots from
// its carry, and the returns leave LDS with coalesced accesses again.  Sums over slots are fixed trees, sums over
// sequences a single block, so results repeat bit for bit.

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_internal.hpp"

namespace grpo {

constexpr int kAdvThreads = 256;
constexpr int kAdvChunk = 8;                           // consecutive slots per thread in a tile
constexpr int kAdvTile = kAdvThreads * kAdvChunk;      // slots per tile
constexpr int kAdvPad = kAdvChunk + 1;                 // LDS row per thread (bank spread)
constexpr int kMomentThreads = 1024;
constexpr int kGdpoThreads = 1024;

struct AdvShared {
  double v[kAdvThreads * kAdvPad];  // a tile's token rewards, then its returns
  uint8_t act[kAdvTile];            // a tile's mask
  double wh[kAdvThreads / kWave];  // per wave: its chunks' composed map (h + g x)
  double wg[kAdvThreads / kWave];
  double red[kAdvThreads / kWave];
  long long red_i[kAdvThreads / kWave];
  double cval;                // baseline difference of the sequence
  long long last;             // last active slot (-1: none)
};

// LDS index of tile slot q (thread q / kAdvChunk owns kAdvChunk consecutive slots)
__device__ __forceinline__ int adv_lds(int q) { return (q / kAdvChunk) * kAdvPad + q % kAdvChunk; }

__device__ __forceinline__ bool adv_active(const TokAdvArgs& a, int64_t r) {
  return a.mask == nullptr || a.mask[r] != 0;
}

__device__ __forceinline__ double clamp_adv(const TokAdvArgs& a, double v) {
  if (!a.clip) return v;
  return v < a.clip_lo ? a.clip_lo : (v > a.clip_hi ? a.clip_hi : v);  // keeps a NaN
}

// Calls f(t, active, A_t) once for every slot t of sequence i (A_t the raw
// advantage, 0 at masked slots); each thread visits slots t = tile start +
// threadIdx.x + k * blockDim.x, tiles from the right end.  All threads of
// the block must call it.
template <typename F>
__device__ void for_each_raw(const TokAdvArgs& a, int64_t i, AdvShared& sh, F&& f) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  const int64_t T = a.T, base = i * a.T;
  if (a.estimator == GRPO_ADV_REINFORCE_PP_BASELINE) {
    const double c = sh.cval;
    constexpr int U = 8;
    for (int64_t t0 = tid; t0 < T; t0 += int64_t(U) * kAdvThreads) {
      bool act[U];
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t t = t0 + int64_t(k) * kAdvThreads;
        act[k] = t < T && adv_active(a, base + t);
      }
#pragma unroll
      for (int k = 0; k < U; ++k) {
        const int64_t t = t0 + int64_t(k) * kAdvThreads;
        if (t < T) f(t, act[k], act[k] ? c : 0.0);
      }
    }
    return;
  }
  const double R = double(a.rewards[i]);
  const long long last = sh.last;
  const bool shaped = a.kl_coef != 0.0;
  constexpr int kPer = kAdvTile / kAdvThreads;
  constexpr int NW = kAdvThreads / kWave;
  const int lane = tid % kWave, wv = tid / kWave;
  double tile_carry = 0.0;  // return at the slot after the current tile (same in every thread)
  for (int64_t end = T; end > 0; end -= kAdvTile) {
    const int64_t start = end > kAdvTile ? end - kAdvTile : 0;
    const int n = int(end - start);
    __syncthreads();  // the previous tile's values are consumed
    // token rewards r_t = m_t (-kl_coef (old - ref) + [t = T_i] R): every load of
    // the tile is issued before any is used; masked values are discarded by selection
    uint8_t mk[kPer];
    float ov[kPer], rv[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = tid + k * kAdvThreads;
      mk[k] = 0;
      ov[k] = rv[k] = 0.0f;
      if (q < n) {
        mk[k] = a.mask ? a.mask[base + start + q] : 1;
        if (shaped) {
          ov[k] = a.old[base + start + q];
          rv[k] = a.ref[base + start + q];
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = tid + k * kAdvThreads;
      if (q >= n) continue;
      const bool act = mk[k] != 0;
      double v = 0.0;
      if (act) {
        if (shaped) v = -a.kl_coef * (double(ov[k]) - double(rv[k]));
        if (start + q == last) v = v + R;
      }
      sh.v[adv_lds(q)] = v;
      sh.act[q] = act ? 1 : 0;
    }
    __syncthreads();
    // this thread's chunk as an affine map x -> h + g x of the return after it
    const int q0 = tid * kAdvChunk < n ? tid * kAdvChunk : n;
    const int q1 = q0 + kAdvChunk < n ? q0 + kAdvChunk : n;
    double h = 0.0, g = 1.0;
    for (int q = q1 - 1; q >= q0; --q) {
      h = sh.v[adv_lds(q)] + a.gamma * h;
      g = g * a.gamma;
    }
    // suffix scan of the maps (chunk j composed with chunks j+1 ...): in the
    // wave, then across waves, in a fixed tree
    double sh_ = h, sg = g;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const double oh = __shfl_down(sh_, off), og = __shfl_down(sg, off);
      if (lane + off < kWave) {
        sh_ = sh_ + sg * oh;
        sg = sg * og;
      }
    }
    if (lane == 0) {
      sh.wh[wv] = sh_;
      sh.wg[wv] = sg;
    }
    __syncthreads();
    // the map of the waves after this one, applied to the tile's carry
    double x = tile_carry;
    for (int w = NW - 1; w > wv; --w) x = sh.wh[w] + sh.wg[w] * x;
    // exclusive suffix in the wave: the next lane's inclusive map
    double nh = __shfl_down(sh_, 1), ng = __shfl_down(sg, 1);
    if (lane == kWave - 1) {
      nh = 0.0;
      ng = 1.0;
    }
    double acc = nh + ng * x;  // return at the slot after this chunk
    // the carry into the next tile: the whole tile's map applied to tile_carry
    double tc = tile_carry;
    for (int w = NW - 1; w >= 0; --w) tc = sh.wh[w] + sh.wg[w] * tc;
    tile_carry = tc;
    for (int q = q1 - 1; q >= q0; --q) {
      acc = sh.v[adv_lds(q)] + a.gamma * acc;
      sh.v[adv_lds(q)] = acc;
    }
    __syncthreads();
    for (int q = tid; q < n; q += kAdvThreads) {
      const bool act = sh.act[q] != 0;
      f(start + q, act, act ? sh.v[adv_lds(q)] : 0.0);
    }
  }
}

// One block per sequence; a.pass selects the work (see TokAdvArgs).
__global__ __launch_bounds__(kAdvThreads) void grpo_tokadv_kernel(TokAdvArgs a) {
#pragma clang fp contract(off)
  __shared__ AdvShared sh;
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = i * a.T;
  if (i == 0 && tid == 0 && a.pass == 0) a.hdr->status = 0;

  if (a.estimator == GRPO_ADV_REINFORCE_PP) {
    if (a.pass == 0) {
      // last active slot of the sequence, kept for the later passes
      long long mx = -1;
      constexpr int U = 8;
      for (int64_t t0 = tid; t0 < a.T; t0 += int64_t(U) * kAdvThreads) {
        bool act[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
          const int64_t t = t0 + int64_t(k) * kAdvThreads;
          act[k] = t < a.T && adv_active(a, base + t);
        }
#pragma unroll
        for (int k = 0; k < U; ++k)
          if (act[k]) mx = t0 + int64_t(k) * kAdvThreads;
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) {
        const long long o = __shfl_xor(mx, off);
        mx = o > mx ? o : mx;
      }
      if (tid % kWave == 0) sh.red_i[tid / kWave] = mx;
      __syncthreads();
      if (tid == 0) {
        long long m = -1;
        for (int k = 0; k < kAdvThreads / kWave; ++k) m = sh.red_i[k] > m ? sh.red_i[k] : m;
        sh.last = m;
        a.last[i] = m;
      }
    } else if (tid == 0) {
      sh.last = a.last[i];
    }
  } else if (tid == 0) {
    // group mean (the sample itself included), summed in index order
    int64_t s, e;
    if (a.spp > 0) {
      s = (i / a.spp) * a.spp;
      e = s + a.spp;
    } else {
      int lo = 0, hi = a.num_groups;
      while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (a.offsets[mid] <= i) lo = mid; else hi = mid;
      }
      s = a.offsets[lo];
      e = a.offsets[lo + 1];
    }
    double total = 0.0;
    for (int64_t j = s; j < e; ++j) total = total + double(a.rewards[j]);
    sh.cval = double(a.rewards[i]) - total / double(e - s);
  }
  __syncthreads();

  if (a.pass == 0 && !a.normalize) {
    for_each_raw(a, i, sh, [&](int64_t t, bool, double v) { a.out[base + t] = float(clamp_adv(a, v)); });
    if (i == 0 && tid == 0 && a.status) *a.status = 0u;
    return;
  }
  if (a.pass == 2) {
    const double mu = a.hdr->mu, sd = a.hdr->sd;
    for_each_raw(a, i, sh, [&](int64_t t, bool act, double v) {
      a.out[base + t] = act ? float(clamp_adv(a, (v - mu) / sd)) : 0.0f;
    });
    if (i == 0 && tid == 0 && a.status) *a.status = a.hdr->status;
    return;
  }
  // pass 0: sum and count; pass 1: squared deviations from the mean
  const double mu = a.pass == 1 ? a.hdr->mu : 0.0;
  double sum = 0.0;
  long long cnt = 0;
  for_each_raw(a, i, sh, [&](int64_t, bool act, double v) {
    if (!act) return;
    if (a.pass == 0) {
      sum = sum + v;
      ++cnt;
    } else {
      const double dv = v - mu;
      sum = sum + dv * dv;
    }
  });
  sum = block_sum_f64<kAdvThreads>(sum, sh.red);
  cnt = block_sum_i64<kAdvThreads>(cnt, sh.red_i);
  if (tid == 0) {
    a.S[i] = sum;
    if (a.pass == 0) a.L[i] = int32_t(cnt);
  }
}

// One block: pass 0 -> N and the mean; pass 1 -> the floored std.
__global__ __launch_bounds__(kMomentThreads) void grpo_tokadv_moments_kernel(TokAdvArgs a) {
#pragma clang fp contract(off)
  __shared__ double sh_f64[kMomentThreads / kWave];
  __shared__ long long sh_i64[kMomentThreads / kWave];
  const int tid = threadIdx.x;
  double s = 0.0;
  long long n = 0;
  for (int64_t k = tid; k < a.B; k += kMomentThreads) {
    s = s + a.S[k];
    n += a.L[k];
  }
  s = block_sum_f64<kMomentThreads>(s, sh_f64);
  n = block_sum_i64<kMomentThreads>(n, sh_i64);
  if (tid != 0) return;
  if (a.pass == 0) {
    a.hdr->num_tokens = n;
    a.hdr->mu = n > 0 ? s / double(n) : 0.0;
    if (n == 0) a.hdr->status |= GRPO_FAULT_NO_TOKENS;
  } else {
    const double var = n > 0 ? s / double(n) : 0.0;
    a.hdr->sd = sqrt(var > 1e-8 ? var : 1e-8);
  }
}

hipError_t launch_token_advantages(const TokAdvArgs& base, hipStream_t s) {
  TokAdvArgs a = base;
  const dim3 grid(unsigned(a.B));
  a.pass = 0;
  hipLaunchKernelGGL(grpo_tokadv_kernel, grid, dim3(kAdvThreads), 0, s, a);
  if (!a.normalize) return hipGetLastError();
  hipLaunchKernelGGL(grpo_tokadv_moments_kernel, dim3(1), dim3(kMomentThreads), 0, s, a);
  a.pass = 1;
  hipLaunchKernelGGL(grpo_tokadv_kernel, grid, dim3(kAdvThreads), 0, s, a);
  hipLaunchKernelGGL(grpo_tokadv_moments_kernel, dim3(1), dim3(kMomentThreads), 0, s, a);
  a.pass = 2;
  hipLaunchKernelGGL(grpo_tokadv_kernel, grid, dim3(kAdvThreads), 0, s, a);
  return hipGetLastError();
}

// GDPO: thread g forms group g's per-component advantages (sums in member
// order, as the group-relative advantages do) and adds them up in component
// order; then the block renormalises the totals over the batch.
__global__ __launch_bounds__(kGdpoThreads) void grpo_gdpo_kernel(GdpoArgs a) {
#pragma clang fp contract(off)
  __shared__ double sh_f64[kGdpoThreads / kWave];
  const int tid = threadIdx.x;
  const int64_t G = a.spp > 0 ? a.B / a.spp : int64_t(a.num_groups);
  for (int64_t g = tid; g < G; g += kGdpoThreads) {
    const int64_t s0 = a.spp > 0 ? g * a.spp : a.offsets[g];
    const int64_t e0 = a.spp > 0 ? s0 + a.spp : a.offsets[g + 1];
    const int64_t n = e0 - s0;
    for (int64_t j = s0; j < e0; ++j) a.total[j] = 0.0;
    for (int c = 0; c < a.C; ++c) {
      const float* r = a.rewards + int64_t(c) * a.B;
      double S = 0.0;
      for (int64_t j = s0; j < e0; ++j) S = S + double(r[j]);
      const double mean = S / double(n);
      double sq = 0.0;
      for (int64_t j = s0; j < e0; ++j) {
        const double dev = double(r[j]) - mean;
        sq = sq + dev * dev;
      }
      const double sd = sqrt(sq / double(n));
      const double denom = sd >= a.std_eps ? sd : a.std_eps;
      for (int64_t j = s0; j < e0; ++j) {
        const double rj = double(r[j]);
        const double b = a.leave_one_out ? (S - rj) / double(n - 1) : mean;
        const double diff = rj - b;
        a.total[j] = a.total[j] + (a.scale_by_std ? diff / denom : diff);
      }
    }
  }
  __syncthreads();
  double s = 0.0;
  for (int64_t j = tid; j < a.B; j += kGdpoThreads) s = s + a.total[j];
  const double mu = block_sum_f64<kGdpoThreads>(s, sh_f64) / double(a.B);
  double q = 0.0;
  for (int64_t j = tid; j < a.B; j += kGdpoThreads) {
    const double dv = a.total[j] - mu;
    q = q + dv * dv;
  }
  const double sd = sqrt(block_sum_f64<kGdpoThreads>(q, sh_f64) / double(a.B));
  const double denom = sd >= a.std_eps ? sd : a.std_eps;
  for (int64_t j = tid; j < a.B; j += kGdpoThreads) {
    double v = (a.total[j] - mu) / denom;
    if (a.clip) v = v < a.clip_lo ? a.clip_lo : (v > a.clip_hi ? a.clip_hi : v);
    a.out[j] = float(v);
  }
}

hipError_t launch_gdpo(const GdpoArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(grpo_gdpo_kernel, dim3(1), dim3(kGdpoThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace grpo
