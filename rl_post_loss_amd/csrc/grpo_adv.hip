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
// with coalesced loads as they arrive (the terminal reward is added at the
// last active slot, found in the first tile from the right that has an
// active slot, so the mask is read once), thread j folds its kAdvChunk
// consecutive slots into an affine map x -> h + g x of the return after the
// chunk, a suffix scan of those maps (wave shuffles, then the waves in
// order) gives every chunk its carry and the carry into the next tile, every
// chunk replays its slots from its carry, and the returns leave LDS with
// coalesced accesses again.
//
// With the global normalization the returns are kept in binary64 in the
// workspace and each sequence leaves the moments (count, mean, sum of squared
// deviations) of its active values: per thread from sums of deviations
// from its first value, merged across the block in two fixed-order sums.  The output pass then writes (A - mu) x (1 / sd); each of its
// blocks first issues its loads, then forms mu and sd from the sequences'
// moments in fixed-order sums (the same bits in every block, so results
// repeat bit for bit).
// Two launches in all (three beyond kFusedMomentsMaxB sequences, where one
// block merges the moments once).

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_groupadv.hpp"
#include "grpo_internal.hpp"

namespace grpo {

constexpr int kAdvThreads = 256;
// 16 slots per thread (one tile for T = 4,096) measured slower: the extra
// registers halve the waves per SIMD or spill
constexpr int kAdvChunk = 8;                           // consecutive slots per thread in a tile
constexpr int kAdvTile = kAdvThreads * kAdvChunk;      // slots per tile
constexpr int kAdvPad = kAdvChunk + 1;                 // LDS row per thread (bank spread)
constexpr int kMomentThreads = 1024;
constexpr int kGdpoThreads = 1024;

struct AdvShared {
  double v[kAdvThreads * kAdvPad];  // a tile's token rewards, then its returns
  int wmax[kAdvThreads / kWave];    // per wave: its last active tile slot (-1: none)
  double wh[kAdvThreads / kWave];  // per wave: its chunks' composed map (h + g x)
  double wg[kAdvThreads / kWave];
  double red[kAdvThreads / kWave];
  long long red_i[kAdvThreads / kWave];
  double cval;                // baseline difference of the sequence
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
  // the last active slot (it takes the terminal reward), found in the first
  // tile from the right that has an active slot; the same in every thread
  int64_t last = -1;
  const bool shaped = a.kl_coef != 0.0;
  constexpr int kPer = kAdvTile / kAdvThreads;
  constexpr int NW = kAdvThreads / kWave;
  const int lane = tid % kWave, wv = tid / kWave;
  double tile_carry = 0.0;  // return at the slot after the current tile (same in every thread)
  // a tile's inputs in registers: every load of the tile is issued before any
  // is used (loading the next tile during this one's scan measured slower)
  uint32_t mk = 0;  // bit k: slot tid + k NT of the tile is active
  float ov[kPer], rv[kPer];
  auto load_tile = [&](int64_t end) {
    const int64_t start = end > kAdvTile ? end - kAdvTile : 0;
    const int n = int(end - start);
    mk = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = tid + k * kAdvThreads;
      ov[k] = rv[k] = 0.0f;
      if (q < n) {
        if (a.mask == nullptr || a.mask[base + start + q] != 0) mk |= 1u << k;
        if (shaped) {
          ov[k] = a.old[base + start + q];
          rv[k] = a.ref[base + start + q];
        }
      }
    }
  };
  if (T > 0) load_tile(T);
  for (int64_t end = T; end > 0; end -= kAdvTile) {
    const int64_t start = end > kAdvTile ? end - kAdvTile : 0;
    const int n = int(end - start);
    if (end != T) {
      load_tile(end);
      __syncthreads();  // the previous tile's values are consumed
    }
    // token rewards m_t (-kl_coef (old - ref)) go to LDS as soon as they
    // arrive (masked values are discarded by selection); the terminal reward
    // is added at the last active slot once that is known, below
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int q = tid + k * kAdvThreads;
      if (q >= n) continue;
      double v = 0.0;
      if (shaped && ((mk >> k) & 1u)) v = -a.kl_coef * (double(ov[k]) - double(rv[k]));
      sh.v[adv_lds(q)] = v;
    }
    if (last < 0) {
      int qm = -1;
      if (mk != 0) qm = tid + (31 - __builtin_clz(mk)) * kAdvThreads;  // q < n wherever mk is set
      qm = wave_max_i32(qm);
      if (lane == 0) sh.wmax[wv] = qm;
    }
    __syncthreads();  // the tile's rewards and wmax are complete
    if (last < 0) {
      int m = -1;
      for (int w = 0; w < NW; ++w) m = sh.wmax[w] > m ? sh.wmax[w] : m;
      if (m >= 0) {
        last = start + m;
        // r_T = shaped + R at the last active slot: the thread that folds the
        // slot's chunk adds it (nobody else touches that chunk before the
        // next barrier)
        if (m / kAdvChunk == tid) sh.v[adv_lds(m)] = sh.v[adv_lds(m)] + R;
      }
    }
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
    // the mask comes from the registers: thread tid loaded slots tid + k NT
#pragma unroll 2
    for (int k = 0; k < kPer; ++k) {
      const int q = tid + k * kAdvThreads;
      if (q < n) {
        const bool act = (mk >> k) & 1u;
        f(start + q, act, act ? sh.v[adv_lds(q)] : 0.0);
      }
    }
  }
}

// Moments (count, mean, sum of squared deviations) of a set of values.
struct Moments {
  double n, m, M2;
};

// Block sums of two binary64 values through one LDS exchange: the butterfly
// in each wave, then the wave partials in wave order (every thread gets the
// totals).  sh holds 2 * NT / kWave doubles.
template <int NT>
__device__ __forceinline__ void block_sum2_f64(double& x, double& y, double* sh) {
  constexpr int NW = NT / kWave;
  x = wave_sum_f64<kWave>(x);
  y = wave_sum_f64<kWave>(y);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) {
    sh[w] = x;
    sh[NW + w] = y;
  }
  __syncthreads();
  double tx = 0.0, ty = 0.0;
  for (int k = 0; k < NW; ++k) {
    tx += sh[k];
    ty += sh[NW + k];
  }
  x = tx;
  y = ty;
}

// One block per sequence: the raw advantages.  Without normalization they are
// the output; with it, REINFORCE++'s returns go to the workspace and every
// sequence leaves the moments of its active slots' values (the baseline's
// value is the same at every active slot: L_i copies of R_i - group mean).
__global__ __launch_bounds__(kAdvThreads) void grpo_tokadv_kernel(TokAdvArgs a) {
#pragma clang fp contract(off)
  __shared__ AdvShared sh;
  __shared__ double sh_mom[3 * (kAdvThreads / kWave)];
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = i * a.T;
  if (i == 0 && tid == 0) a.hdr->status = 0;

  if (a.estimator != GRPO_ADV_REINFORCE_PP) {
    // group mean (the sample itself included), summed in index order by one
    // thread from rewards the whole block stages in LDS (rounds of kAdvTile)
    GroupSpec g{};
    g.spp = a.spp;
    g.num_groups = a.num_groups;
    g.offsets = a.offsets;
    int64_t s, e;
    group_bounds(g, i, &s, &e);
    float* stage = reinterpret_cast<float*>(sh.v);
    double total = 0.0;
    for (int64_t b = s; b < e; b += kAdvTile) {
      const int64_t m = (e - b) < kAdvTile ? (e - b) : kAdvTile;
      __syncthreads();
      for (int64_t k = tid; k < m; k += kAdvThreads) stage[k] = a.rewards[b + k];
      __syncthreads();
      if (tid == 0)
        for (int64_t k = 0; k < m; ++k) total = total + double(stage[k]);
    }
    if (tid == 0) sh.cval = double(a.rewards[i]) - total / double(e - s);
  }
  __syncthreads();

  if (!a.normalize) {
    for_each_raw(a, i, sh, [&](int64_t t, bool, double v) { a.out[base + t] = float(clamp_adv(a, v)); });
    if (i == 0 && tid == 0 && a.status) *a.status = 0u;
    return;
  }
  if (a.estimator == GRPO_ADV_REINFORCE_PP) {
    // per thread, sums of the deviations from its first value (no division
    // per value, and no cancellation unless that value is an outlier many
    // spreads away); the threads' moments then merge in a fixed tree
    double c = 0.0, s1 = 0.0, s2 = 0.0, n = 0.0;
    for_each_raw(a, i, sh, [&](int64_t t, bool act, double v) {
      if (!act) return;
      a.V[base + t] = v;
      if (n == 0.0) c = v;
      const double d = v - c;
      s1 = s1 + d;
      s2 = s2 + d * d;
      n = n + 1.0;
    });
    Moments mo{0.0, 0.0, 0.0};
    if (n > 0.0) {
      const double dm = s1 / n;
      const double m2 = s2 - s1 * dm;
      mo = Moments{n, c + dm, m2 > 0.0 ? m2 : 0.0};
    }
    {
      // the threads' moments in two block sums: count and n mean give the
      // mean, then M2 = sum (M2_t + n_t (mean_t - mean)^2) (a tree of Chan
      // et al.'s pairwise merges, a division each, measured 1.7 us more per
      // call at 1024 x 4096 and gave the same outputs)
      double sx = mo.n * mo.m, sn = mo.n;
      block_sum2_f64<kAdvThreads>(sx, sn, sh_mom);
      const double mean = sn > 0.0 ? sx / sn : 0.0;
      const double d = mo.m - mean;
      double q = mo.n > 0.0 ? mo.M2 + mo.n * (d * d) : 0.0, unused = 0.0;
      block_sum2_f64<kAdvThreads>(q, unused, sh_mom);
      mo = Moments{sn, mean, q};
    }
    if (tid == 0) {
      a.L[i] = int32_t(mo.n);
      a.mean[i] = mo.m;
      a.M2[i] = mo.M2;
    }
  } else {
    long long cnt = 0;
    if (a.mask == nullptr) {
      cnt = tid == 0 ? a.T : 0;
    } else if (a.T % 4 == 0 && (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0) {
      const uint32_t* w4 = reinterpret_cast<const uint32_t*>(a.mask + base);
      for (int64_t k = tid; k < a.T / 4; k += kAdvThreads) cnt += nonzero_bytes(w4[k]);
    } else {
      for (int64_t t = tid; t < a.T; t += kAdvThreads) cnt += a.mask[base + t] != 0 ? 1 : 0;
    }
    cnt = block_sum_i64<kAdvThreads>(cnt, sh.red_i);
    if (tid == 0) {
      a.L[i] = int32_t(cnt);
      a.mean[i] = sh.cval;
      a.M2[i] = 0.0;
    }
  }
}

// (v - mu) / sd as a product with the binary64 reciprocal of sd, formed once
// per block: a division per slot measured 1.1-1.3 us more per call.  The
// product is within one binary64 ulp of the quotient, so after the rounding
// to float32 the two differ only where the quotient lies that close to a
// float32 rounding boundary.
__device__ __forceinline__ double adv_scale(double v, double mu, double inv) {
#pragma clang fp contract(off)
  return (v - mu) * inv;
}

constexpr int kNormThreads = 256;
#ifndef GRPO_NORM_QUADS
#define GRPO_NORM_QUADS 4
#endif
constexpr int kNormQuads = GRPO_NORM_QUADS;  // quads of 4 slots per thread
// Up to this many sequences every block of the output pass merges the
// sequences' moments itself (no separate one-block kernel and launch);
// beyond it the merge runs once in grpo_tokadv_moments_kernel.
constexpr int64_t kFusedMomentsMaxB = 4096;
#ifndef GRPO_MERGE_BATCH
#define GRPO_MERGE_BATCH 4
#endif
constexpr int kMergeBatch = GRPO_MERGE_BATCH;  // sequences per thread per batch of loads

// mu and the floored sd of the global masked normalization from the
// sequences' moments (count L_i, mean_i, sum of squared deviations M2_i), in
// fixed-order sums: every block that runs it holds the same bits; with
// `publish` it also stores the count, the moments and the no-token fault in
// the header.
template <int NT>
__device__ void merge_global_moments(const TokAdvArgs& a, double* sh_mom, double* sh_out,
                                     bool publish) {
#pragma clang fp contract(off)
  const int tid = threadIdx.x;
  // N and sum_i L_i mean_i give mu; then M2 = sum_i (M2_i + L_i (mean_i - mu)^2),
  // every term non-negative; thread t takes sequences t, t + NT, ... in order.
  // (Chan et al.'s pairwise merge in a shuffle tree, a division per merge,
  // measured 0.7 us more per call at B = 1024 and gave the same outputs.)
  // The loads go in batches of kMergeBatch sequences per thread, every load
  // of a batch issued before any is used (a load after each test of L_i made
  // a chain of dependent cache round trips); the first batch stays in
  // registers for the second sum.  Per thread the order of the terms is the
  // sequence order either way.
  constexpr int kB = kMergeBatch;
  auto load = [&](int64_t k0, int32_t* n, double* m, double* q2) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int64_t k = k0 + int64_t(u) * NT;
      const bool in = k < a.B;
      n[u] = in ? a.L[k] : 0;
      m[u] = in ? a.mean[k] : 0.0;
      q2[u] = in ? a.M2[k] : 0.0;
    }
  };
  auto add_first = [&](const int32_t* n, const double* m, double& s, double& cnt) {
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (n[u] > 0) {
        s = s + double(n[u]) * m[u];
        cnt = cnt + double(n[u]);
      }
  };
  auto add_second = [&](const int32_t* n, const double* m, const double* q2, double mu, double& q) {
#pragma unroll
    for (int u = 0; u < kB; ++u)
      if (n[u] > 0) {
        const double d = m[u] - mu;
        q = q + (q2[u] + double(n[u]) * (d * d));
      }
  };
  constexpr int64_t kStride = int64_t(NT) * kB;
  int32_t n0[kB];
  double m0[kB], q0[kB];
  load(tid, n0, m0, q0);
  double s = 0.0, cnt = 0.0;
  add_first(n0, m0, s, cnt);
  for (int64_t k0 = tid + kStride; k0 < a.B; k0 += kStride) {
    int32_t n[kB];
    double m[kB], q2[kB];
    load(k0, n, m, q2);
    add_first(n, m, s, cnt);
  }
  block_sum2_f64<NT>(s, cnt, sh_mom);
  const double mu = cnt > 0.0 ? s / cnt : 0.0;
  double q = 0.0, unused = 0.0;
  add_second(n0, m0, q0, mu, q);
  for (int64_t k0 = tid + kStride; k0 < a.B; k0 += kStride) {
    int32_t n[kB];
    double m[kB], q2[kB];
    load(k0, n, m, q2);
    add_second(n, m, q2, mu, q);
  }
  block_sum2_f64<NT>(q, unused, sh_mom);
  if (tid == 0) {
    const double var = cnt > 0.0 ? q / cnt : 0.0;
    const double sd = sqrt(var > 1e-8 ? var : 1e-8);
    sh_out[0] = mu;
    sh_out[1] = sd;
    if (publish) {
      a.hdr->num_tokens = (long long)cnt;
      a.hdr->mu = mu;
      a.hdr->sd = sd;
      if (cnt == 0.0) a.hdr->status |= GRPO_FAULT_NO_TOKENS;
    }
  }
  __syncthreads();
}

// One block: the batch's moments from the sequences' (beyond
// kFusedMomentsMaxB sequences, where every output block merging them would
// cost more than this launch); mu and the floored std for the output pass.
__global__ __launch_bounds__(kMomentThreads) void grpo_tokadv_moments_kernel(TokAdvArgs a) {
  __shared__ double sh_mom[3 * (kMomentThreads / kWave)];
  __shared__ double sh_out[2];
  merge_global_moments<kMomentThreads>(a, sh_mom, sh_out, true);
}

// Output pass over the slots: (A - mu) / sd at active slots, 0 elsewhere;
// kNormQuads quads of four slots per thread when the rows allow 16-byte
// accesses, else one slot per thread.  kFused: mu and sd from the
// sequences' moments, merged by every block (block 0 publishes them).
template <bool kFused>
__global__ __launch_bounds__(kNormThreads) void grpo_tokadv_norm_kernel(TokAdvArgs a, int vec) {
#pragma clang fp contract(off)
  __shared__ double sh_mom[3 * (kNormThreads / kWave)];
  __shared__ double sh_musd[2];
  double mu = 0.0, sd = 1.0;
  if constexpr (!kFused) {
    mu = a.hdr->mu;
    sd = a.hdr->sd;
  }
  const bool rpp = a.estimator == GRPO_ADV_REINFORCE_PP;
  const int64_t rows = a.B * a.T;
  if (vec) {
    const int64_t nq = rows / 4;
    const int64_t q0 = int64_t(blockIdx.x) * (kNormThreads * kNormQuads) + threadIdx.x;
    uint32_t m4[kNormQuads];
    f32x4 lo[kNormQuads], hi[kNormQuads];
#pragma unroll
    for (int u = 0; u < kNormQuads; ++u) {
      const int64_t q = q0 + int64_t(u) * kNormThreads;
      m4[u] = q < nq ? (a.mask ? *reinterpret_cast<const uint32_t*>(a.mask + 4 * q) : 0x01010101u) : 0u;
    }
    if (rpp) {
      // a quad with no active slot reads the first slot's line instead (its
      // values are not used), so that the loads need no branch
#pragma unroll
      for (int u = 0; u < kNormQuads; ++u) {
        const int64_t src = m4[u] != 0 ? 4 * (q0 + int64_t(u) * kNormThreads) : 0;
        lo[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.V + src));
        hi[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.V + src + 2));
      }
    }
    if constexpr (kFused) {
      // the merge runs while this block's loads are in flight
      merge_global_moments<kNormThreads>(a, sh_mom, sh_musd, blockIdx.x == 0);
      mu = sh_musd[0];
      sd = sh_musd[1];
    }
    const double inv = 1.0 / sd;
#pragma unroll
    for (int u = 0; u < kNormQuads; ++u) {
      const int64_t q = q0 + int64_t(u) * kNormThreads;
      if (q >= nq) continue;
      double v[4];
      if (rpp) {
        v[0] = __builtin_bit_cast(double, f2{lo[u].x, lo[u].y});
        v[1] = __builtin_bit_cast(double, f2{lo[u].z, lo[u].w});
        v[2] = __builtin_bit_cast(double, f2{hi[u].x, hi[u].y});
        v[3] = __builtin_bit_cast(double, f2{hi[u].z, hi[u].w});
      } else {
        v[0] = v[1] = v[2] = v[3] = a.mean[(4 * q) / a.T];
      }
      float o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = ((m4[u] >> (8 * j)) & 0xffu) ? float(clamp_adv(a, adv_scale(v[j], mu, inv))) : 0.0f;
      __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(a.out + 4 * q));
    }
    if (q0 == 0 && a.status) *a.status = a.hdr->status;  // block 0, after it published
  } else {
    if constexpr (kFused) {
      merge_global_moments<kNormThreads>(a, sh_mom, sh_musd, blockIdx.x == 0);
      mu = sh_musd[0];
      sd = sh_musd[1];
    }
    const double inv = 1.0 / sd;
    const int64_t gid = int64_t(blockIdx.x) * kNormThreads + threadIdx.x;
    if (gid >= rows) return;
    const bool act = adv_active(a, gid);
    float o = 0.0f;
    if (act) {
      const double v = rpp ? a.V[gid] : a.mean[gid / a.T];
      o = float(clamp_adv(a, adv_scale(v, mu, inv)));
    }
    a.out[gid] = o;
    if (gid == 0 && a.status) *a.status = a.hdr->status;
  }
}

hipError_t launch_token_advantages(const TokAdvArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(grpo_tokadv_kernel, dim3(unsigned(a.B)), dim3(kAdvThreads), 0, s, a);
  if (!a.normalize) return hipGetLastError();
  const bool fused = a.B <= kFusedMomentsMaxB;
  if (!fused) hipLaunchKernelGGL(grpo_tokadv_moments_kernel, dim3(1), dim3(kMomentThreads), 0, s, a);
  const int64_t rows = a.B * a.T;
  const int vec = (a.T % 4 == 0 && (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.out) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.V) & 15) == 0) ? 1 : 0;
  const int64_t per_block = vec ? int64_t(kNormThreads) * kNormQuads : int64_t(kNormThreads);
  const int64_t items = vec ? rows / 4 : rows;
  const int64_t blocks = (items + per_block - 1) / per_block;
  if (fused)
    hipLaunchKernelGGL(grpo_tokadv_norm_kernel<true>, dim3(unsigned(blocks)), dim3(kNormThreads),
                       0, s, a, vec);
  else
    hipLaunchKernelGGL(grpo_tokadv_norm_kernel<false>, dim3(unsigned(blocks)), dim3(kNormThreads),
                       0, s, a, vec);
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
