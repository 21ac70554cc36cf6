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
// as they arrive (the terminal reward is added at the last active slot,
// found in the first tile from the right that has an active slot, so the
// mask is read once), every thread folds one chunk of kAdvChunk consecutive
// slots into an affine map x -> h + g x of the return after the chunk, a
// scan of those maps (DPP lane patterns within a wave, then the waves in
// order) gives every chunk its carry and the carry into the next tile,
// every chunk replays its slots from its carry, and the returns leave LDS.
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
  long long red_i[kAdvThreads / kWave];
  double cval;                // baseline difference of the sequence
};

// LDS index of tile slot q (chunk q / kAdvChunk: kAdvChunk consecutive slots)
__device__ __forceinline__ int adv_lds(int q) { return (q / kAdvChunk) * kAdvPad + q % kAdvChunk; }

__device__ __forceinline__ bool adv_active(const TokAdvArgs& a, int64_t r) {
  return a.mask == nullptr || a.mask[r] != 0;
}

__device__ __forceinline__ double clamp_adv(const TokAdvArgs& a, double v) {
  if (!a.clip) return v;
  return v < a.clip_lo ? a.clip_lo : (v > a.clip_hi ? a.clip_hi : v);  // keeps a NaN
}

// The baseline's raw advantage at every slot of sequence i: f(t, active, A_t)
// with A_t = c at active slots and 0 elsewhere; thread j visits slots
// j + k * blockDim.x.  All threads of the block must call it.
template <typename F>
__device__ void for_each_baseline(const TokAdvArgs& a, int64_t i, double c, F&& f) {
  const int tid = threadIdx.x;
  const int64_t T = a.T, base = i * a.T;
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

// A thread's moments from sums of the deviations from its first value (no
// division per value, and no cancellation unless that value is an outlier
// many spreads away), then the block's in two fixed-order sums: count and
// n mean give the mean, then M2 = sum (M2_t + n_t (mean_t - mean)^2).  (A
// tree of Chan et al.'s pairwise merges, a division each, measured 1.7 us
// more per call at 1024 x 4096 and gave the same outputs.)  Sequence i's
// moments go to L, mean and M2.
struct MomentSums {
  double c = 0.0, s1 = 0.0, s2 = 0.0, n = 0.0;
  __device__ __forceinline__ void add(double v) {
#pragma clang fp contract(off)
    if (n == 0.0) c = v;
    const double d = v - c;
    s1 = s1 + d;
    s2 = s2 + d * d;
    n = n + 1.0;
  }
};

__device__ void store_sequence_moments(const TokAdvArgs& a, int64_t i, const MomentSums& ms,
                                       double* sh_mom) {
#pragma clang fp contract(off)
  Moments mo{0.0, 0.0, 0.0};
  if (ms.n > 0.0) {
    const double dm = ms.s1 / ms.n;
    const double m2 = ms.s2 - ms.s1 * dm;
    mo = Moments{ms.n, ms.c + dm, m2 > 0.0 ? m2 : 0.0};
  }
  double sx = mo.n * mo.m, sn = mo.n;
  block_sum2_f64<kAdvThreads>(sx, sn, sh_mom);
  const double mean = sn > 0.0 ? sx / sn : 0.0;
  const double d = mo.m - mean;
  double q = mo.n > 0.0 ? mo.M2 + mo.n * (d * d) : 0.0, unused = 0.0;
  block_sum2_f64<kAdvThreads>(q, unused, sh_mom);
  if (threadIdx.x == 0) {
    a.L[i] = int32_t(sn);
    a.mean[i] = mean;
    a.M2[i] = q;
  }
}

// REINFORCE++-baseline, one block per sequence: C_i = R_i - (group mean, i
// included).  Without normalization the output is written here; with it,
// the sequence leaves L_i (its active slots), mean C_i and M2 = 0 (L_i
// copies of one value) for the output pass.
__global__ __launch_bounds__(kAdvThreads) void grpo_tokadv_kernel(TokAdvArgs a) {
#pragma clang fp contract(off)
  __shared__ AdvShared sh;
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = i * a.T;
  if (i == 0 && tid == 0) a.hdr->status = 0;

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
  __syncthreads();
  const double c = sh.cval;

  if (!a.normalize) {
    for_each_baseline(a, i, c, [&](int64_t t, bool, double v) { a.out[base + t] = float(clamp_adv(a, v)); });
    if (i == 0 && tid == 0 && a.status) *a.status = 0u;
    return;
  }
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
    a.mean[i] = c;
    a.M2[i] = 0.0;
  }
}

// --- REINFORCE++ returns -----------------------------------------------------
// A chunk's returns depend on the return after it through an affine map
// x -> h + g x (h: the chunk's discounted rewards, g: gamma to the chunk's
// length); the map of a run of chunks is the composition
// (h, g) o (h', g') = (h + g h', g g'), the left map belonging to the chunk
// further left.

// A binary64 value moved between lanes by a DPP lane pattern (both halves);
// lanes whose source lies outside the pattern, or whose row the row mask
// leaves out, take `old`.  Every lane of the wave must be active.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ double dpp_f64(double x, double old) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(old), __double2loint(x), CTRL, ROWMASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(old), __double2hiint(x), CTRL, ROWMASK, 0xF, false);
  return __hiloint2double(hi, lo);
}

// One step of the inclusive lane-order scan of chunk maps: this lane's map is
// composed with the one the pattern selects from a lower lane (a chunk
// further right).  Unselected lanes compose with (-0, 1), which is exact:
// h + g (-0) = h for every g >= 0, and g 1 = g.
template <int CTRL, int ROWMASK, bool kG1>
__device__ __forceinline__ void map_scan_step(double& h, double& g) {
#pragma clang fp contract(off)
  const double oh = dpp_f64<CTRL, ROWMASK>(h, -0.0);
  if constexpr (kG1) {
    h = h + oh;  // g = 1 throughout: the same bits as h + 1 oh
  } else {
    const double og = dpp_f64<CTRL, ROWMASK>(g, 1.0);
    h = h + g * oh;
    g = g * og;
  }
}

// Inclusive scan over the wave's lanes, lane 0 first: row shifts by 1, 2, 4
// and 8 within each row of 16 lanes, then row 0's last lane into row 1 and
// row 2's into row 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31).  Lane l ends with the composition of lanes l, l-1, ..., 0.
template <bool kG1>
__device__ __forceinline__ void wave_map_scan(double& h, double& g) {
  map_scan_step<0x111, 0xF, kG1>(h, g);
  map_scan_step<0x112, 0xF, kG1>(h, g);
  map_scan_step<0x114, 0xF, kG1>(h, g);
  map_scan_step<0x118, 0xF, kG1>(h, g);
  map_scan_step<0x142, 0xA, kG1>(h, g);
  map_scan_step<0x143, 0xC, kG1>(h, g);
}

typedef double d2 __attribute__((ext_vector_type(2)));

// REINFORCE++, one block per sequence: tiles of kAdvTile slots from the right
// end.  A tile's token rewards m_t (-kl_coef (old - ref)) go to LDS (the
// terminal reward is added at the last active slot, found in the first tile
// from the right that has one, so the mask is read once); thread j folds
// chunk own(j) = 64 w + 63 - l (w its wave, l its lane) of kAdvChunk
// consecutive slots into its map.  Chunks run right to left across a wave's
// lanes, so the suffix scan over chunks is a prefix scan over lanes (DPP row
// shifts and row broadcasts, no LDS traffic); the waves' maps then compose
// in wave order, every chunk replays its slots from its carry, and the
// returns leave LDS.  kVec: T % 4 == 0 and 16-byte aligned rows, so each
// thread loads and stores quads of four consecutive slots (tile slots
// 4 (j + 256 u) + c, u = 0, 1); otherwise single slots j + 256 k.  kG1:
// gamma = 1, where every slope is exactly 1 and is not carried (the same
// bits as the general maps).  Without normalization the advantages are
// written here; with it, the returns of active slots go to V and the
// sequence leaves the moments of its active returns.
template <bool kVec, bool kG1>
__global__ __launch_bounds__(kAdvThreads) void grpo_tokadv_returns_kernel(TokAdvArgs a) {
#pragma clang fp contract(off)
  __shared__ AdvShared sh;
  __shared__ double sh_mom[2 * (kAdvThreads / kWave)];
  constexpr int NW = kAdvThreads / kWave;
  constexpr int kBits = kAdvTile / kAdvThreads;  // slots per thread per tile
  static_assert(kBits == 8 && kAdvChunk == 8, "two quads or eight slots per thread");
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  const int64_t T = a.T, base = i * T;
  if (i == 0 && tid == 0) a.hdr->status = 0;
  const double R = double(a.rewards[i]);
  const bool shaped = a.kl_coef != 0.0;
  const double gam = kG1 ? 1.0 : a.gamma;
  const int own = wv * kWave + (kWave - 1 - lane);
  // slope of a full chunk: kAdvChunk factors of gamma in the partial fold's order
  double g_full = 1.0;
  if constexpr (!kG1)
    for (int j = 0; j < kAdvChunk; ++j) g_full = g_full * gam;
  // tile slot of bit b of this thread's mask word (increasing in b)
  auto slot = [&](int b) -> int {
    return kVec ? 4 * (tid + kAdvThreads * (b >> 2)) + (b & 3) : tid + kAdvThreads * b;
  };
  int64_t last = -1;
  double tile_carry = 0.0;  // return at the slot after the current tile (same in every thread)
  MomentSums ms;
  for (int64_t end = T; end > 0; end -= kAdvTile) {
    const int64_t start = end > kAdvTile ? end - kAdvTile : 0;
    const int n = int(end - start);  // a multiple of 4 when kVec
    const int64_t row0 = base + start;
    // the tile's mask bits and log-probs: every load issued before any is used
    uint32_t mk = 0;  // bit b: slot(b) is active
    float ov[kBits], rv[kBits];
    if constexpr (kVec) {
      uint32_t m4[2];
      f32x4 o4[2], r4[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int q = slot(4 * u);
        m4[u] = 0u;
        o4[u] = r4[u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        if (q < n) {
          m4[u] = a.mask ? *reinterpret_cast<const uint32_t*>(a.mask + row0 + q) : 0x01010101u;
          if (shaped) {
            o4[u] = *reinterpret_cast<const f32x4*>(a.old + row0 + q);
            r4[u] = *reinterpret_cast<const f32x4*>(a.ref + row0 + q);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if ((m4[u] >> (8 * c)) & 0xffu) mk |= 1u << (4 * u + c);
          ov[4 * u + c] = o4[u][c];
          rv[4 * u + c] = r4[u][c];
        }
    } else {
#pragma unroll
      for (int b = 0; b < kBits; ++b) {
        const int q = slot(b);
        ov[b] = rv[b] = 0.0f;
        if (q < n) {
          if (a.mask == nullptr || a.mask[row0 + q] != 0) mk |= 1u << b;
          if (shaped) {
            ov[b] = a.old[row0 + q];
            rv[b] = a.ref[row0 + q];
          }
        }
      }
    }
    if (end != T) __syncthreads();  // the previous tile's returns are consumed
    // token rewards to LDS (masked slots hold 0)
#pragma unroll
    for (int b = 0; b < kBits; ++b) {
      const int q = slot(b);
      if (q >= n) continue;
      double v = 0.0;
      if (shaped && ((mk >> b) & 1u)) v = -a.kl_coef * (double(ov[b]) - double(rv[b]));
      sh.v[adv_lds(q)] = v;
    }
    if (last < 0) {
      int qm = mk != 0 ? slot(31 - __builtin_clz(mk)) : -1;
      qm = wave_max_i32(qm);
      if (lane == 0) sh.wmax[wv] = qm;
    }
    __syncthreads();  // the tile's rewards and wmax are complete
    if (last < 0) {
      int m = -1;
      for (int w = 0; w < NW; ++w) m = sh.wmax[w] > m ? sh.wmax[w] : m;
      if (m >= 0) {
        last = start + m;
        // r_T = shaped + R at the last active slot, added by the thread whose
        // chunk holds it (nobody else touches that chunk before the next barrier)
        if (m / kAdvChunk == own) sh.v[adv_lds(m)] = sh.v[adv_lds(m)] + R;
      }
    }
    // this thread's chunk as a map
    const int q0 = own * kAdvChunk;
    const bool full = q0 + kAdvChunk <= n;
    const int q1 = full ? q0 + kAdvChunk : (q0 < n ? n : q0);
    double cv[kAdvChunk];
    double h = 0.0, g = 1.0;
    if (full) {
#pragma unroll
      for (int j = 0; j < kAdvChunk; ++j) cv[j] = sh.v[own * kAdvPad + j];
#pragma unroll
      for (int j = kAdvChunk - 1; j >= 0; --j) h = cv[j] + gam * h;
      g = g_full;
    } else {
      for (int q = q1 - 1; q >= q0; --q) {
        h = sh.v[adv_lds(q)] + gam * h;
        if constexpr (!kG1) g = g * gam;
      }
    }
    double ih = h, ig = g;
    wave_map_scan<kG1>(ih, ig);
    if (lane == kWave - 1) {
      sh.wh[wv] = ih;
      sh.wg[wv] = ig;
    }
    // the previous lane's inclusive map (lane 0: the identity) is the map
    // from the return after the wave to the return after this chunk
    const double eh = dpp_f64<0x138, 0xF>(ih, -0.0);  // wave_shr:1
    const double eg = kG1 ? 1.0 : dpp_f64<0x138, 0xF>(ig, 1.0);
    __syncthreads();
    // the return after this wave: the later waves' maps applied to the tile's carry
    double x = tile_carry;
    for (int w = NW - 1; w > wv; --w) x = sh.wh[w] + sh.wg[w] * x;
    double acc = eh + eg * x;  // return after this chunk
    double tc = tile_carry;
    for (int w = NW - 1; w >= 0; --w) tc = sh.wh[w] + sh.wg[w] * tc;
    tile_carry = tc;
    if (full) {
#pragma unroll
      for (int j = kAdvChunk - 1; j >= 0; --j) {
        acc = cv[j] + gam * acc;
        cv[j] = acc;
      }
#pragma unroll
      for (int j = 0; j < kAdvChunk; ++j) sh.v[own * kAdvPad + j] = cv[j];
    } else {
      for (int q = q1 - 1; q >= q0; --q) {
        acc = sh.v[adv_lds(q)] + gam * acc;
        sh.v[adv_lds(q)] = acc;
      }
    }
    __syncthreads();  // the tile's returns are in LDS
    if constexpr (kVec) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int q = slot(4 * u);
        if (q >= n) continue;
        const uint32_t bits = (mk >> (4 * u)) & 0xFu;
        const int r = adv_lds(q);  // the quad's four returns are consecutive in LDS
        const double v[4] = {sh.v[r], sh.v[r + 1], sh.v[r + 2], sh.v[r + 3]};
        if (a.normalize) {
          if (bits != 0u) {
            d2* dst = reinterpret_cast<d2*>(a.V + row0 + q);
            dst[0] = d2{v[0], v[1]};
            dst[1] = d2{v[2], v[3]};
          }
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if ((bits >> c) & 1u) ms.add(v[c]);
        } else {
          float o[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) o[c] = ((bits >> c) & 1u) ? float(clamp_adv(a, v[c])) : 0.0f;
          *reinterpret_cast<f32x4*>(a.out + row0 + q) = f32x4{o[0], o[1], o[2], o[3]};
        }
      }
    } else {
#pragma unroll 2
      for (int b = 0; b < kBits; ++b) {
        const int q = slot(b);
        if (q >= n) continue;
        const bool act = (mk >> b) & 1u;
        const double v = sh.v[adv_lds(q)];
        if (a.normalize) {
          if (act) {
            a.V[row0 + q] = v;
            ms.add(v);
          }
        } else {
          a.out[row0 + q] = act ? float(clamp_adv(a, v)) : 0.0f;
        }
      }
    }
  }
  if (a.normalize) {
    store_sequence_moments(a, i, ms, sh_mom);
  } else if (i == 0 && tid == 0 && a.status) {
    *a.status = 0u;
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

// Output-pass block sizes: REINFORCE++'s pass (which also reads the
// binary64 returns) is fastest in blocks of 1,024 threads, the baseline's in
// blocks of 256 (1,024 x 4,096 slots: 23.7 against 24.8 us, and 11.6 against
// 12.6 us, per call); every block merges the sequences' moments once.
constexpr int kNormThreadsReturns = 1024;
constexpr int kNormThreadsBaseline = 256;
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
template <bool kFused, int kNormThreads>
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
      // values are not used), so that the loads need no branch; plain loads:
      // the returns kernel has just written these lines and part of them is
      // still cached (non-temporal loads measured 1 us more per call at
      // 1024 x 4096)
#pragma unroll
      for (int u = 0; u < kNormQuads; ++u) {
        const int64_t src = m4[u] != 0 ? 4 * (q0 + int64_t(u) * kNormThreads) : 0;
        lo[u] = *reinterpret_cast<const f32x4*>(a.V + src);
        hi[u] = *reinterpret_cast<const f32x4*>(a.V + src + 2);
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
  if (a.estimator == GRPO_ADV_REINFORCE_PP) {
    auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & m) == 0; };
    const bool shaped = a.kl_coef != 0.0;
    const bool vec = a.T % 4 == 0 && al(a.mask, 3) && (!shaped || (al(a.old, 15) && al(a.ref, 15))) &&
                     (a.normalize ? al(a.V, 15) : al(a.out, 15));
    const bool g1 = a.gamma == 1.0;
    const dim3 grid(unsigned(a.B)), block(kAdvThreads);
    if (vec && g1) hipLaunchKernelGGL((grpo_tokadv_returns_kernel<true, true>), grid, block, 0, s, a);
    else if (vec) hipLaunchKernelGGL((grpo_tokadv_returns_kernel<true, false>), grid, block, 0, s, a);
    else if (g1) hipLaunchKernelGGL((grpo_tokadv_returns_kernel<false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((grpo_tokadv_returns_kernel<false, false>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL(grpo_tokadv_kernel, dim3(unsigned(a.B)), dim3(kAdvThreads), 0, s, a);
  }
  if (!a.normalize) return hipGetLastError();
  const bool fused = a.B <= kFusedMomentsMaxB;
  if (!fused) hipLaunchKernelGGL(grpo_tokadv_moments_kernel, dim3(1), dim3(kMomentThreads), 0, s, a);
  const int64_t rows = a.B * a.T;
  const int vec = (a.T % 4 == 0 && (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.out) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.V) & 15) == 0) ? 1 : 0;
  const int nt = a.estimator == GRPO_ADV_REINFORCE_PP ? kNormThreadsReturns : kNormThreadsBaseline;
  const int64_t per_block = vec ? int64_t(nt) * kNormQuads : int64_t(nt);
  const int64_t items = vec ? rows / 4 : rows;
  const int64_t blocks = (items + per_block - 1) / per_block;
  const dim3 grid{unsigned(blocks)}, block{unsigned(nt)};
  if (nt == kNormThreadsReturns) {
    if (fused) hipLaunchKernelGGL((grpo_tokadv_norm_kernel<true, kNormThreadsReturns>), grid, block, 0, s, a, vec);
    else hipLaunchKernelGGL((grpo_tokadv_norm_kernel<false, kNormThreadsReturns>), grid, block, 0, s, a, vec);
  } else {
    if (fused) hipLaunchKernelGGL((grpo_tokadv_norm_kernel<true, kNormThreadsBaseline>), grid, block, 0, s, a, vec);
    else hipLaunchKernelGGL((grpo_tokadv_norm_kernel<false, kNormThreadsBaseline>), grid, block, 0, s, a, vec);
  }
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
