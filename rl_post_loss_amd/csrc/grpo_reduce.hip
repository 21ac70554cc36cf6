// Fixed-order reductions and the logprob-level token loss.
//
// Two nested reductions with fixed extents, as "GRPO Loss" (RL-Kernel docs,
// Tensor and Data Parallel) lays them out: the token slots of one sequence
// reduce to a per-sequence total, then the B totals reduce to the scalar.
// Both stages run in a fixed tree in binary64 without atomics, so results
// are bit-identical from run to run.  The grpo.cpp README (CUDA section)
// measures per-token atomics against block reduction for the same loss; here
// no atomic is used for values at all: the per-sequence stage is one kernel
// (a block per sequence) and the scalar stage a second, single-block kernel,
// so no block ever waits on, or fences for, another.  (A single kernel whose
// last block forms the scalars needs a device-scope release fence per block;
// on gfx950 that writes back the XCD's L2 and cost more than the launch it
// saves.)

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_groupadv.hpp"
#include "grpo_internal.hpp"
#include "grpo_objective.hpp"

namespace grpo {

constexpr int kRedThreads = 256;
// Token kernel: threads per sequence block, and quads of 4 tokens each thread
// takes per round (kTokThreads * kTokQuads * 4 tokens per round).
#ifndef GRPO_TOK_THREADS
#define GRPO_TOK_THREADS 256
#endif
constexpr int kTokThreads = GRPO_TOK_THREADS;
#ifndef GRPO_TOK_QUADS
#define GRPO_TOK_QUADS (1024 / GRPO_TOK_THREADS > 0 ? 1024 / GRPO_TOK_THREADS : 1)
#endif
constexpr int kTokQuads = GRPO_TOK_QUADS;
// GRPO_TOK_PIPE: issue the next round's loads before the current round's
// arithmetic and stores (mask words two rounds ahead).  GRPO_TOK_SPEC: data
// loads that do not wait for the mask words (1: the first round, 2: every
// round); a masked quad's values are then read but never used.
#ifndef GRPO_XCD_TOK
#define GRPO_XCD_TOK 4  // token kernel: runs of 4 consecutive sequences per XCD (xcd_runs)
#endif
#ifndef GRPO_TOK_PIPE
#define GRPO_TOK_PIPE 0
#endif
#ifndef GRPO_TOK_SPEC
#define GRPO_TOK_SPEC 0
#endif

// Scalar stage (one block): policy_loss = sum_i w_i P_i, kl = sum_i w_i K_i in
// binary64, written as float32, plus the token and clip counts and the fault
// bits of the call.  For REAL the policy loss is instead the sum of the group
// losses over the number of groups (ms-swift REAL blog, source walkthrough).
constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(kFinalThreads) void grpo_final_kernel(FinalArgs a) {
#pragma clang fp contract(off)
  // every sum in the tree of block_sum_* (butterfly in each wave, then the
  // wave partials in wave order), all of them through one LDS exchange
  constexpr int NW = kFinalThreads / kWave;
  __shared__ double sh_pl[NW], sh_kl[NW], sh_gl[NW];
  __shared__ long long sh_ct[NW], sh_n[NW];
  __shared__ uint32_t sh_f[NW];
  const int tid = threadIdx.x, lane = tid % kWave, wv = tid / kWave;
  double pl = 0.0, kl = 0.0, gl = 0.0;
  long long ct = 0, n = 0;
  uint32_t f = 0;
#pragma unroll 1
  for (int64_t j = tid; j < a.B; j += kFinalThreads) {
    pl = pl + a.w[j] * a.P[j];
    kl = kl + a.w[j] * a.K[j];
    ct += a.C[j];
    if (a.L) n += a.L[j];
    if (a.fault) f |= a.fault[j];
  }
  if (a.gloss) {
#pragma unroll 1
    for (int64_t g = tid; g < a.num_groups; g += kFinalThreads) gl = gl + a.gloss[g];
  }
  pl = wave_sum_f64<kWave>(pl);
  kl = wave_sum_f64<kWave>(kl);
  gl = wave_sum_f64<kWave>(gl);
  ct = wave_sum_i64<kWave>(ct);
  n = wave_sum_i64<kWave>(n);
  f = wave_or_u32(f);
  if (lane == 0) {
    sh_pl[wv] = pl;
    sh_kl[wv] = kl;
    sh_gl[wv] = gl;
    sh_ct[wv] = ct;
    sh_n[wv] = n;
    sh_f[wv] = f;
  }
  __syncthreads();
  if (tid != 0) return;
  double tpl = 0.0, tkl = 0.0, tgl = 0.0;
  long long tct = 0, tn = 0;
  uint32_t tf = 0;
#pragma unroll 4
  for (int k = 0; k < NW; ++k) {
    tpl += sh_pl[k];
    tkl += sh_kl[k];
    tgl += sh_gl[k];
    tct += sh_ct[k];
    tn += sh_n[k];
    tf |= sh_f[k];
  }
  // REAL: the policy loss is the sum of the group losses over the number of
  // groups (ms-swift REAL blog, source walkthrough)
  if (a.gloss) tpl = tgl / double(a.num_groups);
  // with the token kernel's own weights, N and its fault bit are formed
  // here; without a prep kernel the call's faults are the per-sequence words
  uint32_t st = a.fault ? (tf & GRPO_FAULT_NONFINITE) : a.hdr->status;
  if (a.L) {
    a.hdr->num_tokens = tn;
    if (tn == 0) st |= GRPO_FAULT_NO_TOKENS;
    a.hdr->status = st;
  }
  const double loss = tpl + double(a.beta) * tkl;
  a.scalars[0] = float(loss);
  a.scalars[1] = float(tpl);
  a.scalars[2] = float(tkl);
  if (a.counts) {
    a.counts[0] = a.L ? tn : a.hdr->num_tokens;
    a.counts[1] = tct;
  }
  if (a.status) *a.status = st;
}

hipError_t launch_final(const FinalArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(grpo_final_kernel, dim3(1), dim3(kFinalThreads), 0, stream, a);
  return hipGetLastError();
}

// Stage 1 over the per-token values the row kernel left in the workspace.
__global__ __launch_bounds__(kRedThreads) void grpo_reduce_kernel(ReduceArgs a) {
#pragma clang fp contract(off)
  __shared__ double sh_f64[kRedThreads / kWave];
  __shared__ long long sh_i64[kRedThreads / kWave];
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = i * a.T;
  double p = 0.0, k = 0.0;
  long long c = 0;
  for (int64_t t = tid; t < a.T; t += kRedThreads) {
    p = p + double(a.tok_loss[base + t]);
    k = k + double(a.tok_kl[base + t]);
    c += a.flags[base + t] & 1;
  }
  p = block_sum_f64<kRedThreads>(p, sh_f64);
  k = block_sum_f64<kRedThreads>(k, sh_f64);
  c = block_sum_i64<kRedThreads>(c, sh_i64);
  if (tid == 0) {
    a.P[i] = p;
    a.K[i] = k;
    a.C[i] = c;
    if (a.seq_policy) a.seq_policy[i] = float(p);
    if (a.seq_kl) a.seq_kl[i] = float(k);
  }
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(grpo_reduce_kernel, dim3(unsigned(a.B)), dim3(kRedThreads), 0, stream, a);
  return hipGetLastError();
}

// Sequence-level losses: a token's policy loss from its sequence's (GSPO:
// omega_t * l_i, counted as clipped with its sequence; REAL: 0).
__device__ __forceinline__ void seq_token(const Objective& o, TokObj& r, bool gspo, double lseq,
                                          bool cseq, float old, float gen, bool has_gen) {
  if (gspo) {
    const float om = has_gen ? token_is_weight(o, old, gen) : 1.0f;
    r.loss = float(double(om) * lseq);
    r.clipped = cseq;
  }
}

// One block per sequence: tokens -> dlogp and the per-sequence totals.  The
// grpo.cpp README's token-loss kernels (CUDA section) compute the same loss
// from per-token log-probs.  kGeneral selects the objective code path (see
// token_objective).  kWeights: 0 takes w_i from the workspace; 1 forms it
// from the prep kernel's counts; 2 also counts the sequence's own mask and
// forms its group advantage (no prep kernel: reductions that do not need N).
template <bool kGeneral, int kWeights>
__global__ __launch_bounds__(kTokThreads) void grpo_token_kernel(TokenArgs a) {
#pragma clang fp contract(off)
  __shared__ double sh_f64[kTokThreads / kWave];
  __shared__ long long sh_i64[kTokThreads / kWave];
  __shared__ float sh_r[kWeights == 2 ? kRewardStage : 1];
  __shared__ float sh_adv;
  const int64_t i = xcd_runs(blockIdx.x, gridDim.x, GRPO_XCD_TOK);
  const int tid = threadIdx.x;
  const int64_t base = i * a.T;
  const bool vec = (a.T & 3) == 0 && ((reinterpret_cast<uintptr_t>(a.logp) |
                                       reinterpret_cast<uintptr_t>(a.old) |
                                       reinterpret_cast<uintptr_t>(a.ref) |
                                       reinterpret_cast<uintptr_t>(a.gen) |
                                       reinterpret_cast<uintptr_t>(a.adv_tok) |
                                       reinterpret_cast<uintptr_t>(a.dlogp) |
                                       reinterpret_cast<uintptr_t>(a.out_loss) |
                                       reinterpret_cast<uintptr_t>(a.out_kl)) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0;
  const bool has_ref = a.ref != nullptr;
  const bool has_gen = a.gen != nullptr;
  const bool has_atok = a.adv_tok != nullptr;
  // vector path: each thread takes QU quads of 4 tokens per round: their mask
  // words, then the log-prob loads of the active ones, then the arithmetic.
  // The first round's loads are issued before the prologue below (counts,
  // weights, advantage) waits on anything but the mask words.
  constexpr int QU = kTokQuads;
  constexpr bool kPipe = GRPO_TOK_PIPE != 0;
  const int64_t n4 = a.T / 4;
  const int64_t step = int64_t(QU) * kTokThreads;
  uint32_t m4[QU], mn[QU];
  f32x4 lp[QU], od[QU], rf[QU], gn[QU], av[QU];
  auto load_masks_to = [&](int64_t q0, uint32_t (&m)[QU]) {
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t q = q0 + int64_t(u) * kTokThreads;
      m[u] = q < n4 ? (a.mask ? *reinterpret_cast<const uint32_t*>(a.mask + base + 4 * q)
                              : 0x01010101u)
                    : 0u;
    }
  };
  auto load_masks = [&](int64_t q0) { load_masks_to(q0, m4); };
  // Branch-free: a quad with no active token (or past the row's end) reads the
  // row's first quad instead, an in-bounds line that every thread of the row
  // touches anyway, and its values are never used.  Without per-quad branches
  // the compiler can wait for each quad's own loads alone rather than for
  // every outstanding load and store.
  auto load_data = [&](int64_t q0, bool spec) {
#pragma unroll
    for (int u = 0; u < QU; ++u) {
      const int64_t q = q0 + int64_t(u) * kTokThreads;
      const int64_t t0 = base + ((spec ? q < n4 : m4[u] != 0) ? 4 * q : 0);
      lp[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.logp + t0));
      od[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.old + t0));
      rf[u] = gn[u] = av[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (has_ref) rf[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.ref + t0));
      if (has_gen) gn[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.gen + t0));
      if (has_atok) av[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.adv_tok + t0));
    }
  };
  // weights mode 2: the group's rewards are requested with the mask words
  // (one per thread when the group fits the block); the load is issued
  // unconditionally, from a valid address, so that nothing waits on it early
  int64_t g_s = 0, g_n = 0;
  float r_pre = 0.0f;
  if constexpr (kWeights == 2) {
    if (a.rewards) {
      int64_t g_e;
      group_bounds(a.grp, i, &g_s, &g_e);
      g_n = g_e - g_s;
    }
    const float* rsrc = a.rewards ? a.rewards : a.logp;
    r_pre = rsrc[g_s + (tid < g_n ? tid : 0)];
  }
  const bool staged = kWeights == 2 && a.rewards != nullptr && g_n <= kTokThreads;
  if (vec) {
    load_masks(tid);
    if (kPipe && tid + step < n4) load_masks_to(tid + step, mn);
  }
  // stage the rewards before any data load is issued, so that waiting for
  // them never waits for those loads
  if (staged && tid < g_n) sh_r[tid] = r_pre;
  if (vec) load_data(tid, GRPO_TOK_SPEC >= 1);
  float adv;
  long long Li = 0;
  double wi;
  if constexpr (kWeights == 2) {
    // L_i from this block's own mask words, and A_i: the count's wave
    // partials and the staged rewards share one barrier
    long long cnt = 0;
    if (vec) {
#pragma unroll
      for (int u = 0; u < QU; ++u) cnt += nonzero_bytes(m4[u]);
      for (int64_t q = tid + QU * kTokThreads; q < n4; q += kTokThreads)
        cnt += a.mask ? nonzero_bytes(*reinterpret_cast<const uint32_t*>(a.mask + base + 4 * q)) : 4;
    } else {
      for (int64_t t = tid; t < a.T; t += kTokThreads) cnt += (a.mask == nullptr || a.mask[base + t] != 0);
    }
    cnt = wave_sum_i64<kWave>(cnt);
    if (tid % kWave == 0) sh_i64[tid / kWave] = cnt;
    __syncthreads();
    for (int w = 0; w < kTokThreads / kWave; ++w) Li += sh_i64[w];
    if (staged) {
      if (tid == 0) sh_adv = group_advantage_staged(a.grp, sh_r, g_n, i - g_s);
    } else if (a.rewards) {
      const float v = group_advantage<kTokThreads>(a.grp, a.rewards, i, sh_r);
      if (tid == 0) sh_adv = v;
    }
    __syncthreads();
    adv = a.rewards ? sh_adv : 0.0f;
    wi = sequence_weight(a.reduction, a.alpha, a.norm_constant, a.B, Li, 0);
  } else if constexpr (kWeights == 1) {
    adv = a.A[i];
    // the token mean needs N = sum_j L_j, the live-sequence mean the number
    // of sequences with an active token (the prep kernel's counts, fixed tree)
    long long C = 0;
    if (a.reduction == GRPO_TOKEN_MEAN || a.reduction == GRPO_SEQUENCE_MEAN_LIVE) {
      long long n = 0;
      for (int64_t j = tid; j < a.B; j += kTokThreads) n += reduction_count(a.reduction, a.L[j]);
      C = block_sum_i64<kTokThreads>(n, sh_i64);
    }
    wi = sequence_weight(a.reduction, a.alpha, a.norm_constant, a.B, a.L[i], C);
  } else {
    adv = a.A[i];
    wi = a.w[i];
  }
  const float wg = float(wi) * (a.grad_scale ? *a.grad_scale : 1.0f);
  const float keep = a.iwseq ? float(a.iwseq[i]) : 1.0f;
  // sequence-level losses: the sequence kernels' loss, clip flag and
  // gradient coefficient (grad_scale included) of this sequence
  const bool seqlv = kGeneral && a.obj.seq;
  const bool gspo = seqlv && a.obj.pg == GRPO_PG_GSPO;
  const double lseq = gspo ? a.lseq[i] : 0.0;
  const bool cseq = gspo && a.cseq[i] != 0;
  const float useq = seqlv ? a.useq[i] : 0.0f;
  double p = 0.0, k = 0.0;
  long long c = 0;
  // A non-finite token loss or KL carries into p or k (float values cannot
  // overflow a binary64 sum), and a non-finite gradient value into gz, which
  // gains g * 0: 0 for every finite g, NaN otherwise.  One test after the
  // loop then flags exactly the sequences with a non-finite value.
  float gz = 0.0f;
  // the clip bounds as kernel constants in canonical form, so that the
  // per-token clamp needs no canonicalisation of them
  Objective obj = a.obj;
  obj.lo = __builtin_canonicalizef(obj.lo);
  obj.hi = __builtin_canonicalizef(obj.hi);
  if (vec) {
    int cn = 0;
    for (int64_t q0 = tid; q0 < n4; q0 += step) {
      if (!kPipe && q0 != tid) {
        load_masks(q0);
        load_data(q0, GRPO_TOK_SPEC >= 2);
      }
      // this round's values; with kPipe the next round's loads go out now
      uint32_t cm[QU];
      f32x4 clp[QU], cod[QU], crf[QU], cgn[QU], cav[QU];
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        cm[u] = m4[u];
        clp[u] = lp[u];
        cod[u] = od[u];
        crf[u] = rf[u];
        cgn[u] = gn[u];
        cav[u] = av[u];
      }
      if (kPipe && q0 + step < n4) {
#pragma unroll
        for (int u = 0; u < QU; ++u) m4[u] = mn[u];
        load_data(q0 + step, GRPO_TOK_SPEC >= 2);
        if (q0 + 2 * step < n4) load_masks_to(q0 + 2 * step, mn);
      }
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const int64_t q = q0 + int64_t(u) * kTokThreads;
        if (q >= n4) continue;
        const int64_t t0 = base + 4 * q;
        const float lpv[4] = {clp[u].x, clp[u].y, clp[u].z, clp[u].w};
        const float odv[4] = {cod[u].x, cod[u].y, cod[u].z, cod[u].w};
        const float rfv[4] = {crf[u].x, crf[u].y, crf[u].z, crf[u].w};
        const float gnv[4] = {cgn[u].x, cgn[u].y, cgn[u].z, cgn[u].w};
        const float avv[4] = {cav[u].x, cav[u].y, cav[u].z, cav[u].w};
        float gv[4] = {0.f, 0.f, 0.f, 0.f}, tl[4] = {0.f, 0.f, 0.f, 0.f}, tk[4] = {0.f, 0.f, 0.f, 0.f};
        // every token of the quad is evaluated and the mask selects the
        // results: straight-line code for all tokens of the round, so their
        // independent chains interleave (a masked token's inputs may be any
        // bits, its values are discarded by the selects)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool on = ((cm[u] >> (8 * j)) & 0xffu) != 0;
          const float d = has_ref ? rfv[j] - lpv[j] : 0.0f;
          TokObj r = token_objective<kGeneral>(obj, lpv[j], odv[j], d, has_atok ? avv[j] : adv,
                                               gnv[j], keep);
          if (seqlv) seq_token(obj, r, gspo, lseq, cseq, odv[j], gnv[j], has_gen);
          gv[j] = on ? (seqlv ? wg * r.g + useq : wg * r.g) : 0.0f;
          tl[j] = on ? r.loss : 0.0f;
          tk[j] = on ? r.kl : 0.0f;
          p = p + double(tl[j]);
          k = k + double(tk[j]);
          cn += (on & r.clipped) ? 1 : 0;
          gz = fmaf(gv[j], 0.0f, gz);
        }
        if (a.dlogp)
          __builtin_nontemporal_store(f32x4{gv[0], gv[1], gv[2], gv[3]},
                                      reinterpret_cast<f32x4*>(a.dlogp + t0));
        if (a.out_loss) *reinterpret_cast<f32x4*>(a.out_loss + t0) = f32x4{tl[0], tl[1], tl[2], tl[3]};
        if (a.out_kl) *reinterpret_cast<f32x4*>(a.out_kl + t0) = f32x4{tk[0], tk[1], tk[2], tk[3]};
      }
    }
    c += cn;
  } else {
    for (int64_t t = tid; t < a.T; t += kTokThreads) {
      const int64_t s = base + t;
      float g = 0.f, tl = 0.f, tk = 0.f;
      if (a.mask == nullptr || a.mask[s] != 0) {
        const float lps = a.logp[s];
        const float d = has_ref ? a.ref[s] - lps : 0.0f;
        const float ods = a.old[s], gns = has_gen ? a.gen[s] : 0.0f;
        TokObj r = token_objective<kGeneral>(obj, lps, ods, d, has_atok ? a.adv_tok[s] : adv, gns,
                                             keep);
        if (seqlv) seq_token(obj, r, gspo, lseq, cseq, ods, gns, has_gen);
        g = seqlv ? wg * r.g + useq : wg * r.g;
        tl = r.loss;
        tk = r.kl;
        p = p + double(r.loss);
        k = k + double(r.kl);
        c += r.clipped ? 1 : 0;
        gz = fmaf(g, 0.0f, gz);
      }
      if (a.dlogp) a.dlogp[s] = g;
      if (a.out_loss) a.out_loss[s] = tl;
      if (a.out_kl) a.out_kl[s] = tk;
    }
  }
  const bool nonfinite = !(isfinite(p) && isfinite(k) && isfinite(gz));
  if constexpr (kWeights != 2) {
    if (nonfinite) atomicOr(&a.hdr->status, GRPO_FAULT_NONFINITE);
  }
  // the sequence's totals: the tree of block_sum_* (butterfly in each wave,
  // then the wave partials in wave order), all four through one exchange
  constexpr int NW = kTokThreads / kWave;
  __shared__ double sh_pk[2][NW];
  __shared__ long long sh_c[NW];
  __shared__ int sh_bad[NW];
  p = wave_sum_f64<kWave>(p);
  k = wave_sum_f64<kWave>(k);
  c = wave_sum_i64<kWave>(c);
  const bool wbad = __ballot(nonfinite ? 1 : 0) != 0;
  const int lane = tid % kWave, wv = tid / kWave;
  __syncthreads();  // earlier readers of shared memory are done
  if (lane == 0) {
    sh_pk[0][wv] = p;
    sh_pk[1][wv] = k;
    sh_c[wv] = c;
    sh_bad[wv] = wbad ? 1 : 0;
  }
  __syncthreads();
  bool bad = false;
  if (tid == 0) {
    double tp = 0.0, tk = 0.0;
    long long tc = 0;
    int tb = 0;
    for (int w = 0; w < NW; ++w) {
      tp += sh_pk[0][w];
      tk += sh_pk[1][w];
      tc += sh_c[w];
      tb |= sh_bad[w];
    }
    p = tp;
    k = tk;
    c = tc;
    bad = tb != 0;
  }
  if (tid == 0) {
    a.P[i] = p;
    a.K[i] = k;
    a.C[i] = c;
    if (a.seq_policy) a.seq_policy[i] = float(p);
    if (a.seq_kl) a.seq_kl[i] = float(k);
    if constexpr (kWeights != 0) {
      a.w_out[i] = wi;
      if (a.seq_weight_out) a.seq_weight_out[i] = float(wi);
    }
    if constexpr (kWeights == 2) {
      // what the prep kernel would have written, and this sequence's faults
      a.L[i] = int32_t(Li);
      if (a.seq_tokens_out) a.seq_tokens_out[i] = int32_t(Li);
      if (a.rewards && a.adv_out) a.adv_out[i] = adv;
      a.fault[i] = bad ? GRPO_FAULT_NONFINITE : 0u;
    }
  }
}

hipError_t launch_token(const TokenArgs& a, hipStream_t stream) {
  const dim3 grid(unsigned(a.B)), block(kTokThreads);
#define GRPO_TOKEN_LAUNCH(W)                                                              \
  if (a.obj.general)                                                                      \
    hipLaunchKernelGGL((grpo_token_kernel<true, W>), grid, block, 0, stream, a);          \
  else                                                                                    \
    hipLaunchKernelGGL((grpo_token_kernel<false, W>), grid, block, 0, stream, a);
  if (a.weights_mode == 2) {
    GRPO_TOKEN_LAUNCH(2)
  } else if (a.weights_mode == 1) {
    GRPO_TOKEN_LAUNCH(1)
  } else {
    GRPO_TOKEN_LAUNCH(0)
  }
#undef GRPO_TOKEN_LAUNCH
  return hipGetLastError();
}

}  // namespace grpo
