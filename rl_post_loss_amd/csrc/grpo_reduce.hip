// Fixed-order reductions and the logprob-level token loss.
//
// Two nested reductions with fixed extents, as "GRPO Loss" (RL-Kernel docs,
// Tensor and Data Parallel) lays them out: the token slots of one sequence
// reduce to a per-sequence total, then the B totals reduce to the scalar.
// Both stages run in a fixed tree in binary64 without atomics, so results
// are bit-identical from run to run.  The grpo.cpp README (CUDA section)
// measures per-token atomics against block reduction for the same loss; here
// no atomic is used at all: the per-sequence stage is one kernel (a block per
// sequence) and the scalar stage a second, single-block kernel, so no block
// ever waits on, or fences for, another.

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_internal.hpp"
#include "grpo_objective.hpp"

namespace grpo {

constexpr int kRedThreads = 256;

// Scalar stage (one block): policy_loss = sum_i w_i P_i, kl = sum_i w_i K_i in
// binary64, written as float32, plus the token and clip counts and the fault
// bits of the call.  For REAL the policy loss is instead the sum of the group
// losses over the number of groups (ms-swift REAL blog, source walkthrough).
constexpr int kFinalThreads = 1024;

__global__ __launch_bounds__(kFinalThreads) void grpo_final_kernel(FinalArgs a) {
#pragma clang fp contract(off)
  __shared__ double sh_f64[kFinalThreads / kWave];
  __shared__ long long sh_i64[kFinalThreads / kWave];
  const int tid = threadIdx.x;
  double pl = 0.0, kl = 0.0;
  long long ct = 0;
  for (int64_t j = tid; j < a.B; j += kFinalThreads) {
    pl = pl + a.w[j] * a.P[j];
    kl = kl + a.w[j] * a.K[j];
    ct += a.C[j];
  }
  pl = block_sum_f64<kFinalThreads>(pl, sh_f64);
  kl = block_sum_f64<kFinalThreads>(kl, sh_f64);
  ct = block_sum_i64<kFinalThreads>(ct, sh_i64);
  if (a.gloss) {
    double gl = 0.0;
    for (int64_t g = tid; g < a.num_groups; g += kFinalThreads) gl = gl + a.gloss[g];
    gl = block_sum_f64<kFinalThreads>(gl, sh_f64);
    pl = gl / double(a.num_groups);
  }
  if (tid == 0) {
    const double loss = pl + double(a.beta) * kl;
    a.scalars[0] = float(loss);
    a.scalars[1] = float(pl);
    a.scalars[2] = float(kl);
    if (a.counts) {
      a.counts[0] = a.hdr->num_tokens;
      a.counts[1] = ct;
    }
    if (a.status) *a.status = a.hdr->status;
  }
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
// token_objective).
template <bool kGeneral>
__global__ __launch_bounds__(kRedThreads) void grpo_token_kernel(TokenArgs a) {
#pragma clang fp contract(off)
  __shared__ double sh_f64[kRedThreads / kWave];
  __shared__ long long sh_i64[kRedThreads / kWave];
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = i * a.T;
  const float adv = a.A[i];
  const float wg = float(a.w[i]) * (a.grad_scale ? *a.grad_scale : 1.0f);
  const bool has_ref = a.ref != nullptr;
  const bool has_gen = a.gen != nullptr;
  const bool has_atok = a.adv_tok != nullptr;
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
  bool nonfinite = false;
  const bool vec = (a.T & 3) == 0 && ((reinterpret_cast<uintptr_t>(a.logp) |
                                       reinterpret_cast<uintptr_t>(a.old) |
                                       reinterpret_cast<uintptr_t>(a.ref) |
                                       reinterpret_cast<uintptr_t>(a.gen) |
                                       reinterpret_cast<uintptr_t>(a.adv_tok) |
                                       reinterpret_cast<uintptr_t>(a.dlogp) |
                                       reinterpret_cast<uintptr_t>(a.out_loss) |
                                       reinterpret_cast<uintptr_t>(a.out_kl)) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.mask) & 3) == 0;
  if (vec) {
    // each thread takes QU quads of 4 tokens per round: their mask words
    // first, then the log-prob loads of the active ones, then the arithmetic,
    // so a round costs two memory round trips
    constexpr int QU = 4;
    const int64_t n4 = a.T / 4;
    for (int64_t q0 = tid; q0 < n4; q0 += QU * kRedThreads) {
      uint32_t m4[QU];
      f32x4 lp[QU], od[QU], rf[QU], gn[QU], av[QU];
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const int64_t q = q0 + int64_t(u) * kRedThreads;
        m4[u] = q < n4 ? (a.mask ? *reinterpret_cast<const uint32_t*>(a.mask + base + 4 * q)
                                 : 0x01010101u)
                       : 0u;
      }
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const int64_t t0 = base + 4 * (q0 + int64_t(u) * kRedThreads);
        lp[u] = od[u] = rf[u] = gn[u] = av[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (m4[u] != 0) {
          lp[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.logp + t0));
          od[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.old + t0));
          if (has_ref) rf[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.ref + t0));
          if (has_gen) gn[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.gen + t0));
          if (has_atok) av[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.adv_tok + t0));
        }
      }
#pragma unroll
      for (int u = 0; u < QU; ++u) {
        const int64_t q = q0 + int64_t(u) * kRedThreads;
        if (q >= n4) continue;
        const int64_t t0 = base + 4 * q;
        const float lpv[4] = {lp[u].x, lp[u].y, lp[u].z, lp[u].w};
        const float odv[4] = {od[u].x, od[u].y, od[u].z, od[u].w};
        const float rfv[4] = {rf[u].x, rf[u].y, rf[u].z, rf[u].w};
        const float gnv[4] = {gn[u].x, gn[u].y, gn[u].z, gn[u].w};
        const float avv[4] = {av[u].x, av[u].y, av[u].z, av[u].w};
        float gv[4] = {0.f, 0.f, 0.f, 0.f}, tl[4] = {0.f, 0.f, 0.f, 0.f}, tk[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if ((m4[u] >> (8 * j)) & 0xffu) {
            const float d = has_ref ? rfv[j] - lpv[j] : 0.0f;
            TokObj r = token_objective<kGeneral>(a.obj, lpv[j], odv[j], d, has_atok ? avv[j] : adv,
                                                 gnv[j], keep);
            if (seqlv) seq_token(a.obj, r, gspo, lseq, cseq, odv[j], gnv[j], has_gen);
            gv[j] = seqlv ? wg * r.g + useq : wg * r.g;
            tl[j] = r.loss;
            tk[j] = r.kl;
            p = p + double(r.loss);
            k = k + double(r.kl);
            c += r.clipped ? 1 : 0;
            nonfinite |= !(isfinite(r.loss) && isfinite(r.kl) && isfinite(gv[j]));
          }
        }
        if (a.dlogp)
          __builtin_nontemporal_store(f32x4{gv[0], gv[1], gv[2], gv[3]},
                                      reinterpret_cast<f32x4*>(a.dlogp + t0));
        if (a.out_loss) *reinterpret_cast<f32x4*>(a.out_loss + t0) = f32x4{tl[0], tl[1], tl[2], tl[3]};
        if (a.out_kl) *reinterpret_cast<f32x4*>(a.out_kl + t0) = f32x4{tk[0], tk[1], tk[2], tk[3]};
      }
    }
  } else {
    for (int64_t t = tid; t < a.T; t += kRedThreads) {
      const int64_t s = base + t;
      float g = 0.f, tl = 0.f, tk = 0.f;
      if (a.mask == nullptr || a.mask[s] != 0) {
        const float lps = a.logp[s];
        const float d = has_ref ? a.ref[s] - lps : 0.0f;
        const float ods = a.old[s], gns = has_gen ? a.gen[s] : 0.0f;
        TokObj r = token_objective<kGeneral>(a.obj, lps, ods, d, has_atok ? a.adv_tok[s] : adv, gns,
                                             keep);
        if (seqlv) seq_token(a.obj, r, gspo, lseq, cseq, ods, gns, has_gen);
        g = seqlv ? wg * r.g + useq : wg * r.g;
        tl = r.loss;
        tk = r.kl;
        p = p + double(r.loss);
        k = k + double(r.kl);
        c += r.clipped ? 1 : 0;
        nonfinite |= !(isfinite(r.loss) && isfinite(r.kl) && isfinite(g));
      }
      if (a.dlogp) a.dlogp[s] = g;
      if (a.out_loss) a.out_loss[s] = tl;
      if (a.out_kl) a.out_kl[s] = tk;
    }
  }
  if (nonfinite) atomicOr(&a.hdr->status, GRPO_FAULT_NONFINITE);
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

hipError_t launch_token(const TokenArgs& a, hipStream_t stream) {
  if (a.obj.general)
    hipLaunchKernelGGL(grpo_token_kernel<true>, dim3(unsigned(a.B)), dim3(kRedThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(grpo_token_kernel<false>, dim3(unsigned(a.B)), dim3(kRedThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace grpo
