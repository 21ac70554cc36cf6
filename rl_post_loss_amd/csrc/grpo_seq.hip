// Sequence phase of the sequence-level policy losses.
//
// GSPO (Relax REINFORCE++ page, Formula-level comparison: the sequence ratio
// exp of the masked mean of logp - old, expanded to the sequence's tokens and
// clipped as in PPO; dockyard_rl, One loss many algorithms: sequence-level
// importance ratios) and REAL (ms-swift REAL blog: REAL formalisation and the
// source walkthrough) both need every log-prob of a sequence before any of
// its tokens' gradients is known.  The row (or token) pass leaves the
// log-probs behind; these kernels then form, per sequence,
//   s_i = (sum over active tokens of (logp - old)) / max(L_i, 1)
// and the per-sequence gradient coefficient u_i that the gradient pass adds
// to each active token's KL part:
//   GSPO  u_i = w_i * mean_t(omega_t) * (clipped_i ? 0 : -A_i exp(s_i))
//   REAL  u_i = (d policy_loss / d s_i) / L_i
// with the call's grad_scale folded in.  Everything per sequence is binary64
// in fixed trees (no atomics), so results repeat bit for bit.

#include "../../include/grpo.h"
#include "grpo_device.hpp"
#include "grpo_internal.hpp"
#include "grpo_objective.hpp"

namespace grpo {

constexpr int kSeqThreads = 256;
constexpr int kRealThreads = 256;

__device__ __forceinline__ bool seq_token_active(const SeqArgs& a, int64_t r) {
  if (a.mask != nullptr && a.mask[r] == 0) return false;
  // a slot whose action id was out of range contributes nothing
  return a.stash == nullptr || a.stash[r].act != 0.0f;
}

// One block per sequence.
__global__ __launch_bounds__(kSeqThreads) void grpo_seq_kernel(SeqArgs a) {
#pragma clang fp contract(off)
  __shared__ double sh_f64[kSeqThreads / kWave];
  __shared__ long long sh_i64[kSeqThreads / kWave];
  const int64_t i = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = i * a.T;

  double acc = 0.0;
  for (int64_t t = tid; t < a.T; t += kSeqThreads) {
    const int64_t r = base + t;
    if (seq_token_active(a, r)) acc = acc + (double(a.logp[r]) - double(a.old[r]));
  }
  acc = block_sum_f64<kSeqThreads>(acc, sh_f64);
  const int32_t L = a.L[i];
  const double s = acc / double(L > 0 ? L : 1);
  const double gs = a.grad_scale ? double(*a.grad_scale) : 1.0;

  const bool gspo = a.pg == GRPO_PG_GSPO;
  double lseq = 0.0;
  bool clipped = false;
  if (gspo) {
    const double A = double(a.A[i]);
    const double rho = exp(s);
    clipped = (A > 0.0 && rho > a.hi) || (A < 0.0 && rho < a.lo);
    const double cr = rho < a.lo ? a.lo : (rho > a.hi ? a.hi : rho);
    const double unc = rho * A, clp = cr * A;
    lseq = -(unc < clp ? unc : clp);
    const double dl_ds = clipped ? 0.0 : -A * rho;
    const double wbar = a.iwseq ? a.iwseq[i] : 1.0;
    if (tid == 0) {
      a.useq[i] = float(a.w[i] * wbar * dl_ds * gs);
      a.lseq[i] = lseq;
      a.cseq[i] = clipped ? 1 : 0;
    }
  }
  if (tid == 0) {
    a.slogr[i] = s;
    if (a.seq_logratio) a.seq_logratio[i] = float(s);
  }
  if (!a.fill) return;

  // logits path: the token losses (GSPO: omega_t * l_i; REAL: 0), clip flags
  // and the per-sequence totals over the row pass's KL values
  double p = 0.0, k = 0.0;
  long long c = 0;
  for (int64_t t = tid; t < a.T; t += kSeqThreads) {
    const int64_t r = base + t;
    if (!seq_token_active(a, r)) continue;
    float tl = 0.0f;
    if (gspo) {
      const float om = a.gen ? token_is_weight(a.obj, a.old[r], a.gen[r]) : 1.0f;
      tl = float(double(om) * lseq);
      c += clipped ? 1 : 0;
    }
    a.tok_loss[r] = tl;
    a.flags[r] = clipped ? 1 : 0;
    if (a.out_loss) a.out_loss[r] = tl;
    p = p + double(tl);
    k = k + double(a.tok_kl[r]);
  }
  p = block_sum_f64<kSeqThreads>(p, sh_f64);
  k = block_sum_f64<kSeqThreads>(k, sh_f64);
  c = block_sum_i64<kSeqThreads>(c, sh_i64);
  if (tid == 0) {
    if (!(isfinite(p) && isfinite(lseq))) atomicOr(&a.hdr->status, GRPO_FAULT_NONFINITE);
    a.P[i] = p;
    a.K[i] = k;
    a.C[i] = c;
    if (a.seq_policy) a.seq_policy[i] = float(p);
    if (a.seq_kl) a.seq_kl[i] = float(k);
  }
}

hipError_t launch_seq(const SeqArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(grpo_seq_kernel, dim3(unsigned(a.B)), dim3(kSeqThreads), 0, stream, a);
  return hipGetLastError();
}

// REAL: one block; thread g handles group g (and g + kRealThreads, ...).  In a
// group, sequences with at least one active token are positive when A > 0
// and negative when A < 0.  With both sides present, the group loss is
//   log(1 + sum_pos exp(-s/tau)) + log(1 + sum_neg exp(s/tau)),
// each a log-sum-exp over the members' exponents and the appended 0, summed
// in member order after the largest exponent is taken out.
__global__ __launch_bounds__(kRealThreads) void grpo_real_kernel(RealArgs a) {
#pragma clang fp contract(off)
  const int64_t G = a.spp > 0 ? a.B / a.spp : int64_t(a.num_groups);
  const double gs = a.grad_scale ? double(*a.grad_scale) : 1.0;
  const double tau = a.tau;
  for (int64_t g = threadIdx.x; g < G; g += kRealThreads) {
    const int64_t s0 = a.spp > 0 ? g * a.spp : a.offsets[g];
    const int64_t e0 = a.spp > 0 ? s0 + a.spp : a.offsets[g + 1];
    double mp = 0.0, mn = 0.0;  // largest exponents, the appended 0 included
    int np = 0, nn = 0;
    for (int64_t k = s0; k < e0; ++k) {
      if (a.L[k] <= 0) continue;
      const double z = a.slogr[k] / tau;
      if (a.A[k] > 0.0f) {
        ++np;
        mp = -z > mp ? -z : mp;
      } else if (a.A[k] < 0.0f) {
        ++nn;
        mn = z > mn ? z : mn;
      }
    }
    const bool valid = np > 0 && nn > 0;
    double lp = 0.0, ln = 0.0;
    if (valid) {
      double sp = exp(-mp), sn = exp(-mn);
      for (int64_t k = s0; k < e0; ++k) {
        if (a.L[k] <= 0) continue;
        const double z = a.slogr[k] / tau;
        if (a.A[k] > 0.0f) sp = sp + exp(-z - mp);
        else if (a.A[k] < 0.0f) sn = sn + exp(z - mn);
      }
      lp = mp + log(sp);
      ln = mn + log(sn);
    }
    a.gloss[g] = valid ? lp + ln : 0.0;
    for (int64_t k = s0; k < e0; ++k) {
      double u = 0.0;
      const int32_t Lk = a.L[k];
      if (valid && Lk > 0) {
        const double z = a.slogr[k] / tau;
        if (a.A[k] > 0.0f) u = -(1.0 / tau) * exp(-z - lp) / double(G) / double(Lk);
        else if (a.A[k] < 0.0f) u = (1.0 / tau) * exp(z - ln) / double(G) / double(Lk);
      }
      a.useq[k] = float(u * gs);
    }
  }
}

hipError_t launch_real(const RealArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(grpo_real_kernel, dim3(1), dim3(kRealThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace grpo
