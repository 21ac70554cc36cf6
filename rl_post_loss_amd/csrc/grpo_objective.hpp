// Per-token objective: policy loss, reference-KL estimator and the token's
// d loss / d logp, shared by the logits row kernels and the log-prob token
// kernel.
//
// Policy-loss forms follow the dockyard_rl design doc (One loss many
// algorithms: the clipped surrogate, its dual clip, REINFORCE and the
// on-policy form; CISPO) and the Relax REINFORCE++ page (Formula-level
// comparison: SAPO's soft sigmoid gate).  KL estimators follow dockyard_rl
// (Reference-KL penalty), the off-policy weight its Off-policy correction
// section.  Everything is float32, as the rest of the row epilogue.  The
// sequence-level losses (GSPO, REAL) need whole sequences: here they
// contribute only their KL part, and the sequence kernels add the rest.
#pragma once

#include <math.h>

#include "../../include/grpo.h"
#include "grpo_internal.hpp"

// 1: the per-token exponentials use the hardware base-2 exponential and the
// KL estimator a short series (exp_hw, k3_expm1 below); 0: the math
// library's expf and expm1f.
#ifndef GRPO_FAST_TOKEN_MATH
#define GRPO_FAST_TOKEN_MATH 1
#endif

namespace grpo {

// e^x as 2^(fl(x log2 e)) on the hardware exponential: about 2 ulp for
// |x| up to ~10 (the rounding of x log2 e adds |x| 2^-24 relative), exactly
// 1 at x = 0; results below 2^-126 flush to zero.
__device__ __forceinline__ float exp_hw(float x) {
#if GRPO_FAST_TOKEN_MATH
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
#else
  return expf(x);
#endif
}

// The k3 estimator e^d - 1 - d and e^d - 1 together.  For |d| < 1,
// k3 = d^2 (1/2! + d/3! + ... + d^9/11!): the first omitted term is below
// 2^-26 of k3, and nothing cancels, where e^d - 1 - d loses the leading
// digits for small d; e^d - 1 = d + k3.  Otherwise both come from the
// hardware exponential: k3 = e^d - 1 - d then magnifies its error at most
// e/(e - 2) ~ 3.8 times (at d = 1).  NaN and +-inf give what expm1f gives:
// k3(NaN) = NaN, k3(+inf) = NaN, k3(-inf) = +inf.
struct K3Pair {
  float k3, em1;
};
__device__ __forceinline__ K3Pair k3_expm1(float d) {
#pragma clang fp contract(off)
#if GRPO_FAST_TOKEN_MATH
  float p = 1.0f / 39916800.0f;
  p = fmaf(p, d, 1.0f / 3628800.0f);
  p = fmaf(p, d, 1.0f / 362880.0f);
  p = fmaf(p, d, 1.0f / 40320.0f);
  p = fmaf(p, d, 1.0f / 5040.0f);
  p = fmaf(p, d, 1.0f / 720.0f);
  p = fmaf(p, d, 1.0f / 120.0f);
  p = fmaf(p, d, 1.0f / 24.0f);
  p = fmaf(p, d, 1.0f / 6.0f);
  p = fmaf(p, d, 0.5f);
  const float ks = (d * d) * p;
  const float e = exp_hw(d) - 1.0f;
  const bool small = fabsf(d) < 1.0f;
  return K3Pair{small ? ks : e - d, small ? d + ks : e};
#else
  const float em = expm1f(d);
  return K3Pair{em - d, em};
#endif
}

struct TokObj {
  float loss;    // policy loss l
  float kl;      // KL estimator value
  float g;       // dl/dlogp + beta * dkl/dlogp, before the token weight
  bool clipped;  // counted in the clip statistic
};

// clip(x, -v, v) that keeps a NaN (fminf/fmaxf would replace it by a bound)
__device__ __forceinline__ float clamp_sym(float x, float v) {
  return x != x ? x : fminf(fmaxf(x, -v), v);
}

// Per-sequence token weight w_i of the reduction (binary64, contraction
// off): token mean 1/N ("GRPO Loss", Normalizer semantics), sequence mean
// 1/(B L_i) (Relax REINFORCE++ page, PPO and KL reduction), the mean over
// live sequences 1/(B_live L_i) ("GRPO Loss", Normalizer semantics,
// per_sequence_then_mean), length weighting L_i^alpha / (B L_i) (grpo.cpp
// README, The length-normalization detail), or a declared constant.  `cnt`
// is the batch count the reduction needs: N for the token mean, B_live for
// the live-sequence mean (reduction_count).  Shared by the weights kernel
// and the token kernel so both give the same bits.
__device__ inline double sequence_weight(int32_t reduction, double alpha, double norm_constant,
                                  int64_t B, int64_t L, int64_t cnt) {
#pragma clang fp contract(off)
  if (reduction == GRPO_TOKEN_MEAN) return 1.0 / double(cnt > 0 ? cnt : 1);
  if (reduction == GRPO_SEQUENCE_MEAN_LIVE)
    return L > 0 ? 1.0 / (double(cnt > 0 ? cnt : 1) * double(L)) : 0.0;
  if (reduction == GRPO_FIXED_CONSTANT) return 1.0 / norm_constant;
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

// A sequence's share of the batch count sequence_weight needs: its L_i for
// the token mean, 1 if it has an active token for the live-sequence mean.
__device__ __forceinline__ long long reduction_count(int32_t reduction, long long L) {
  return reduction == GRPO_SEQUENCE_MEAN_LIVE ? (L > 0 ? 1 : 0) : L;
}

// Off-policy weight of one token: exp(old - gen), truncated for tis/icepop.
__device__ __forceinline__ float token_is_weight(const Objective& o, float old, float gen) {
  float wi = exp_hw(old - gen);
  if (o.tis) wi = wi != wi ? wi : fminf(fmaxf(wi, o.tis_lo), o.tis_hi);
  return wi;
}

// kGeneral = false: the clipped surrogate with k3, no dual clip, no clamps.
// kGeneral = true: every form the Objective selects.  For the default
// settings both evaluate the same expressions in the same order.  `keep` is
// the sequence's seq-mask flag (read only with o.seq_mask).
template <bool kGeneral>
__device__ __forceinline__ TokObj token_objective(const Objective& o, float logp, float old,
                                                  float d, float adv, float gen,
                                                  float keep = 1.0f) {
#pragma clang fp contract(off)
  TokObj r;
  const float rho = exp_hw(logp - old);
  if constexpr (!kGeneral) {
    const K3Pair k = k3_expm1(d);
    r.kl = k.k3;
    // bitwise, not short-circuit: no branch per token
    r.clipped = ((adv > 0.0f) & (rho > o.hi)) | ((adv < 0.0f) & (rho < o.lo));
    const float unc = rho * adv;
    const float clp = fminf(fmaxf(rho, o.lo), o.hi) * adv;
    r.loss = -fminf(unc, clp);
    const float dloss = r.clipped ? 0.0f : -adv * rho;
    r.g = dloss + o.beta * -k.em1;
    return r;
  } else {
    float dloss;
    r.clipped = false;
    if (o.seq) {
      // GSPO / REAL: the policy part is formed per sequence
      r.loss = 0.0f;
      dloss = 0.0f;
    } else if (o.pg == GRPO_PG_CLIP) {
      r.clipped = (adv > 0.0f && rho > o.hi) || (adv < 0.0f && rho < o.lo);
      const float unc = rho * adv;
      const float clp = fminf(fmaxf(rho, o.lo), o.hi) * adv;
      float obj = fminf(unc, clp);
      dloss = r.clipped ? 0.0f : -adv * rho;
      // dual clip: for A < 0 the objective is bounded below by c A
      if (o.dual_c > 0.0f && adv < 0.0f && obj < o.dual_c * adv) {
        obj = o.dual_c * adv;
        dloss = 0.0f;
        r.clipped = true;
      }
      r.loss = -obj;
    } else if (o.pg == GRPO_PG_CISPO) {
      // the clipped ratio weights -A logp as a constant
      const float wgt = fminf(fmaxf(rho, o.lo), o.hi);
      r.clipped = rho < o.lo || rho > o.hi;
      dloss = -adv * wgt;
      r.loss = dloss * logp;
    } else if (o.pg == GRPO_PG_SAPO) {
      // f(rho) = 4 s / tau with s = sigmoid(tau (rho - 1)); f'(rho) = 4 s (1 - s).
      // s and 1 - s both come from e = exp(-|x|), so neither cancels.
      const float tau = adv > 0.0f ? o.tau_pos : o.tau_neg;
      const float x = tau * (rho - 1.0f);
      const float e = exp_hw(-fabsf(x));
      const float inv = 1.0f / (1.0f + e);
      const float s = x >= 0.0f ? inv : e * inv;
      const float sc = x >= 0.0f ? e * inv : inv;
      r.loss = -(4.0f * s / tau) * adv;
      dloss = -adv * 4.0f * s * sc * rho;
    } else if (o.pg == GRPO_PG_REINFORCE) {
      r.loss = -adv * logp;
      dloss = -adv;
    } else {  // GRPO_PG_ON_POLICY: rho = exp(logp - sg(logp)) = 1
      r.loss = -adv;
      dloss = -adv;
    }
    if (o.has_is && !o.seq) {
      // constant weight of the current to the generating policy; a masked
      // sequence (seq-mask) has weight 0 whatever the token's ratio
      float wi = token_is_weight(o, old, gen);
      if (o.seq_mask) wi = keep != 0.0f ? wi : 0.0f;
      r.loss = r.loss * wi;
      dloss = dloss * wi;
    }

    bool pass = true;
    float dc = d;
    if (o.kl_in > 0.0f) {
      pass = fabsf(d) <= o.kl_in;
      dc = clamp_sym(d, o.kl_in);
    }
    float val, dval;  // estimator and its derivative in d
    if (o.kl == GRPO_KL_K1) {
      val = -dc;
      dval = -1.0f;
    } else if (o.kl == GRPO_KL_K2) {
      val = 0.5f * dc * dc;
      dval = dc;
    } else {
      const K3Pair k = k3_expm1(dc);
      val = k.k3;
      dval = k.em1;
    }
    if (o.kl_out > 0.0f) {
      pass = pass && fabsf(val) <= o.kl_out;
      val = clamp_sym(val, o.kl_out);
    }
    r.kl = val;
    const float dkl = pass ? -dval : 0.0f;  // dd/dlogp = -1
    r.g = dloss + o.beta * dkl;
    return r;
  }
}

}  // namespace grpo
