/*
 * libgrpo -- the GRPO loss hot path for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a plain pointer plus sizes; no framework
 * types appear here.  Pointers are DEVICE pointers unless a comment says
 * HOST.  Every entry point is asynchronous on the given HIP stream (passed as
 * `void *stream`, a hipStream_t; NULL selects the default stream) and never
 * synchronises the host; results are valid once the stream reaches them.
 * The library never allocates or frees memory: the caller owns every buffer,
 * including the workspace sized by grpo_workspace_bytes().  (The one entry
 * point without a workspace argument, grpo_loss_fwd_bwd_noalloc, uses a
 * fixed array that the library's code object holds on each GPU.)
 *
 * What is computed follows these pages (cited by title and section):
 *   [GRPO-LOSS]  RL-Kernel docs, "GRPO Loss": Entry Point, Group
 *                specification, Tensor Contract, Normalizer semantics,
 *                Accuracy.
 *   [REAL-BLOG]  ms-swift blog on the REAL loss, background: the GRPO
 *                objective and its per-token gradient weight.
 *   [RPP]        Relax docs, "REINFORCE++ and REINFORCE++-baseline": Notation
 *                and mask contract, PPO and KL reduction.
 *   [GRPO-CPP]   grpo.cpp README: The length-normalization detail, CUDA.
 *   [DOCKYARD]   dockyard_rl, "GRPO and the clipped policy-gradient loss":
 *                Advantage estimation, One loss many algorithms, CISPO,
 *                Reference-KL penalty, Off-policy correction (async GRPO).
 *   [RPP-F]      Relax docs, "REINFORCE++ and REINFORCE++-baseline":
 *                Formula-level comparison (SAPO's soft gate, GSPO's sequence
 *                ratio).
 *   [REAL]       ms-swift blog on the REAL loss: REAL formalisation and the
 *                source walkthrough (in-group classification of sequences).
 *   [RPP-A]      Relax docs, "REINFORCE++ and REINFORCE++-baseline":
 *                REINFORCE++, REINFORCE++-baseline, Global masked
 *                normalization (token-level advantages).
 *   [GDPO]       dockyard_rl, "GRPO and the clipped policy-gradient loss":
 *                GDPO multi-reward advantage.
 *
 * Objective (per active token (i, t) of sequence i, action a = action_ids[i,t]),
 * in the default settings (GRPO_PG_CLIP, GRPO_KL_K3, no clamps):
 *   logp     = log softmax(policy_logits[i,t,:])[a]
 *   logp_ref = log softmax(ref_logits[i,t,:])[a]
 *   rho      = exp(logp - old_logps[i,t])
 *   d        = logp_ref - logp,   k3 = exp(d) - d - 1
 *   l        = -min(rho * A_i, clip(rho, 1 - eps_low, 1 + eps_high) * A_i)
 *   policy_loss = sum_i w_i * sum_t m_it * l_it,   kl = sum_i w_i * sum_t m_it * k3_it
 *   loss        = policy_loss + beta * kl
 * with A_i the group-relative advantage and w_i the per-sequence token weight
 * of the chosen reduction (see grpo_reduction).  The gradient is analytic:
 *   d loss / d logits[i,t,v] = G_it * (onehot(a)_v - softmax(policy_logits[i,t,:])_v)
 *   G_it = w_i * grad_scale * ( (clipped ? 0 : -A_i * rho) + beta * (1 - exp(d)) )
 * A token is clipped when rho lies strictly outside [1 - eps_low, 1 + eps_high]
 * on the side that the sign of A_i selects; at the exact bound the gradient
 * flows.  In general G_it = w_i * grad_scale * (dl/dlogp + beta * dkl/dlogp)
 * for the policy loss and KL estimator that grpo_cfg selects (grpo_pg_loss,
 * grpo_kl_estimator); "kl" then stands for the selected estimator.
 *
 * Masks: a nonzero byte marks an active slot ([GRPO-LOSS] Tensor Contract;
 * torch.bool and uint8 both work).  Selection is boolean ([RPP] Notation and
 * mask contract): values stored at masked slots never influence any result,
 * and masked logits rows are not read at all.
 *
 * Determinism: there are no floating-point atomics.  Every reduction runs in
 * a fixed order, so repeated calls with the same inputs and sizes give
 * bit-identical outputs.
 *
 * Workspace: grpo_workspace_bytes() bytes of device memory, 256-byte aligned.
 * Its contents need no initialisation: every call writes each workspace value
 * before it uses it (a 16-byte access may also fetch neighbouring slots the
 * call leaves unused, whose values are discarded).  A workspace serves one
 * call at a time: calls that share a workspace must be ordered on one stream.
 * grpo_loss_fwd_bwd() with grad_out == NULL leaves per-row state in the
 * workspace that grpo_loss_bwd() consumes; it stays valid until the next
 * call that uses the same workspace.
 *
 * Errors: every entry point validates its arguments on the host and returns a
 * grpo_status without launching anything when they are wrong.  Faults that
 * depend on device data are reported as bits in outputs->status (see
 * GRPO_FAULT_*), never by reading or writing out of bounds.
 */
#ifndef GRPO_H
#define GRPO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GRPO_ABI_VERSION 8

#ifndef GRPO_API
#define GRPO_API __attribute__((visibility("default")))
#endif

typedef enum grpo_status {
  GRPO_OK = 0,
  GRPO_ERR_NULL = 1,       /* a required pointer is NULL */
  GRPO_ERR_SHAPE = 2,      /* B, T or V not positive, a row stride < V, or sizes overflow
                              (the logits entry points take at most 2^31 - 1 rows B*T, the
                              token advantages at most 2^31 - 1 blocks of 256 slots) */
  GRPO_ERR_DTYPE = 3,      /* unknown dtype code */
  GRPO_ERR_GROUPS = 4,     /* group specification invalid ([GRPO-LOSS] Group specification) */
  GRPO_ERR_CONFIG = 5,     /* a grpo_cfg field invalid, or beta > 0 without a reference */
  GRPO_ERR_WORKSPACE = 6,  /* workspace NULL, misaligned or smaller than grpo_workspace_bytes() */
  GRPO_ERR_ALIAS = 7,      /* grad_out overlaps policy_logits without being exactly in place */
  GRPO_ERR_HIP = 8         /* a HIP runtime call or kernel launch failed */
} grpo_status;

/* Floating-point storage of logits and gradients.  Supported (logits ->
 * gradient) pairs: F32 -> F32 | BF16, BF16 -> BF16 | F32, F16 -> F16 | F32;
 * others return GRPO_ERR_DTYPE.  Arithmetic is float32 for every storage;
 * 16-bit gradients round to nearest even. */
typedef enum grpo_fdtype { GRPO_F32 = 0, GRPO_BF16 = 1, GRPO_F16 = 2 } grpo_fdtype;

/* Integer storage of action ids. */
typedef enum grpo_idtype { GRPO_I64 = 0, GRPO_I32 = 1 } grpo_idtype;

/* Per-sequence token weight w_i ([GRPO-LOSS] Normalizer semantics; [RPP] PPO
 * and KL reduction; [GRPO-CPP] The length-normalization detail).  L_i is the
 * number of active tokens of sequence i, N = sum_i L_i and B_live the number
 * of sequences with L_i > 0.
 *   GRPO_TOKEN_MEAN     w_i = 1 / max(N, 1)              (global token mean)
 *   GRPO_SEQUENCE_MEAN  w_i = 1 / (B * max(L_i, 1))      (mean in sequence, then over B)
 *   GRPO_LENGTH_ALPHA   w_i = L_i^alpha / (B * L_i), 0 when L_i = 0
 *   GRPO_FIXED_CONSTANT w_i = 1 / norm_constant          (a declared denominator)
 *   GRPO_SEQUENCE_MEAN_LIVE  w_i = 1 / (B_live * L_i), 0 when L_i = 0
 *                       (mean in sequence, then over the sequences with an
 *                       active token: [GRPO-LOSS] Normalizer semantics,
 *                       per_sequence_then_mean)
 * The weights are computed in binary64 and are bit-exact for alpha in
 * {0, 0.5, 1}; other alpha use pow() and may differ in the last bit. */
typedef enum grpo_reduction {
  GRPO_TOKEN_MEAN = 0,
  GRPO_SEQUENCE_MEAN = 1,
  GRPO_LENGTH_ALPHA = 2,
  GRPO_FIXED_CONSTANT = 3,
  GRPO_SEQUENCE_MEAN_LIVE = 4
} grpo_reduction;

/* Per-token policy loss l(logp) and its derivative, rho = exp(logp - old),
 * clip(.) = clip(., 1 - eps_low, 1 + eps_high) ([DOCKYARD] One loss many
 * algorithms, CISPO; [RPP-F] Formula-level comparison):
 *   GRPO_PG_CLIP       l = -min(rho A, clip(rho) A); with dual_clip_c = c > 1
 *                      and A < 0 the objective is bounded below by c A, and
 *                      below that bound the token has no surrogate gradient
 *   GRPO_PG_CISPO      l = -A sg(clip(rho)) logp: dl/dlogp = -A clip(rho)
 *                      (the clipped ratio is a constant weight)
 *   GRPO_PG_SAPO       l = -A f(rho), f(rho) = 4 sigmoid(tau (rho - 1)) / tau,
 *                      tau = sapo_tau_pos if A > 0 else sapo_tau_neg:
 *                      dl/dlogp = -4 A s (1 - s) rho with s the sigmoid
 *   GRPO_PG_REINFORCE  l = -A logp: dl/dlogp = -A
 *   GRPO_PG_ON_POLICY  ratio pinned to 1 by a stop-gradient: l = -A,
 *                      dl/dlogp = -A
 * Sequence-level forms ([RPP-F] GSPO row; [DOCKYARD] sequence-level
 * importance ratios; [REAL]) use s_i, the mean over sequence i's active
 * tokens of (logp - old_logps):
 *   GRPO_PG_GSPO       rho_i = exp(s_i) replaces the token ratio in the
 *                      clipped surrogate; l_i = -min(rho_i A, clip(rho_i) A)
 *                      is every active token's loss, so d loss / d logp_t =
 *                      w_i * (mean of the tokens' off-policy weights, 1
 *                      without them) * (clipped ? 0 : -A rho_i).  Not with
 *                      GRPO_TOKEN_MEAN (sequence ratios exclude token-level
 *                      reduction) nor the dual clip.
 *   GRPO_PG_REAL       in-group classification: in group g, sequences with
 *                      at least one active token are positive when A > 0 and
 *                      negative when A < 0; a group lacking either side adds
 *                      0; group loss log(1 + sum_pos exp(-s/tau)) +
 *                      log(1 + sum_neg exp(s/tau)) with tau = real_tau;
 *                      policy_loss = (sum of group losses) / (number of
 *                      groups); token t of sequence k gets d policy_loss /
 *                      d s_k / L_k.  Tokens carry no per-token policy loss
 *                      (their token loss and seq_policy read 0).  Needs
 *                      GRPO_TOKEN_MEAN (the KL term is the global token mean)
 *                      and no gen_logps.
 * The clip count (outputs->counts[1]) counts clipped tokens for CLIP (dual
 * clip included), tokens whose ratio lies outside the band for CISPO and the
 * active tokens of clipped sequences for GSPO. */
typedef enum grpo_pg_loss {
  GRPO_PG_CLIP = 0,
  GRPO_PG_CISPO = 1,
  GRPO_PG_SAPO = 2,
  GRPO_PG_REINFORCE = 3,
  GRPO_PG_ON_POLICY = 4,
  GRPO_PG_GSPO = 5,
  GRPO_PG_REAL = 6
} grpo_pg_loss;

/* Reference-KL estimator of d = logp_ref - logp ([DOCKYARD] Reference-KL
 * penalty), after the optional input clamp d -> clip(d, -kl_input_clamp,
 * kl_input_clamp) and followed by the optional output clamp of its value to
 * [-kl_output_clamp, kl_output_clamp].  A clamp passes the gradient at its
 * exact bound and cuts it strictly outside.
 *   GRPO_KL_K3  exp(d) - d - 1     dkl/dlogp = 1 - exp(d)
 *   GRPO_KL_K1  -d                 dkl/dlogp = 1
 *   GRPO_KL_K2  d^2 / 2            dkl/dlogp = -d */
typedef enum grpo_kl_estimator { GRPO_KL_K3 = 0, GRPO_KL_K1 = 1, GRPO_KL_K2 = 2 } grpo_kl_estimator;

/* Off-policy correction ([DOCKYARD] Off-policy correction (async GRPO)).
 * When the caller passes the generating policy's log-probs gen_logps, every
 * token's policy loss l and its gradient are multiplied by the importance
 * weight of the current policy (old_logps) to the generating one,
 *   omega = exp(old_logps - gen_logps),
 * a constant (it depends on no logit); the KL term is not weighted.
 *   GRPO_TIS_NONE      omega as is
 *   GRPO_TIS_TIS       clip(omega, tis_ratio_min, tis_ratio_max), min usually 0
 *   GRPO_TIS_ICEPOP    clip(omega, tis_ratio_min, tis_ratio_max), both bounds
 *                      chosen by the caller
 *   GRPO_TIS_SEQ_MASK  sequence masking: a sequence whose geometric-mean
 *                      weight exp(mean over its active tokens of (old_logps -
 *                      gen_logps)) lies outside [tis_ratio_min,
 *                      tis_ratio_max] has omega = 0 on every token; the other
 *                      sequences keep their untruncated omega.  Not with the
 *                      sequence-level policy losses.
 * Truncation needs gen_logps. */
typedef enum grpo_tis {
  GRPO_TIS_NONE = 0,
  GRPO_TIS_TIS = 1,
  GRPO_TIS_ICEPOP = 2,
  GRPO_TIS_SEQ_MASK = 3
} grpo_tis;

/* Device-detected data faults, OR-ed into outputs->status (which each call
 * overwrites). */
#define GRPO_FAULT_BAD_ACTION 1u  /* an active slot's action id is outside [0, V): that slot
                                     contributes no loss, no KL and a zero gradient row */
#define GRPO_FAULT_NO_TOKENS 2u   /* no active token at all (N = 0): loss = 0, gradient = 0 */
#define GRPO_FAULT_NONFINITE 4u   /* a non-finite per-token value at an active slot */

/* Reward groups ([GRPO-LOSS] Group specification; [DOCKYARD] Advantage
 * estimation).  Give exactly one of samples_per_prompt > 0 (uniform groups,
 * B must be a multiple) or group_boundaries (CSR offsets, HOST memory,
 * num_groups + 1 strictly increasing entries from 0 to B).  Every group needs
 * at least two members.  Advantages, per group g = [s, e) of n members, in
 * binary64 and index order:
 *   S = sum r, mean = S / n, var = sum (r - mean)^2 / n, std = sqrt(var)
 *   baseline b_i = mean, or (S - r_i) / (n - 1) with leave_one_out
 *   A_i = (r_i - b_i) / max(std, std_eps) if scale_by_std, else r_i - b_i
 * rounded once to float.  With leave_one_out the difference is divided by
 * the whole group's population std.  With clip_advantages the binary64 value
 * is clamped to [adv_clip_low, adv_clip_high] before the rounding ([DOCKYARD]
 * Advantage estimation). */
typedef struct grpo_groups {
  int32_t samples_per_prompt;       /* > 1, or 0 when group_boundaries is given */
  int32_t num_groups;               /* CSR: number of groups; ignored for uniform groups */
  const int64_t *group_boundaries;  /* HOST pointer or NULL; read during the call and
                                       passed to the device as kernel arguments (240
                                       offsets per launch of a small copy kernel), so
                                       every entry point enqueues kernel launches only
                                       and may be captured in a HIP graph; the array is
                                       not read after the call returns */
  int32_t leave_one_out;            /* 0 or 1 */
  int32_t scale_by_std;             /* 0 or 1 (the usual GRPO setting is 1) */
  double std_eps;                   /* floor of the std, > 0 (usually 1e-6) */
  int32_t clip_advantages;          /* 0 or 1 */
  double adv_clip_low;              /* finite, <= adv_clip_high; read when clip_advantages */
  double adv_clip_high;             /* finite; read when clip_advantages */
} grpo_groups;

/* Token-level advantage estimators ([RPP-A] below), for grpo_token_advantages().
 *   GRPO_ADV_REINFORCE_PP           r_t = m_t (-kl_coef * (old_logp_t - ref_logp_t)
 *                                   + [t = T_i] R_i), T_i the last active slot of
 *                                   sequence i; A_t = m_t sum_{u >= t} gamma^(u-t) r_u
 *                                   (the discount counts slot positions)
 *   GRPO_ADV_REINFORCE_PP_BASELINE  A_t = m_t (R_i - mean of R over i's group, i
 *                                   included; no std division) */
typedef enum grpo_adv_estimator {
  GRPO_ADV_REINFORCE_PP = 0,
  GRPO_ADV_REINFORCE_PP_BASELINE = 1
} grpo_adv_estimator;

/* Objective settings.  A symmetric clip sets eps_low == eps_high.  Zero in
 * pg_loss .. tis_ratio_max selects the clipped surrogate with the k3
 * estimator, no dual clip, no KL clamps and no truncation. */
typedef struct grpo_cfg {
  double eps_low;          /* in [0, 1) */
  double eps_high;         /* >= 0 */
  double beta;             /* reference-KL coefficient, >= 0 */
  int32_t reduction;       /* grpo_reduction */
  double alpha;            /* in [0, 1]; used by GRPO_LENGTH_ALPHA only */
  int32_t pg_loss;         /* grpo_pg_loss (0: the clipped surrogate) */
  int32_t kl_estimator;    /* grpo_kl_estimator (0: k3) */
  double dual_clip_c;      /* 0: off; else > 1, GRPO_PG_CLIP only */
  double sapo_tau_pos;     /* > 0, read by GRPO_PG_SAPO only */
  double sapo_tau_neg;     /* > 0, read by GRPO_PG_SAPO only */
  double kl_input_clamp;   /* 0: off; else > 0 and finite */
  double kl_output_clamp;  /* 0: off; else > 0 and finite */
  double norm_constant;    /* > 0 and finite, read by GRPO_FIXED_CONSTANT only */
  int32_t tis_type;        /* grpo_tis (0: no truncation) */
  double tis_ratio_min;    /* >= 0, <= tis_ratio_max; read when tis_type != 0 */
  double tis_ratio_max;    /* > 0 and finite; read when tis_type != 0 */
  double real_tau;         /* > 0 and finite, read by GRPO_PG_REAL only (usually 0.5) */
} grpo_cfg;

/* Outputs (DEVICE pointers).  Only `scalars` is required; any other field may
 * be NULL.  Per-sequence arrays have B entries; per-token arrays B * T
 * (row-major [B, T], 0 at masked slots). */
typedef struct grpo_outputs {
  float *scalars;      /* [3] loss, policy_loss, kl (float32) */
  float *advantages;   /* [B] A_i */
  float *seq_policy;   /* [B] sum over the sequence's active tokens of l */
  float *seq_kl;       /* [B] sum over the sequence's active tokens of the KL estimator */
  float *seq_weight;   /* [B] w_i */
  int32_t *seq_tokens; /* [B] L_i */
  int64_t *counts;     /* [2] N (active tokens), number of clipped active tokens */
  uint32_t *status;    /* [1] GRPO_FAULT_* bits of this call */
  float *tok_logp;     /* [B*T] logp of the taken token (logits entry points only) */
  float *tok_loss;     /* [B*T] token loss l */
  float *tok_kl;       /* [B*T] KL estimator */
  float *seq_logratio; /* [B] s_i, the mean log-ratio of sequence i (written by the
                          sequence-level policy losses only) */
} grpo_outputs;

/* ABI version of the loaded library (GRPO_ABI_VERSION it was built with). */
GRPO_API int grpo_abi_version(void);

/* Static text for a status code. */
GRPO_API const char *grpo_status_str(int status);

/* Workspace bytes needed for B sequences of T slots and, for CSR groups,
 * num_groups groups (pass 0 for uniform groups).  Returns 0 when the sizes
 * are not positive or overflow.  One workspace of this size serves every
 * entry point below for these sizes. */
GRPO_API size_t grpo_workspace_bytes(int64_t B, int64_t T, int32_t num_groups);

/* Zero-fills a workspace.  Optional (no result depends on a workspace value
 * the call did not write); useful to make a fresh workspace's contents
 * defined. */
GRPO_API grpo_status grpo_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* Group-relative advantages alone ([GRPO-LOSS] Accuracy; [DOCKYARD]
 * Advantage estimation).  rewards: [B] float32.  adv_out: [B] float32. */
GRPO_API grpo_status grpo_advantages(const float *rewards, int64_t B, const grpo_groups *groups,
                            float *adv_out, void *ws, size_t ws_bytes, void *stream);

/* Token-level advantages [B, T] ([RPP-A]), computed in binary64 and rounded
 * once to float32 (0 at masked slots).
 *   estimator: grpo_adv_estimator.  rewards: [B] float32 (R_i).
 *   old_logp, ref_logp: [B, T] float32 (GRPO_ADV_REINFORCE_PP only; ref_logp
 *     may be NULL when kl_coef == 0, old_logp may then be NULL too).
 *   mask: [B, T] bytes or NULL (all active).
 *   groups: the reward groups, required by GRPO_ADV_REINFORCE_PP_BASELINE
 *     (whose leave_one_out / scale_by_std must be 0: the baseline is the
 *     inclusive mean without std division); optional for GRPO_ADV_REINFORCE_PP.
 *     Its clamp, if set, is applied last.
 *   kl_coef >= 0 and finite; gamma in (0, 1].
 *   normalize: 1 applies the global masked normalization over every active
 *     slot of the batch: A <- (A - mu) / sqrt(max(var, 1e-8)), population
 *     moments (an empty mask gives zeros and GRPO_FAULT_NO_TOKENS).
 *   adv_out: [B, T] float32.  status: device uint32 for GRPO_FAULT_* bits, or NULL.
 * Errors as for the loss entry points (GRPO_ERR_CONFIG for a bad estimator,
 * kl_coef or gamma, or a missing input it needs). */
GRPO_API grpo_status grpo_token_advantages(int32_t estimator, const float *rewards,
                                           const float *old_logp, const float *ref_logp,
                                           const uint8_t *mask, int64_t B, int64_t T,
                                           const grpo_groups *groups, double kl_coef,
                                           double gamma, int32_t normalize, float *adv_out,
                                           uint32_t *status, void *ws, size_t ws_bytes,
                                           void *stream);

/* Multi-reward advantages [B] ([GDPO]).  rewards: [num_components, B]
 * float32 (component c of sample i at c * B + i), num_components >= 2.  For
 * each component the group baseline and std scaling follow `groups` exactly
 * as grpo_advantages does (GDPO uses leave_one_out = 1); the per-component
 * advantages are summed in binary64, the sum is renormalised over the batch
 * to zero mean and unit population std (floored at groups->std_eps), then
 * clamped if the groups ask for it, and rounded once to float32.
 * adv_out: [B] float32. */
GRPO_API grpo_status grpo_gdpo_advantages(const float *rewards, int32_t num_components, int64_t B,
                                          const grpo_groups *groups, float *adv_out, void *ws,
                                          size_t ws_bytes, void *stream);

/* Logprob-level token loss ([GRPO-CPP] CUDA: token loss from per-token
 * log-probs, returning dlogp).  logp, old_logp, ref_logp: [B, T] float32,
 * contiguous; ref_logp may be NULL only when beta == 0 (then d = 0).
 * gen_logp: [B, T] float32 log-probs of the generating policy, or NULL (no
 * off-policy correction; see grpo_tis).
 * mask: [B, T] bytes or NULL (all active).  rewards: [B] float32.
 * token_advantages: [B, T] float32 precomputed advantages (e.g. from
 *   grpo_token_advantages), or NULL.  When given, rewards and groups must be
 *   NULL, out->advantages is not written, and the sequence-level policy
 *   losses are rejected (they take one advantage per sequence).
 * dlogp_out: [B, T] float32, d loss / d logp (0 at masked slots), or NULL
 * for the forward only.  grad_scale: device float scalar multiplying every
 * gradient, or NULL for 1.  The per-token outputs tok_logp are not written
 * by this entry point. */
GRPO_API grpo_status grpo_token_loss(const float *logp, const float *old_logp, const float *ref_logp,
                            const float *gen_logp, const uint8_t *mask, const float *rewards,
                            const float *token_advantages, int64_t B, int64_t T,
                            const grpo_groups *groups, const grpo_cfg *cfg, float *dlogp_out,
                            const float *grad_scale, const grpo_outputs *out, void *ws,
                            size_t ws_bytes, void *stream);

/* Fused loss forward + analytic backward from vocabulary logits
 * ([GRPO-LOSS] Entry Point, Tensor Contract; [GRPO-CPP] CUDA, fused
 * logits boundary).
 *   policy_logits, ref_logits: [B, T, V] in logits_dtype, row (i, t) starting
 *     at element (i*T + t) * row_stride, row_stride >= V.  ref_logits may be
 *     NULL only when beta == 0.  ref_logits may equal policy_logits.
 *   action_ids: [B, T] in ids_dtype, contiguous.
 *   old_logps: [B, T] float32.  gen_logps: [B, T] float32 or NULL (the
 *     generating policy's log-probs for the off-policy correction; see
 *     grpo_tis).  mask: [B, T] bytes or NULL.  rewards: [B].
 *   token_advantages: [B, T] float32 or NULL, as for grpo_token_loss.
 *   grad_out: [B, T, V] in grad_dtype with row stride grad_row_stride >= V;
 *     masked rows are written with zeros.  grad_out may be policy_logits
 *     itself (in place; then grad_dtype, grad_row_stride must equal
 *     logits_dtype, row_stride).  grad_out == NULL runs the forward only and
 *     keeps per-row state in the workspace for grpo_loss_bwd().
 *   grad_scale: device float scalar (autograd's upstream gradient) or NULL
 *     for 1.
 * Vector (16-byte) loads are used when every row of every logits/grad tensor
 * is 16-byte aligned; other layouts take a slower scalar path. */
GRPO_API grpo_status grpo_loss_fwd_bwd(const void *policy_logits, const void *ref_logits,
                              int32_t logits_dtype, int64_t row_stride, const void *action_ids,
                              int32_t ids_dtype, const float *old_logps, const float *gen_logps,
                              const uint8_t *mask, const float *rewards,
                              const float *token_advantages, int64_t B, int64_t T,
                              int64_t V, const grpo_groups *groups, const grpo_cfg *cfg, void *grad_out,
                              int32_t grad_dtype, int64_t grad_row_stride,
                              const float *grad_scale, const grpo_outputs *out, void *ws,
                              size_t ws_bytes, void *stream);

/* Size of the library's own scratch array that grpo_loss_fwd_bwd_noalloc
 * uses as its workspace: 8 MiB on every GPU the library runs on, held until
 * the process ends.  It covers grpo_workspace_bytes(B, T, num_groups) up to
 * that size, about 280,000 token slots (B * T). */
#define GRPO_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* grpo_loss_fwd_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  It allocates nothing (no hipMalloc, no
 * allocating library routine); the workspace is the library's static scratch
 * array of GRPO_NOALLOC_SCRATCH_BYTES on the GPU that runs `stream` (the
 * current GPU for the null stream), whose device address is looked up once
 * per GPU on the first call there.  Every other argument, output and error is
 * as for grpo_loss_fwd_bwd; in addition it returns GRPO_ERR_WORKSPACE,
 * without launching anything, when grpo_workspace_bytes(B, T, num_groups)
 * exceeds GRPO_NOALLOC_SCRATCH_BYTES.  The scratch array keeps the last
 * call's contents; no result depends on them (every value is written before
 * it is read).  All calls on one GPU share that one array: calls that can
 * overlap on a GPU (other streams, other host threads) race and must be
 * ordered by the caller.  With grad_out == NULL it runs the forward only;
 * grpo_loss_bwd cannot follow it (that takes a caller's workspace). */
GRPO_API grpo_status grpo_loss_fwd_bwd_noalloc(const void *policy_logits, const void *ref_logits,
                                               int32_t logits_dtype, int64_t row_stride,
                                               const void *action_ids, int32_t ids_dtype,
                                               const float *old_logps, const float *gen_logps,
                                               const uint8_t *mask, const float *rewards,
                                               const float *token_advantages, int64_t B, int64_t T,
                                               int64_t V, const grpo_groups *groups,
                                               const grpo_cfg *cfg, void *grad_out,
                                               int32_t grad_dtype, int64_t grad_row_stride,
                                               const float *grad_scale, const grpo_outputs *out,
                                               void *stream);

/* Backward of a preceding grpo_loss_fwd_bwd(..., grad_out = NULL, ...) call on
 * the same workspace and the same policy_logits/action_ids/mask/sizes:
 * writes d loss / d policy_logits, multiplied by *grad_scale (device float,
 * NULL = 1) on top of any scale the forward applied. */
GRPO_API grpo_status grpo_loss_bwd(const void *policy_logits, int32_t logits_dtype, int64_t row_stride,
                          const void *action_ids, int32_t ids_dtype, const uint8_t *mask,
                          int64_t B, int64_t T, int64_t V, void *grad_out, int32_t grad_dtype,
                          int64_t grad_row_stride, const float *grad_scale, void *ws,
                          size_t ws_bytes, void *stream);

/* Multiplies rows x V gradient elements (row stride row_stride >= V
 * elements, storage grad_dtype) in place by the device float *scale, and
 * returns without touching them when *scale == 1.  For an autograd wrapper
 * whose forward call already wrote d loss / d policy_logits with an upstream
 * gradient of 1 ([GRPO-LOSS] Entry Point: the gradient lands in the logits
 * buffer): its backward scales by the true upstream gradient.  One rounding
 * per element (float32 product, then round to nearest even to the storage).
 * Errors: NULL pointers, unknown dtype, non-positive or overflowing sizes,
 * row_stride < V. */
GRPO_API grpo_status grpo_scale_grad(void *grad, int32_t grad_dtype, int64_t rows, int64_t V,
                                     int64_t row_stride, const float *scale, void *stream);

/* Optional timing hook for profiling tools: when both are non-NULL, the
 * logits entry points record `start` right before and `stop` right after
 * the launch of their vocabulary-streaming kernel, grpo_token_loss around
 * its token kernel and grpo_token_advantages around its kernels, on the
 * call's stream.
 * The events are hipEvent_t handles owned by the caller; pass NULLs to turn
 * the hook off.  Not thread-safe: set it from the thread that launches. */
GRPO_API void grpo_set_timing_events(void *start, void *stop);

#ifdef __cplusplus
}
#endif

#endif /* GRPO_H */
