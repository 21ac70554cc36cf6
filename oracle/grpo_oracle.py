"""Plain fp64 CPU oracle for the GRPO loss hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this module:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use it.  It shares no code, constants or helpers with the HIP
library under ``rl_post_loss_amd/``.

Everything is computed in float64 with numpy (or Python floats, which are the
same IEEE binary64), in the plain order the definitions give.  No blocking, no
online softmax, no fusion: a reader can check each function against the pages.

Sources, cited by page title and section:

* [GRPO-LOSS]  RL-Kernel documentation, "GRPO Loss" (sections: Group
  specification, Tensor Contract, Normalizer semantics, Accuracy).
* [REAL-BLOG]  ms-swift blog post on the REAL loss, background section on the
  GRPO objective and its per-token gradient weight (clip indicator times
  A * e^s).
* [RPP]        Relax documentation, "REINFORCE++ and REINFORCE++-baseline"
  (sections: Notation and mask contract, PPO and KL reduction, Formula-level
  comparison).
* [GRPO-CPP]   grpo.cpp README (sections: The length-normalization detail,
  CUDA).
* [DOCKYARD]   dockyard_rl design doc, "GRPO and the clipped policy-gradient
  loss" (sections: Advantage estimation, One loss many algorithms, CISPO,
  Reference-KL penalty, Off-policy correction (async GRPO)).

Readings taken where the pages are silent or ambiguous (each is listed in the
repository design notes as well):

* KL estimator: k3 = exp(d) - d - 1 with d = logp_ref - logp_theta; its
  gradient with respect to logp_theta is the pathwise derivative 1 - exp(d)
  (autograd of the loss as written), not a score-function variant.
* Group std: population std (ddof = 0), floored at ``std_eps`` (default 1e-6).
* Leave-one-out with std scaling divides the leave-one-out difference by the
  whole group's population std.
* Sequence-mean denominator: all B sequences, each sequence's own count
  clamped to >= 1.
* Length-alpha weighting: per-token weight L_i**(alpha - 1) / B, i.e. a total
  weight of L_i**alpha / B for response i; 0 when L_i = 0.
* Token-mean with no active token: weight 1 / max(N, 1); every term is then 0.
* Clipping: a token is clipped only when rho lies strictly outside the band on
  the side selected by the sign of A; at the exact bound the gradient still
  flows (inclusive clamp, tie split of the minimum sums to the full gradient).
* Masked slots are never read (boolean selection), so NaN/Inf or garbage ids
  stored there cannot reach any output.
* Dual clip: for A < 0 the clipped objective is bounded below by c * A
  (c > 1); below that bound the token carries no surrogate gradient.
* CISPO: the clipped ratio multiplies -A logp as a constant (stop-gradient),
  so the gradient is -A clip(rho) for every token, clipped or not.
* SAPO: tau is chosen by the sign of A (tau_pos for A > 0, tau_neg
  otherwise); f_tau(rho) = 4 sigmoid(tau (rho - 1)) / tau, so at rho = 1 the
  gradient equals the unclipped surrogate's.
* On-policy: the ratio is exp(logp - sg(logp)) = 1, so the value is -A and the
  gradient -A (the clip band is inactive at rho = 1).
* KL clamps clamp d = logp_ref - logp to [-v_in, v_in] before the estimator
  and the estimator's value to [-v_out, v_out] after it; as with torch's
  clamp, the gradient passes at an exact bound and is zero strictly outside.
* Fixed-constant normaliser: every active token weighs 1 / C for a declared
  C > 0, independent of the mask.
* Off-policy correction: the importance weight is the ratio of the current
  policy (the old log-probs, which the trainer computes with its weights
  before the update) to the generating policy, exp(old - gen).  It is a
  constant (it depends on no trained parameter), multiplies the policy loss
  and its gradient, and leaves the KL term alone.  tis and icepop both clamp
  it to [min, max]; tis defaults min to 0, icepop requires it.
* Sequence-masked truncation (seq-mask-tis): a sequence's importance ratio
  is the geometric mean of its tokens' weights, exp(mean over active tokens
  of (old - gen)); when it lies outside [min, max] (inclusive bounds) the
  whole sequence's policy term is masked (weight 0), otherwise every token
  keeps its own untruncated weight.
* GSPO: the sequence ratio rho_i = exp(s_i), s_i the mean over active tokens
  of (logp - old), replaces the token ratio in the clipped surrogate; the
  sequence's value l_i is broadcast to its active tokens, which the chosen
  per-sequence weights then reduce (the global token mean is rejected:
  sequence-level ratios exclude token-level reduction).  Its gradient is the
  chain rule through s_i: every active token of sequence i gets
  w_i * (sum_t omega_t / L_i) * dl_i/ds_i, with omega_t the off-policy
  weights (1 without them).
* REAL: the classification logit of sequence k is s_k (as for GSPO).  In a
  group, sequences with at least one active token are positive when A_k > 0
  and negative when A_k < 0; a group lacking either side contributes 0.  The
  group loss is log(1 + sum_pos exp(-s/tau)) + log(1 + sum_neg exp(s/tau)),
  the policy loss is the sum of group losses divided by the number of groups
  in the batch, and the KL term is the global token mean (so REAL requires the
  token_mean reduction).  Tokens carry no per-token policy loss (their token
  loss reads 0); the gradient reaches token t of sequence k as
  (d policy_loss / d s_k) / L_k.

Parity pins: every function here is pinned by CPU tests in
``tests/test_oracle_pins.py`` and ``tests/test_oracle_variants.py`` (closed
forms, library routines, finite differences, an independent autograd
formulation, invariants).  The absolute
loss values of the synthetic workloads are not printed by the pages, so those
are pinned only through the checks above.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

REDUCTIONS = ("token_mean", "sequence_mean", "length_alpha", "fixed_constant",
              "per_sequence_then_mean")


class OracleInputError(ValueError):
    """Raised for inputs that violate the operation's contract."""


# ---------------------------------------------------------------------------
# Group specification  ([GRPO-LOSS] Group specification)
# ---------------------------------------------------------------------------

def group_offsets(B, samples_per_prompt=None, group_boundaries=None):
    """CSR offsets (length G+1) describing the reward groups.

    [GRPO-LOSS] Group specification: exactly one of a uniform
    ``samples_per_prompt`` or CSR ``group_boundaries`` (offsets of length
    num_groups + 1) is given.  Uniform groups need B to be a multiple of the
    group size.  Groups must tile [0, B) in order, and a group needs at least
    two members (a population std over one sample is rejected on the pages).
    """
    if (samples_per_prompt is None) == (group_boundaries is None):
        raise OracleInputError("give exactly one of samples_per_prompt / group_boundaries")
    if samples_per_prompt is not None:
        n = int(samples_per_prompt)
        if n < 2 or B % n != 0:
            raise OracleInputError("samples_per_prompt must be >= 2 and divide B")
        return np.arange(0, B + 1, n, dtype=np.int64)
    off = np.asarray(group_boundaries, dtype=np.int64)
    if off.ndim != 1 or off.size < 2 or off[0] != 0 or off[-1] != B:
        raise OracleInputError("group_boundaries must start at 0 and end at B")
    if np.any(np.diff(off) < 2):
        raise OracleInputError("every group needs at least two members")
    return off


# ---------------------------------------------------------------------------
# Group-relative advantages  ([GRPO-LOSS] Accuracy; [DOCKYARD] Advantage
# estimation)
# ---------------------------------------------------------------------------

def group_advantages(rewards, offsets, leave_one_out=False, scale_by_std=True,
                     std_eps=1e-6):
    """Per-sequence advantage A_i, float64.

    For a group g = [s, e) of n members, in index order:
      S = sum of r (sequential), mean = S / n,
      var = (sum of (r - mean)^2, sequential) / n, std = sqrt(var).
    Baseline b_i = mean, or with leave-one-out b_i = (S - r_i) / (n - 1).
    A_i = (r_i - b_i) / max(std, std_eps) when scaling by std, else r_i - b_i.
    """
    r = [float(v) for v in np.asarray(rewards, dtype=np.float64).ravel()]
    A = np.zeros(len(r), dtype=np.float64)
    for g in range(len(offsets) - 1):
        s, e = int(offsets[g]), int(offsets[g + 1])
        n = e - s
        total = 0.0
        for j in range(s, e):
            total = total + r[j]
        mean = total / n
        sq = 0.0
        for j in range(s, e):
            dev = r[j] - mean
            sq = sq + dev * dev
        std = math.sqrt(sq / n)
        denom = max(std, std_eps)
        for j in range(s, e):
            base = (total - r[j]) / (n - 1) if leave_one_out else mean
            diff = r[j] - base
            A[j] = diff / denom if scale_by_std else diff
    return A


def _advantages_of(rewards, B, groups):
    """(A [B], CSR offsets) from rewards and a group specification, with the
    optional clamp of [DOCKYARD] Advantage estimation (groups keys
    adv_clip_low / adv_clip_high)."""
    off = group_offsets(B, groups.get("samples_per_prompt"), groups.get("group_boundaries"))
    A = group_advantages(rewards, off, groups.get("leave_one_out", False),
                         groups.get("scale_by_std", True), groups.get("std_eps", 1e-6))
    if groups.get("adv_clip_low") is not None:
        lo, hi = float(groups["adv_clip_low"]), float(groups["adv_clip_high"])
        if not lo <= hi:
            raise OracleInputError("advantage clamp needs low <= high")
        A = np.clip(A, lo, hi)
    return A, off


def _advantage_source(rewards, groups, advantages, B, T, cfg):
    """Advantages of every slot: from rewards and groups ([B], broadcast) or
    given per token ([B, T]).  Returns (A [B] or None, offsets or None,
    A per slot [B, T])."""
    if advantages is None:
        A, off = _advantages_of(rewards, B, groups)
        return A, off, np.broadcast_to(A[:, None], (B, T))
    if rewards is not None:
        raise OracleInputError("give rewards or token advantages, not both")
    if cfg.pg_loss in SEQUENCE_PG:
        raise OracleInputError("sequence-level losses take per-sequence advantages")
    At = np.asarray(advantages, dtype=np.float64)
    if At.shape != (B, T):
        raise OracleInputError("token advantages must be [B, T]")
    return None, None, At


# ---------------------------------------------------------------------------
# Token counts and per-sequence weights  ([GRPO-LOSS] Normalizer semantics;
# [RPP] PPO and KL reduction; [GRPO-CPP] The length-normalization detail)
# ---------------------------------------------------------------------------

def sequence_weights(mask, reduction="token_mean", alpha=None, norm_constant=None):
    """Return (L [B] int64, N int, omega [B] float64).

    omega_i is the weight every active token of sequence i carries in the
    scalar loss:
      token_mean     1 / max(N, 1)                 (global active-token mean)
      sequence_mean  1 / (B * max(L_i, 1))          (mean within, then over B)
      length_alpha   L_i**alpha / (B * L_i), 0 if L_i = 0
      fixed_constant 1 / norm_constant            (a declared denominator)
      per_sequence_then_mean
                     1 / (B_live * L_i), 0 if L_i = 0, with B_live the
                     number of sequences that have an active token (the
                     mean within each sequence, then over the live ones:
                     [GRPO-LOSS] Normalizer semantics)
    """
    m = np.asarray(mask).astype(bool)
    if m.ndim != 2:
        raise OracleInputError("mask must be [B, T]")
    B = m.shape[0]
    L = m.sum(axis=1).astype(np.int64)
    N = int(L.sum())
    if reduction == "token_mean":
        w = np.full(B, 1.0 / max(N, 1), dtype=np.float64)
    elif reduction == "sequence_mean":
        w = 1.0 / (float(B) * np.maximum(L, 1).astype(np.float64))
    elif reduction == "length_alpha":
        if alpha is None or not (0.0 <= alpha <= 1.0):
            raise OracleInputError("length_alpha needs alpha in [0, 1]")
        Lf = L.astype(np.float64)
        if alpha == 0.0:
            num = np.ones(B, dtype=np.float64)
        elif alpha == 0.5:
            num = np.sqrt(Lf)
        elif alpha == 1.0:
            num = Lf
        else:
            num = np.power(Lf, float(alpha))
        w = np.where(L > 0, num / (float(B) * np.maximum(Lf, 1.0)), 0.0)
    elif reduction == "fixed_constant":
        if norm_constant is None or not norm_constant > 0:
            raise OracleInputError("fixed_constant needs norm_constant > 0")
        w = np.full(B, 1.0 / float(norm_constant), dtype=np.float64)
    elif reduction == "per_sequence_then_mean":
        live = L > 0
        n_live = int(live.sum())
        w = np.zeros(B, dtype=np.float64)
        w[live] = 1.0 / (float(n_live) * L[live].astype(np.float64))
    else:
        raise OracleInputError(f"unknown reduction {reduction!r}")
    return L, N, w


# ---------------------------------------------------------------------------
# Per-token objective  ([GRPO-LOSS] Accuracy; [REAL-BLOG] background;
# [DOCKYARD] One loss many algorithms, Reference-KL penalty)
# ---------------------------------------------------------------------------

PG_LOSSES = ("clip", "cispo", "sapo", "reinforce", "on_policy", "gspo", "real")
SEQUENCE_PG = ("gspo", "real")
KL_ESTIMATORS = ("k3", "k1", "k2")


@dataclass
class LossConfig:
    """Objective settings.  A symmetric clip sets eps_low = eps_high.

    pg_loss ([DOCKYARD] One loss many algorithms, CISPO; [RPP] Formula-level
    comparison for SAPO):
      clip       -min(rho A, clip(rho) A), optionally dual-clipped for A < 0
      cispo      -A sg(clip(rho)) logp       (the clipped ratio is a constant weight)
      sapo       -f_tau(rho) A, f_tau(rho) = 4 sigmoid(tau (rho - 1)) / tau,
                 tau = sapo_tau_pos for A > 0, sapo_tau_neg otherwise
      reinforce  -A logp                     (the ratio dropped)
      on_policy  the clip loss with the ratio pinned to 1 by a stop-gradient:
                 value -A, gradient -A
      gspo       the clip loss on the sequence ratio exp(mean_t(logp - old))
                 ([RPP] Formula-level comparison, GSPO row; [DOCKYARD] One
                 loss many algorithms, sequence-level importance ratios)
      real       in-group classification of sequences by the sign of A
                 ([REAL-BLOG] REAL formalisation and source walkthrough),
                 temperature real_tau
    kl_estimator ([DOCKYARD] Reference-KL penalty), with d = logp_ref - logp:
      k3 = e^d - d - 1,  k1 = -d = logp - logp_ref,  k2 = d^2 / 2
    kl_input_clamp / kl_output_clamp clamp d and the estimator to [-v, v].
    reduction "fixed_constant" weights every token by 1 / norm_constant
    ([GRPO-LOSS] Normalizer semantics).
    tis_type (None | "tis" | "icepop") truncates the off-policy importance
    weight to [tis_ratio_min, tis_ratio_max]; "seq_mask" instead masks the
    sequences whose geometric-mean weight leaves that range ([DOCKYARD]
    Off-policy correction (async GRPO)); each needs the generating policy's
    log-probs.
    """
    eps_low: float = 0.2
    eps_high: float = 0.2
    beta: float = 0.04
    reduction: str = "token_mean"
    alpha: float | None = None
    pg_loss: str = "clip"
    kl_estimator: str = "k3"
    dual_clip_c: float | None = None
    sapo_tau_pos: float = 1.0
    sapo_tau_neg: float = 1.0
    kl_input_clamp: float | None = None
    kl_output_clamp: float | None = None
    norm_constant: float | None = None
    tis_type: str | None = None
    tis_ratio_min: float | None = None
    tis_ratio_max: float | None = None
    real_tau: float = 0.5


TIS_TYPES = ("tis", "icepop", "seq_mask")


def is_weights(old_logp, gen_logp, cfg: LossConfig, keep=None):
    """Off-policy importance weight per token ([DOCKYARD] Off-policy
    correction (async GRPO)): exp(old - gen), truncated to [min, max] by tis
    (min defaults to 0) or icepop (both bounds given).  For seq_mask the
    weight stays untruncated and ``keep`` (per token: whether its sequence
    passed sequence_mask_keep) multiplies it.  A constant: no gradient flows
    through it."""
    wt = np.exp(np.asarray(old_logp, dtype=np.float64) - np.asarray(gen_logp, dtype=np.float64))
    if cfg.tis_type in ("tis", "icepop"):
        lo = 0.0 if cfg.tis_ratio_min is None else float(cfg.tis_ratio_min)
        wt = np.clip(wt, lo, float(cfg.tis_ratio_max))
    elif cfg.tis_type == "seq_mask":
        if keep is None:
            raise OracleInputError("seq_mask needs each token's sequence keep flag")
        wt = np.where(np.asarray(keep, dtype=bool), wt, 0.0)
    return wt


def _seq_bounds(B, ii):
    """Start/end of each sequence's run in the sorted active-token index ii."""
    return np.searchsorted(ii, np.arange(B + 1))


def sequence_mean(B, ii, values):
    """Per sequence: (exactly rounded sum of ``values`` over its active
    tokens) / max(L_i, 1); ii lists the active tokens' sequences in order."""
    bounds = _seq_bounds(B, ii)
    out = np.zeros(B, dtype=np.float64)
    for i in range(B):
        s0, e0 = int(bounds[i]), int(bounds[i + 1])
        out[i] = math.fsum(values[s0:e0]) / max(e0 - s0, 1)
    return out


def sequence_mask_keep(B, ii, old_act, gen_act, lo, hi):
    """seq-mask-tis ([DOCKYARD] Off-policy correction): sequence i is kept
    when its geometric-mean importance ratio exp(mean_t(old - gen)) lies in
    [lo, hi]."""
    diff = np.asarray(old_act, dtype=np.float64) - np.asarray(gen_act, dtype=np.float64)
    r = np.exp(sequence_mean(B, ii, diff))
    return (r >= lo) & (r <= hi)


def gspo_terms(s, adv, cfg: LossConfig):
    """Sequence-level clipped surrogate ([RPP] Formula-level comparison, GSPO
    row): rho_i = exp(s_i); l_i = -min(rho A, clip(rho) A); dl_i/ds_i =
    -A rho unless clipped (then 0; drho/ds = rho).  Clipped as for the token
    form: strictly outside the band on the side the sign of A selects."""
    s = np.asarray(s, dtype=np.float64)
    A = np.asarray(adv, dtype=np.float64)
    rho = np.exp(s)
    lo = 1.0 - cfg.eps_low
    hi = 1.0 + cfg.eps_high
    obj = np.minimum(rho * A, np.clip(rho, lo, hi) * A)
    clipped = ((A > 0) & (rho > hi)) | ((A < 0) & (rho < lo))
    dl_ds = np.where(clipped, 0.0, -A * rho)
    return rho, -obj, dl_ds, clipped


def _log1p_sum_exp(z):
    """log(1 + sum exp(z)), float64, as a log-sum-exp with a zero appended
    (the appended term is the 1)."""
    vals = [0.0] + [float(v) for v in z]
    M = max(vals)
    return M + math.log(math.fsum(math.exp(v - M) for v in vals))


def real_terms(s, adv, L, offsets, tau):
    """REAL loss ([REAL-BLOG] REAL formalisation; source walkthrough steps
    1-3).  Returns (group_loss [G], dpolicy/ds [B], policy_loss) with
    policy_loss = sum_g group_loss_g / G."""
    s = np.asarray(s, dtype=np.float64)
    A = np.asarray(adv, dtype=np.float64)
    B = s.shape[0]
    G = len(offsets) - 1
    group_loss = np.zeros(G, dtype=np.float64)
    dpol = np.zeros(B, dtype=np.float64)
    for g in range(G):
        members = range(int(offsets[g]), int(offsets[g + 1]))
        pos = [k for k in members if A[k] > 0 and L[k] > 0]
        neg = [k for k in members if A[k] < 0 and L[k] > 0]
        if not pos or not neg:
            continue
        lse_pos = _log1p_sum_exp([-s[k] / tau for k in pos])
        lse_neg = _log1p_sum_exp([s[k] / tau for k in neg])
        group_loss[g] = lse_pos + lse_neg
        for k in pos:
            dpol[k] = -(1.0 / tau) * math.exp(-s[k] / tau - lse_pos) / G
        for k in neg:
            dpol[k] = (1.0 / tau) * math.exp(s[k] / tau - lse_neg) / G
    total = 0.0
    for g in range(G):
        total = total + group_loss[g]
    return group_loss, dpol, total / G


def policy_terms(logp, old_logp, adv, cfg: LossConfig):
    """Per-token policy loss l, its derivative dl/dlogp and the clip flag.

    A flag marks a token whose surrogate gradient is cut by clipping (clip
    loss, including the dual clip) or, for CISPO, whose ratio lies outside
    the band (its weight is clipped).  At an exact bound the gradient flows:
    torch's clamp passes the gradient there and a tie of the minimum splits it
    in halves that sum to the full value.
    """
    logp = np.asarray(logp, dtype=np.float64)
    A = np.asarray(adv, dtype=np.float64)
    rho = np.exp(logp - np.asarray(old_logp, dtype=np.float64))
    lo = 1.0 - cfg.eps_low
    hi = 1.0 + cfg.eps_high
    if cfg.pg_loss == "clip":
        obj = np.minimum(rho * A, np.clip(rho, lo, hi) * A)
        clipped = ((A > 0) & (rho > hi)) | ((A < 0) & (rho < lo))
        dobj = np.where(clipped, 0.0, A * rho)
        if cfg.dual_clip_c is not None:
            # negative-advantage objective bounded below by c * A
            dual = (A < 0) & (obj < cfg.dual_clip_c * A)
            obj = np.where(dual, cfg.dual_clip_c * A, obj)
            dobj = np.where(dual, 0.0, dobj)
            clipped = clipped | dual
        loss, dloss = -obj, -dobj
    elif cfg.pg_loss == "cispo":
        wgt = np.clip(rho, lo, hi)
        loss = -A * wgt * logp
        dloss = -A * wgt
        clipped = (rho < lo) | (rho > hi)
    elif cfg.pg_loss == "sapo":
        tau = np.where(A > 0, cfg.sapo_tau_pos, cfg.sapo_tau_neg)
        sig = 1.0 / (1.0 + np.exp(-tau * (rho - 1.0)))
        loss = -(4.0 * sig / tau) * A
        dloss = -A * 4.0 * sig * (1.0 - sig) * rho
        clipped = np.zeros(np.shape(loss), dtype=bool)
    elif cfg.pg_loss == "reinforce":
        loss = -A * logp
        dloss = -A * np.ones_like(logp)
        clipped = np.zeros(np.shape(loss), dtype=bool)
    elif cfg.pg_loss == "on_policy":
        loss = -A * np.ones_like(logp)
        dloss = -A * np.ones_like(logp)
        clipped = np.zeros(np.shape(loss), dtype=bool)
    elif cfg.pg_loss in SEQUENCE_PG:
        raise OracleInputError("sequence-level losses need whole sequences (sequence_terms)")
    else:
        raise OracleInputError(f"unknown pg_loss {cfg.pg_loss!r}")
    return rho, loss, dloss, clipped


def kl_terms(d, cfg: LossConfig):
    """Per-token KL estimator value and its derivative with respect to logp
    (d = logp_ref - logp, so dd/dlogp = -1)."""
    d = np.asarray(d, dtype=np.float64)
    if cfg.kl_input_clamp is not None:
        v = cfg.kl_input_clamp
        pass_in = np.abs(d) <= v
        dc = np.clip(d, -v, v)
    else:
        pass_in = np.ones(d.shape, dtype=bool)
        dc = d
    if cfg.kl_estimator == "k3":
        val = np.expm1(dc) - dc
        dval_dd = np.expm1(dc)
    elif cfg.kl_estimator == "k1":
        val = -dc
        dval_dd = -np.ones_like(dc)
    elif cfg.kl_estimator == "k2":
        val = 0.5 * dc * dc
        dval_dd = dc
    else:
        raise OracleInputError(f"unknown kl_estimator {cfg.kl_estimator!r}")
    if cfg.kl_output_clamp is not None:
        w = cfg.kl_output_clamp
        pass_out = np.abs(val) <= w
        val = np.clip(val, -w, w)
    else:
        pass_out = np.ones(d.shape, dtype=bool)
    dkl = np.where(pass_in & pass_out, -dval_dd, 0.0)
    return val, dkl


def token_terms(logp, old_logp, logp_ref, adv, cfg: LossConfig, gen_logp=None, keep=None):
    """Per-token quantities, all float64 arrays of the broadcast shape.

    rho, loss, dloss, clipped from policy_terms; d = logp_ref - logp (0
    without a reference), kl and dkl = d kl / d logp from kl_terms.  With the
    default settings: loss = -min(rho A, clip(rho) A), kl = k3 = e^d - d - 1.
    With the generating policy's log-probs, loss and dloss carry the
    off-policy importance weight (is_weights; ``keep`` per token for
    seq_mask).  For the sequence-level losses (gspo, real) the policy part
    needs whole sequences: here loss, dloss and clipped are 0 and
    sequence_terms fills them in.
    """
    logp = np.asarray(logp, dtype=np.float64)
    if cfg.pg_loss in SEQUENCE_PG:
        rho = np.exp(logp - np.asarray(old_logp, dtype=np.float64))
        loss = np.zeros_like(logp)
        dloss = np.zeros_like(logp)
        clipped = np.zeros(logp.shape, dtype=bool)
    else:
        rho, loss, dloss, clipped = policy_terms(logp, old_logp, adv, cfg)
        if gen_logp is not None:
            wt = is_weights(old_logp, gen_logp, cfg, keep)
            loss = loss * wt
            dloss = dloss * wt
    if logp_ref is None:
        d = np.zeros_like(logp)
    else:
        d = np.asarray(logp_ref, dtype=np.float64) - logp
    kl, dkl = kl_terms(d, cfg)
    return dict(rho=rho, d=d, kl=kl, loss=loss, clipped=clipped, dloss=dloss, dkl=dkl)


def sequence_terms(B, ii, logp_act, old_act, gen_act, A, L, w, offsets, cfg: LossConfig):
    """Policy part of the sequence-level losses.  Returns per active token the
    token loss, the clip flag and gpol = d policy_loss / d logp (weights
    included), plus per sequence s_i (the mean log-ratio) and, for REAL, the
    group losses and the policy loss.

    GSPO: policy_loss = sum_i w_i sum_t omega_t l_i, so by the chain rule
    through s_i = mean_t(logp - old), d/dlogp_t = w_i (sum_t omega_t / L_i) dl_i/ds_i.
    REAL: d/dlogp_t = (d policy_loss / d s_i) / L_i.
    """
    diff = np.asarray(logp_act, dtype=np.float64) - np.asarray(old_act, dtype=np.float64)
    s = sequence_mean(B, ii, diff)
    n = len(ii)
    Lc = np.maximum(np.asarray(L), 1).astype(np.float64)
    if cfg.pg_loss == "gspo":
        _, l_seq, dl_ds, clip_seq = gspo_terms(s, A, cfg)
        om = np.ones(n) if gen_act is None else is_weights(old_act, gen_act, cfg)
        om_mean = sequence_mean(B, ii, om)          # sum_t omega_t / max(L_i, 1)
        loss = om * l_seq[ii]
        gpol = np.asarray(w, dtype=np.float64)[ii] * om_mean[ii] * dl_ds[ii]
        return dict(loss=loss, clipped=clip_seq[ii], gpol=gpol, seq_logratio=s,
                    group_loss=None, policy_loss=None)
    group_loss, dpol, policy_loss = real_terms(s, A, L, offsets, cfg.real_tau)
    gpol = dpol[ii] / Lc[ii]
    return dict(loss=np.zeros(n), clipped=np.zeros(n, dtype=bool), gpol=gpol, seq_logratio=s,
                group_loss=group_loss, policy_loss=policy_loss)


def _check_cfg(cfg: LossConfig, have_ref: bool, have_gen: bool = False):
    if not (0.0 <= cfg.eps_low < 1.0) or cfg.eps_high < 0.0 or cfg.beta < 0.0:
        raise OracleInputError("bad clip range or beta")
    if cfg.beta > 0.0 and not have_ref:
        raise OracleInputError("beta > 0 needs reference log-probs")
    if cfg.reduction not in REDUCTIONS:
        raise OracleInputError("unknown reduction")
    if cfg.reduction == "fixed_constant" and not (cfg.norm_constant and cfg.norm_constant > 0):
        raise OracleInputError("fixed_constant needs norm_constant > 0")
    if cfg.pg_loss not in PG_LOSSES or cfg.kl_estimator not in KL_ESTIMATORS:
        raise OracleInputError("unknown pg_loss or kl_estimator")
    if cfg.dual_clip_c is not None and (cfg.pg_loss != "clip" or not cfg.dual_clip_c > 1.0):
        raise OracleInputError("dual clip needs the clip loss and c > 1")
    if cfg.pg_loss == "sapo" and not (cfg.sapo_tau_pos > 0 and cfg.sapo_tau_neg > 0):
        raise OracleInputError("SAPO temperatures must be positive")
    for v in (cfg.kl_input_clamp, cfg.kl_output_clamp):
        if v is not None and not v > 0:
            raise OracleInputError("KL clamps must be positive")
    if cfg.pg_loss == "gspo" and cfg.reduction == "token_mean":
        raise OracleInputError("sequence-level ratios exclude the token-mean reduction")
    if cfg.pg_loss == "real":
        if cfg.reduction != "token_mean":
            raise OracleInputError("REAL takes its KL term as the global token mean")
        if have_gen:
            raise OracleInputError("REAL takes no off-policy weights")
        if not (cfg.real_tau > 0 and math.isfinite(cfg.real_tau)):
            raise OracleInputError("REAL needs a positive temperature")
    if cfg.tis_type is not None:
        if cfg.tis_type not in TIS_TYPES:
            raise OracleInputError("unknown truncated-IS type")
        if not have_gen:
            raise OracleInputError("truncated IS needs the generating policy's log-probs")
        if cfg.tis_ratio_max is None or not cfg.tis_ratio_max > 0:
            raise OracleInputError("truncated IS needs a positive upper bound")
        if cfg.tis_type in ("icepop", "seq_mask") and cfg.tis_ratio_min is None:
            raise OracleInputError("icepop and seq_mask need a lower bound")
        if cfg.tis_type == "seq_mask" and cfg.pg_loss in SEQUENCE_PG:
            raise OracleInputError("seq_mask is not combined with sequence-level losses")
        lo = 0.0 if cfg.tis_ratio_min is None else cfg.tis_ratio_min
        if not (0.0 <= lo <= cfg.tis_ratio_max):
            raise OracleInputError("truncated IS bounds must satisfy 0 <= min <= max")


@dataclass
class OracleResult:
    loss: float
    policy_loss: float
    kl: float
    advantages: np.ndarray          # [B] float64
    seq_policy: np.ndarray          # [B] sum over active tokens of the token loss
    seq_kl: np.ndarray              # [B] sum over active tokens of the KL estimator
    seq_weight: np.ndarray          # [B] omega_i
    seq_tokens: np.ndarray          # [B] L_i
    num_tokens: int                 # N
    clipped: int                    # number of clipped active tokens
    tok: dict = field(default_factory=dict)   # per-token arrays [B, T] (0 at masked slots)
    grad: np.ndarray | None = None  # d loss / d logits [B, T, V] or d loss / d logp [B, T]
    seq_logratio: np.ndarray | None = None  # [B] s_i (sequence-level losses only)
    group_loss: np.ndarray | None = None    # [G] REAL group losses
    seq_keep: np.ndarray | None = None      # [B] seq_mask: sequence kept


def _reduce(P, K, w, beta):
    """Fixed-order scalar reduction: sum_i w_i * P_i, sum_i w_i * K_i."""
    policy_loss = 0.0
    kl = 0.0
    for i in range(len(w)):
        policy_loss = policy_loss + float(w[i]) * float(P[i])
        kl = kl + float(w[i]) * float(K[i])
    return policy_loss + beta * kl, policy_loss, kl


# ---------------------------------------------------------------------------
# Logprob-level token loss  ([GRPO-CPP] CUDA: the token-loss kernels take
# per-token log-probs and return dlogp)
# ---------------------------------------------------------------------------

def grpo_token_loss(logp, old_logp, ref_logp, mask, rewards, *, groups, cfg: LossConfig,
                    grad_scale=1.0, gen_logp=None, advantages=None):
    """GRPO loss from per-token log-probs.  ``grad`` is d loss / d logp [B, T].

    ``groups`` is a dict with keys samples_per_prompt | group_boundaries and
    optional leave_one_out, scale_by_std, std_eps, adv_clip_low/high.
    ``advantages``: precomputed token advantages [B, T] (then rewards and
    groups are None), e.g. from token_advantages.
    """
    logp = np.asarray(logp)
    B, T = logp.shape
    _check_cfg(cfg, ref_logp is not None, gen_logp is not None)
    m = np.ones((B, T), dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    A, off, A_slot = _advantage_source(rewards, groups, advantages, B, T, cfg)
    L, N, w = sequence_weights(m, cfg.reduction, cfg.alpha, cfg.norm_constant)

    ii, tt = np.nonzero(m)                      # boolean selection: masked slots never read
    lp = np.asarray(logp, dtype=np.float64)[ii, tt]
    old = np.asarray(old_logp, dtype=np.float64)[ii, tt]
    ref = None if ref_logp is None else np.asarray(ref_logp, dtype=np.float64)[ii, tt]
    gen = None if gen_logp is None else np.asarray(gen_logp, dtype=np.float64)[ii, tt]
    keep = _keep(B, ii, old, gen, cfg)
    adv = A_slot[ii, tt]
    terms = token_terms(lp, old, ref, adv, cfg, gen, None if keep is None else keep[ii])
    terms["adv"] = adv
    _add_sequence_terms(terms, B, ii, lp, old, gen, A, L, w, off, cfg)
    return _assemble(B, T, ii, tt, terms, A, L, N, w, cfg, grad_scale,
                     grad=None, logp_active=lp, gen_active=gen, keep=keep)


def _keep(B, ii, old, gen, cfg):
    """Per-sequence keep flags of seq_mask (None otherwise)."""
    if cfg.tis_type != "seq_mask":
        return None
    return sequence_mask_keep(B, ii, old, gen, float(cfg.tis_ratio_min), float(cfg.tis_ratio_max))


def _add_sequence_terms(terms, B, ii, lp, old, gen, A, L, w, off, cfg):
    """For gspo / real: fill in the policy part once every log-prob is known."""
    if cfg.pg_loss not in SEQUENCE_PG:
        return
    sq = sequence_terms(B, ii, lp, old, gen, A, L, w, off, cfg)
    terms["loss"] = sq["loss"]
    terms["clipped"] = sq["clipped"]
    terms["gpol"] = sq["gpol"]
    terms["seq"] = sq


def _token_G(terms, w, ii, cfg, grad_scale):
    """G = d loss / d logp per active token: w_i (dl/dlogp + beta dkl/dlogp),
    or, for the sequence-level losses, gpol + w_i beta dkl/dlogp."""
    if "gpol" in terms:
        return (terms["gpol"] + w[ii] * (cfg.beta * terms["dkl"])) * grad_scale
    return w[ii] * (terms["dloss"] + cfg.beta * terms["dkl"]) * grad_scale


def _assemble(B, T, ii, tt, terms, A, L, N, w, cfg, grad_scale, grad, logp_active,
              gen_active=None, keep=None):
    P = np.zeros(B)
    K = np.zeros(B)
    C = np.zeros(B, dtype=np.int64)
    # per-sequence sums (exactly rounded); ii is sorted, so each sequence's
    # active tokens form one contiguous run
    bounds = np.searchsorted(ii, np.arange(B + 1))
    for i in range(B):
        s, e = int(bounds[i]), int(bounds[i + 1])
        P[i] = math.fsum(terms["loss"][s:e])
        K[i] = math.fsum(terms["kl"][s:e])
        C[i] = int(np.count_nonzero(terms["clipped"][s:e]))
    loss, policy_loss, kl = _reduce(P, K, w, cfg.beta)
    seq = terms.get("seq")
    if seq is not None and seq["policy_loss"] is not None:
        policy_loss = seq["policy_loss"]        # REAL: its own group normalisation
        loss = policy_loss + cfg.beta * kl
    G = _token_G(terms, w, ii, cfg, grad_scale)
    tok = {}
    for name in ("rho", "d", "kl", "loss", "dloss", "dkl", "adv"):
        full = np.zeros((B, T))
        full[ii, tt] = terms[name]
        tok[name] = full
    full = np.zeros((B, T), dtype=bool)
    full[ii, tt] = terms["clipped"]
    tok["clipped"] = full
    Gfull = np.zeros((B, T))
    Gfull[ii, tt] = G
    tok["G"] = Gfull
    lfull = np.zeros((B, T))
    lfull[ii, tt] = logp_active
    tok["logp"] = lfull
    if gen_active is not None:        # the input itself, kept for callers that re-evaluate terms
        gfull = np.zeros((B, T))
        gfull[ii, tt] = gen_active
        tok["gen"] = gfull
    if grad is None:
        grad = Gfull.copy()           # token-level: d loss / d logp = m * G
    return OracleResult(loss=loss, policy_loss=policy_loss, kl=kl, advantages=A,
                        seq_policy=P, seq_kl=K, seq_weight=w, seq_tokens=L,
                        num_tokens=N, clipped=int(C.sum()), tok=tok, grad=grad,
                        seq_logratio=None if seq is None else seq["seq_logratio"],
                        group_loss=None if seq is None else seq["group_loss"],
                        seq_keep=keep)


# ---------------------------------------------------------------------------
# Log-softmax of a vocabulary row  ([GRPO-LOSS] intro: ratio and KL come from
# log-softmax over the vocabulary at the taken token)
# ---------------------------------------------------------------------------

def row_logsumexp(rows):
    """log(sum_v exp(x_v)) per row, float64: M + log(sum exp(x - M))."""
    x = np.asarray(rows, dtype=np.float64)
    M = np.max(x, axis=-1, keepdims=True)
    return (M + np.log(np.sum(np.exp(x - M), axis=-1, keepdims=True)))[..., 0]


def logits_rows(x_rows, y_rows, ids, old, adv, w, cfg: LossConfig, grad_scale=1.0,
                want_grad=True, gen=None, keep=None):
    """Forward + gradient for a set of active rows (each row one token slot).

    x_rows, y_rows: [n, V] policy / reference logits (y_rows may be None when
    beta == 0); ids [n]; old [n]; adv [n] = A of the row's sequence; w [n] =
    omega of the row's sequence; keep [n] the seq_mask flag of the row's
    sequence.  Returns the per-row terms, LSEs, G and the gradient rows
    g_v = G * (onehot(a)_v - softmax(x)_v).  For the sequence-level losses G
    here holds only the KL part (the policy part needs whole sequences).
    """
    x = np.asarray(x_rows, dtype=np.float64)
    n, V = x.shape
    ids = np.asarray(ids, dtype=np.int64)
    if np.any(ids < 0) or np.any(ids >= V):
        raise OracleInputError("action id out of range at an active slot")
    r = np.arange(n)
    lse = row_logsumexp(x)
    logp = x[r, ids] - lse
    if y_rows is not None:
        y = np.asarray(y_rows, dtype=np.float64)
        lse_ref = row_logsumexp(y)
        logp_ref = y[r, ids] - lse_ref
    else:
        lse_ref = None
        logp_ref = None
    terms = token_terms(logp, old, logp_ref, adv, cfg, gen, keep)
    G = np.asarray(w, dtype=np.float64) * (terms["dloss"] + cfg.beta * terms["dkl"]) * grad_scale
    out = dict(terms, lse=lse, lse_ref=lse_ref, logp=logp, logp_ref=logp_ref, G=G)
    if want_grad:
        out["grad"] = softmax_grad_rows(x, ids, lse, G)
    return out


def softmax_grad_rows(x_rows, ids, lse, G):
    """g_v = G * (onehot(a)_v - softmax(x)_v) for each row, softmax from the
    row's log-sum-exp."""
    x = np.asarray(x_rows, dtype=np.float64)
    r = np.arange(x.shape[0])
    p = np.exp(x - np.asarray(lse, dtype=np.float64)[:, None])
    g = -G[:, None] * p
    g[r, ids] = G * (1.0 - p[r, ids])
    return g


def grpo_loss_fwd_bwd(policy_logits, ref_logits, action_ids, old_logps, mask, rewards, *,
                      groups, cfg: LossConfig, grad_scale=1.0, want_grad=True,
                      row_chunk=4096, gen_logps=None, advantages=None):
    """GRPO loss and d loss / d policy_logits from [B, T, V] logits.

    Masked rows get an all-zero gradient row and are never read.
    ``advantages``: precomputed token advantages [B, T], as for grpo_token_loss.
    """
    x = np.asarray(policy_logits)
    if x.ndim != 3:
        raise OracleInputError("policy_logits must be [B, T, V]")
    B, T, V = x.shape
    y = None if ref_logits is None else np.asarray(ref_logits)
    grad = np.zeros((B, T, V)) if want_grad else None

    def fetch(ii, tt):
        return x[ii, tt], (None if y is None else y[ii, tt])

    def sink(ii, tt, rows):
        grad[ii, tt] = rows

    res = grpo_loss_rows(fetch, (B, T, V), action_ids, old_logps, mask, rewards, groups=groups,
                         cfg=cfg, have_ref=y is not None, grad_scale=grad_scale,
                         row_chunk=row_chunk, gen_logps=gen_logps, advantages=advantages,
                         grad_sink=sink if want_grad else None)
    res.grad = grad
    return res


def grpo_loss_rows(fetch_rows, shape, action_ids, old_logps, mask, rewards, *, groups,
                   cfg: LossConfig, have_ref=True, grad_scale=1.0, row_chunk=4096,
                   gen_logps=None, advantages=None, grad_sink=None, map_chunks=map):
    """The computation of grpo_loss_fwd_bwd over logits that are not held
    whole: ``fetch_rows(ii, tt)`` returns the policy and reference rows
    ([n, V] each; the reference None without one) of the active slots
    (ii, tt), and ``grad_sink(ii, tt, grad_rows)``, if given, receives the
    gradient rows of those slots instead of a [B, T, V] array.  Chunks of
    ``row_chunk`` active slots are independent, so ``map_chunks`` (the
    builtin ``map`` or a thread pool's ``map``) may evaluate them in any
    order; the per-token values land at their slots and every sum runs in
    _assemble, so the result does not depend on it.  The returned result's
    ``grad`` is None; its ``tok`` also holds each active row's policy
    log-sum-exp (``lse``)."""
    B, T, V = shape
    _check_cfg(cfg, have_ref, gen_logps is not None)
    m = np.ones((B, T), dtype=bool) if mask is None else np.asarray(mask).astype(bool)
    A, off, A_slot = _advantage_source(rewards, groups, advantages, B, T, cfg)
    L, N, w = sequence_weights(m, cfg.reduction, cfg.alpha, cfg.norm_constant)
    ii, tt = np.nonzero(m)
    adv = A_slot[ii, tt]
    ids = np.asarray(action_ids)[ii, tt].astype(np.int64)
    old = np.asarray(old_logps, dtype=np.float64)[ii, tt]
    gen = None if gen_logps is None else np.asarray(gen_logps, dtype=np.float64)[ii, tt]
    keep = _keep(B, ii, old, gen, cfg)
    seq_level = cfg.pg_loss in SEQUENCE_PG
    keys = ("rho", "d", "kl", "loss", "dloss", "dkl", "logp", "lse", "clipped")
    acc = {k: np.zeros(len(ii)) for k in keys[:-1]}
    acc["clipped"] = np.zeros(len(ii), dtype=bool)
    starts = range(0, len(ii), row_chunk)

    def forward_chunk(s):
        sl = slice(s, s + row_chunk)
        xr, yr = fetch_rows(ii[sl], tt[sl])
        rows_grad = grad_sink is not None and not seq_level
        out = logits_rows(xr, yr, ids[sl], old[sl], adv[sl], w[ii[sl]], cfg, grad_scale,
                          rows_grad, None if gen is None else gen[sl],
                          None if keep is None else keep[ii[sl]])
        if rows_grad:
            grad_sink(ii[sl], tt[sl], out["grad"])
        return sl, {k: out[k] for k in keys}

    for sl, part in map_chunks(forward_chunk, starts):
        for k in keys:
            acc[k][sl] = part[k]
    if seq_level:
        # the policy part needs every log-prob of a sequence: a second pass
        # over the rows writes the gradient once G is known
        _add_sequence_terms(acc, B, ii, acc["logp"], old, gen, A, L, w, off, cfg)
        if grad_sink is not None:
            G = _token_G(acc, w, ii, cfg, grad_scale)

            def gradient_chunk(s):
                sl = slice(s, s + row_chunk)
                xr, _ = fetch_rows(ii[sl], tt[sl])
                grad_sink(ii[sl], tt[sl], softmax_grad_rows(xr, ids[sl], acc["lse"][sl], G[sl]))
                return sl

            for _ in map_chunks(gradient_chunk, starts):
                pass
    acc["adv"] = adv
    res = _assemble(B, T, ii, tt, acc, A, L, N, w, cfg, grad_scale, grad=None,
                    logp_active=acc["logp"], gen_active=gen, keep=keep)
    res.grad = None
    lse = np.zeros((B, T))
    lse[ii, tt] = acc["lse"]
    res.tok["lse"] = lse
    return res


def grpo_advantages(rewards, *, groups):
    """Advantages alone, as the boundary's advantage entry point returns them
    (with the group specification's clamp, if any)."""
    r = np.asarray(rewards)
    return _advantages_of(r, r.shape[0], groups)[0]


# ---------------------------------------------------------------------------
# Token-level advantage estimators  ([RPP] REINFORCE++, REINFORCE++-baseline,
# Global masked normalization; [DOCKYARD] Advantage estimation (clamp), GDPO)
# ---------------------------------------------------------------------------

ADV_ESTIMATORS = ("reinforce_pp", "reinforce_pp_baseline")


def reinforce_pp_token_rewards(rewards, old_logp, ref_logp, mask, kl_coef):
    """[RPP] REINFORCE++: r_{i,t} = m_{i,t} (-kl_coef * d_{i,t} + 1(t = T_i) R_i)
    with the signed k1 estimator d = log pi_old - log pi_ref and T_i the last
    valid position of response i.  Masked slots are never read."""
    m = np.asarray(mask).astype(bool)
    B, T = m.shape
    R = np.asarray(rewards, dtype=np.float64)
    shaped = kl_coef != 0.0            # without the KL term the log-probs are not needed
    old = np.asarray(old_logp, dtype=np.float64) if shaped else None
    ref = np.asarray(ref_logp, dtype=np.float64) if shaped else None
    r = np.zeros((B, T))
    for i in range(B):
        valid = np.nonzero(m[i])[0]
        if shaped:
            for t in valid:
                r[i, t] = -kl_coef * (old[i, t] - ref[i, t])
        if valid.size:
            r[i, valid[-1]] = r[i, valid[-1]] + R[i]
    return r


def discounted_returns(r, mask, gamma):
    """G_{i,t} = m_{i,t} sum_{u >= t} gamma^(u - t) r_{i,u}, accumulated
    backwards over positions (r is 0 at masked slots)."""
    m = np.asarray(mask).astype(bool)
    B, T = m.shape
    G = np.zeros((B, T))
    for i in range(B):
        acc = 0.0
        for t in range(T - 1, -1, -1):
            acc = float(r[i, t]) + gamma * acc
            G[i, t] = acc if m[i, t] else 0.0
    return G


def reinforce_pp_baseline_raw(rewards, offsets, mask):
    """[RPP] REINFORCE++-baseline: C_i = R_i - (mean of the group, the sample
    itself included; no std division), broadcast to the valid tokens."""
    m = np.asarray(mask).astype(bool)
    R = [float(v) for v in np.asarray(rewards, dtype=np.float64).ravel()]
    C = np.zeros(len(R))
    for g in range(len(offsets) - 1):
        s, e = int(offsets[g]), int(offsets[g + 1])
        total = 0.0
        for j in range(s, e):
            total = total + R[j]
        b = total / (e - s)
        for j in range(s, e):
            C[j] = R[j] - b
    return np.where(m, C[:, None], 0.0)


def global_masked_normalize(A, mask, var_floor=1e-8):
    """[RPP] Global masked normalization: over every valid token,
    mu = mean, var = population variance (ddof 0), and
    A_hat = m (A - mu) / sqrt(max(var, var_floor)).  An empty mask gives zeros."""
    m = np.asarray(mask).astype(bool)
    vals = np.asarray(A, dtype=np.float64)[m]
    N = vals.size
    if N == 0:
        return np.zeros(m.shape)
    mu = math.fsum(vals) / N
    var = math.fsum((v - mu) * (v - mu) for v in vals) / N
    return np.where(m, (np.asarray(A, dtype=np.float64) - mu) / math.sqrt(max(var, var_floor)), 0.0)


def clamp_advantages(A, low, high):
    """[DOCKYARD] Advantage estimation: clamp to [advantage_clip_low,
    advantage_clip_high]."""
    return np.clip(np.asarray(A, dtype=np.float64), low, high)


def token_advantages(estimator, rewards, old_logp, ref_logp, mask, *, groups=None, kl_coef=0.0,
                     gamma=1.0, normalize=True):
    """[B, T] advantages of a token-level estimator, float64.

    reinforce_pp: returns of the k1-shaped token rewards (KL-to-go plus the
    terminal reward); reinforce_pp_baseline: the inclusive group-mean
    difference broadcast to the valid tokens.  Then, optionally, the global
    masked normalization, and the group specification's clamp if it has one
    (``groups`` keys adv_clip_low / adv_clip_high)."""
    m = np.asarray(mask).astype(bool)
    B, T = m.shape
    if estimator not in ADV_ESTIMATORS:
        raise OracleInputError(f"unknown estimator {estimator!r}")
    if not (0.0 < gamma <= 1.0):
        raise OracleInputError("gamma must lie in (0, 1]")
    if estimator == "reinforce_pp":
        if (ref_logp is None or old_logp is None) and kl_coef != 0.0:
            raise OracleInputError("KL shaping needs the old and reference log-probs")
        r = reinforce_pp_token_rewards(rewards, old_logp, ref_logp, m, kl_coef)
        A = discounted_returns(r, m, gamma)
    else:
        if groups is None:
            raise OracleInputError("the baseline estimator needs reward groups")
        off = group_offsets(B, groups.get("samples_per_prompt"), groups.get("group_boundaries"))
        A = reinforce_pp_baseline_raw(rewards, off, m)
    if normalize:
        A = global_masked_normalize(A, m)
    if groups is not None and groups.get("adv_clip_low") is not None:
        A = np.where(m, clamp_advantages(A, groups["adv_clip_low"], groups["adv_clip_high"]), 0.0)
    return A


def gdpo_advantages(component_rewards, *, groups, std_eps=1e-6):
    """[DOCKYARD] GDPO: for each reward component a per-group baseline (the
    group's leave_one_out flag; the page's GDPO uses leave-one-out),
    optionally divided by the component's group std (scale_by_std), summed
    over components, then renormalized over the batch to zero mean and unit
    population std (floored at std_eps); finally the optional clamp."""
    Rc = np.asarray(component_rewards, dtype=np.float64)
    if Rc.ndim != 2 or Rc.shape[0] < 2:
        raise OracleInputError("GDPO needs at least two reward components [C, B]")
    C, B = Rc.shape
    off = group_offsets(B, groups.get("samples_per_prompt"), groups.get("group_boundaries"))
    total = np.zeros(B)
    for c in range(C):
        total = total + group_advantages(Rc[c], off, groups.get("leave_one_out", True),
                                         groups.get("scale_by_std", True),
                                         groups.get("std_eps", std_eps))
    vals = [float(v) for v in total]
    mu = math.fsum(vals) / B
    sd = math.sqrt(math.fsum((v - mu) * (v - mu) for v in vals) / B)
    A = (total - mu) / max(sd, groups.get("std_eps", std_eps))
    if groups.get("adv_clip_low") is not None:
        A = clamp_advantages(A, groups["adv_clip_low"], groups["adv_clip_high"])
    return A
