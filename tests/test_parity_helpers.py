"""CPU checks of the GPU-parity comparison helpers: they accept the oracle's
own results rounded to the GPU's output precision, for every objective
variant, and reject planted mistakes (a wrong loss, a wrong gradient row, a
wrong branch away from any branch point), while accepting the other branch
exactly at a branch point."""

from types import SimpleNamespace

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from _parity import (LOGP_ABS_ERR, branch_ambiguity, compare_logits_grad, compare_scalars,
                     compare_token_values)

VARIANTS = [
    dict(),
    dict(dual_clip_c=2.0),
    dict(pg_loss="cispo", kl_estimator="k2"),
    dict(pg_loss="sapo", sapo_tau_pos=2.0, sapo_tau_neg=0.5),
    dict(pg_loss="reinforce", kl_estimator="k1"),
    dict(pg_loss="on_policy"),
    dict(kl_input_clamp=0.2, kl_output_clamp=0.02),
    dict(reduction="fixed_constant", norm_constant=50.0),
    dict(tis_type="icepop", tis_ratio_min=0.7, tis_ratio_max=1.4, pg_loss="cispo"),
]


def _case(seed, B=8, T=6, V=40, old_std=1.0):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 2.0, (B, T, V))
    y = x + rng.normal(0, 0.3, (B, T, V))
    ids = rng.integers(0, V, (B, T))
    lse = scipy.special.logsumexp(x, axis=-1)
    old = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse + rng.normal(0, old_std, (B, T))
    lens = rng.integers(1, T + 1, B)
    mask = np.arange(T)[None, :] < lens[:, None]
    r = rng.integers(0, 2, B).astype(np.float64)
    r[0], r[1] = 0.0, 1.0
    return x, y, ids, old, mask, r


def _as_result(ref, grad_dtype=torch.float32):
    f = lambda a: torch.tensor(np.asarray(a), dtype=torch.float32)  # noqa: E731
    return SimpleNamespace(loss=f(ref.loss), policy_loss=f(ref.policy_loss), kl=f(ref.kl),
                           seq_policy=f(ref.seq_policy), seq_kl=f(ref.seq_kl),
                           tok_loss=f(ref.tok["loss"]), tok_kl=f(ref.tok["kl"]),
                           grad=torch.tensor(ref.grad).to(grad_dtype))


@pytest.mark.parametrize("kw", VARIANTS, ids=str)
def test_helpers_accept_rounded_oracle(kw):
    cfg = oracle.LossConfig(beta=0.1, **kw)
    x, y, ids, old, mask, r = _case(3)
    gen = old + np.random.default_rng(9).normal(0, 0.4, old.shape) if "tis_type" in kw else None
    ref = oracle.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2),
                                   cfg=cfg, gen_logps=gen)
    for dt, gdt in ((torch.float32, "f32"), (torch.bfloat16, "bf16"), (torch.float16, "f16")):
        res = _as_result(ref, dt)
        compare_scalars(res, ref, cfg, 1e-5)
        compare_token_values(res, ref, cfg, mask, 1e-5)
        compare_logits_grad(res.grad.double().numpy(), ref, cfg, mask, gdt)


def test_helpers_reject_a_wrong_loss():
    cfg = oracle.LossConfig(beta=0.1)
    x, y, ids, old, mask, r = _case(4)
    ref = oracle.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2),
                                   cfg=cfg)
    res = _as_result(ref)
    res.loss = torch.tensor(ref.loss * (1 + 1e-3), dtype=torch.float32)
    with pytest.raises(AssertionError):
        compare_scalars(res, ref, cfg, 1e-5)
    res = _as_result(ref)
    res.seq_kl = res.seq_kl * 1.01
    with pytest.raises(AssertionError):
        compare_scalars(res, ref, cfg, 1e-5)


@pytest.mark.parametrize("bf16", ["f32", "bf16", "f16"])
def test_helpers_reject_a_wrong_gradient_row(bf16):
    cfg = oracle.LossConfig(beta=0.1, pg_loss="cispo")
    x, y, ids, old, mask, r = _case(5)
    ref = oracle.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2),
                                   cfg=cfg)
    i, t = [int(v[0]) for v in np.nonzero(mask & (np.abs(ref.tok["G"]) > 1e-3))]
    g = ref.grad.copy()
    g[i, t] *= 1.05
    with pytest.raises(AssertionError):
        compare_logits_grad(g, ref, cfg, mask, bf16)


def test_branch_flip_rejected_away_from_bounds_accepted_at_a_bound():
    cfg = oracle.LossConfig(beta=0.0, eps_low=0.2, eps_high=0.2)
    x, y, ids, old, mask, r = _case(6, old_std=0.3)
    lse = scipy.special.logsumexp(x, axis=-1)
    logp = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse
    ref = oracle.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2),
                                   cfg=cfg)
    A = ref.advantages[:, None] * np.ones_like(logp)
    # a clipped token far from its bound: flipping it must be caught
    with np.errstate(divide="ignore"):
        far = mask & ref.tok["clipped"] & (np.abs(np.log(ref.tok["rho"] / 1.2)) > 1e-3) & (A > 0)
    assert far.any()
    i, t = [int(v[0]) for v in np.nonzero(far)]
    p = scipy.special.softmax(x[i, t])
    onehot = np.zeros_like(p)
    onehot[ids[i, t]] = 1.0
    g = ref.grad.copy()
    g[i, t] = -ref.seq_weight[i] * A[i, t] * ref.tok["rho"][i, t] * (onehot - p)
    with pytest.raises(AssertionError):
        compare_logits_grad(g, ref, cfg, mask, False, policy=x, ids=ids)
    # put one token a hair above the upper bound (A > 0): either branch is right
    j = np.nonzero(mask & (A > 0))
    i, t = int(j[0][0]), int(j[1][0])
    old2 = old.copy()
    old2[i, t] = logp[i, t] - np.log(1.2) - LOGP_ABS_ERR
    ref2 = oracle.grpo_loss_fwd_bwd(x, y, ids, old2, mask, r, groups=dict(samples_per_prompt=2),
                                    cfg=cfg)
    flag, anyb, _ = branch_ambiguity(ref2, cfg, mask)
    assert flag[i, t] and anyb[i, t] and ref2.tok["clipped"][i, t]
    # the unclipped branch's row: G = -w A rho times (onehot - softmax)
    p = scipy.special.softmax(x[i, t])
    onehot = np.zeros_like(p)
    onehot[ids[i, t]] = 1.0
    G_un = -ref2.seq_weight[i] * A[i, t] * ref2.tok["rho"][i, t]
    g = ref2.grad.copy()
    g[i, t] = G_un * (onehot - p)
    stats = compare_logits_grad(g, ref2, cfg, mask, False, policy=x, ids=ids)
    assert stats["ambiguous"] >= 1
