"""Pins for the oracle's objective variants (policy-loss forms, KL estimators,
KL clamps, the fixed-constant normaliser, the truncated off-policy importance
weight), each against something other than
the oracle: torch autograd of an independent formulation (stop-gradients as
``detach``), central finite differences where the loss value is the quantity
being differentiated, library KL divergences, and closed forms."""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as orc
from oracle import LossConfig


def _case(rng, B=4, T=4, V=6, ratio_noise=0.5):
    x = rng.normal(0, 1.5, (B, T, V))
    y = x + rng.normal(0, 0.5, (B, T, V))
    ids = rng.integers(0, V, (B, T))
    lse = scipy.special.logsumexp(x, axis=-1)
    old = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse + rng.normal(0, ratio_noise, (B, T))
    lens = rng.integers(1, T + 1, B)
    mask = np.arange(T)[None, :] < lens[:, None]
    r = np.tile([1.0, 0.0], B // 2)
    return x, y, ids, old, mask, r


def _torch_loss(x, y, ids, old, mask, r, spp, cfg, gen=None):
    """Independent formulation with torch autograd (float64, CPU)."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    idt = torch.tensor(ids)[..., None]
    mt = torch.tensor(mask)
    oldt = torch.tensor(old, dtype=torch.float64)
    rt = torch.tensor(r, dtype=torch.float64).view(-1, spp)
    A = ((rt - rt.mean(1, keepdim=True)) / rt.std(1, keepdim=True, unbiased=False).clamp_min(1e-6)).reshape(-1, 1)
    logp = torch.log_softmax(xt, -1).gather(-1, idt)[..., 0]
    logq = torch.log_softmax(torch.tensor(y, dtype=torch.float64), -1).gather(-1, idt)[..., 0]
    lo, hi = 1 - cfg.eps_low, 1 + cfg.eps_high
    ratio = torch.exp(logp - oldt)
    if cfg.pg_loss == "clip":
        surr = torch.minimum(ratio * A, ratio.clamp(lo, hi) * A)
        if cfg.dual_clip_c is not None:
            surr = torch.where(A < 0, torch.maximum(surr, cfg.dual_clip_c * A), surr)
        pg = -surr
    elif cfg.pg_loss == "cispo":
        pg = -A * ratio.clamp(lo, hi).detach() * logp
    elif cfg.pg_loss == "sapo":
        tau = torch.where(A > 0, torch.tensor(cfg.sapo_tau_pos, dtype=torch.float64),
                          torch.tensor(cfg.sapo_tau_neg, dtype=torch.float64))
        pg = -4.0 * torch.sigmoid(tau * (ratio - 1.0)) / tau * A
    elif cfg.pg_loss == "reinforce":
        pg = -A * logp
    else:  # on_policy: the ratio pinned to one by a stop-gradient
        r1 = torch.exp(logp - logp.detach())
        pg = -torch.minimum(r1 * A, r1.clamp(lo, hi) * A)
    if gen is not None:                  # constant off-policy weight
        wis = torch.exp(oldt - torch.tensor(gen, dtype=torch.float64))
        if cfg.tis_type is not None:
            wis = wis.clamp(cfg.tis_ratio_min or 0.0, cfg.tis_ratio_max)
        pg = pg * wis
    lr = logq - logp                     # log(pi_ref / pi_theta)
    if cfg.kl_input_clamp is not None:
        lr = lr.clamp(-cfg.kl_input_clamp, cfg.kl_input_clamp)
    if cfg.kl_estimator == "k3":
        kl = torch.exp(lr) - lr - 1
    elif cfg.kl_estimator == "k1":
        kl = -lr
    else:
        kl = 0.5 * lr ** 2
    if cfg.kl_output_clamp is not None:
        kl = kl.clamp(-cfg.kl_output_clamp, cfg.kl_output_clamp)
    L = mt.sum(1).double()
    B = mt.shape[0]
    if cfg.reduction == "token_mean":
        w = torch.full((B,), 1.0 / float(L.sum()), dtype=torch.float64)
    elif cfg.reduction == "sequence_mean":
        w = 1.0 / (B * L.clamp_min(1))
    elif cfg.reduction == "fixed_constant":
        w = torch.full((B,), 1.0 / cfg.norm_constant, dtype=torch.float64)
    else:
        w = torch.where(L > 0, L ** cfg.alpha / (B * L.clamp_min(1)), torch.zeros_like(L))
    z = torch.zeros_like(pg)
    pol = (w[:, None] * torch.where(mt, pg, z)).sum()
    klv = (w[:, None] * torch.where(mt, kl, z)).sum()
    tot = pol + cfg.beta * klv
    tot.backward()
    return tot.item(), pol.item(), klv.item(), xt.grad.numpy()


VARIANTS = [
    dict(pg_loss="clip", dual_clip_c=3.0),
    dict(pg_loss="clip", dual_clip_c=1.5, eps_low=0.1, eps_high=0.3),
    dict(pg_loss="cispo"),
    dict(pg_loss="cispo", eps_low=0.2, eps_high=0.28, kl_estimator="k2"),
    dict(pg_loss="sapo", sapo_tau_pos=1.0, sapo_tau_neg=1.05),
    dict(pg_loss="sapo", sapo_tau_pos=2.0, sapo_tau_neg=0.5, kl_estimator="k1"),
    dict(pg_loss="reinforce"),
    dict(pg_loss="on_policy", reduction="sequence_mean"),
    dict(kl_estimator="k1"),
    dict(kl_estimator="k2", reduction="sequence_mean"),
    dict(kl_input_clamp=0.3),
    dict(kl_output_clamp=0.05, kl_estimator="k2"),
    dict(kl_input_clamp=0.2, kl_output_clamp=0.01),
    dict(reduction="fixed_constant", norm_constant=37.0),
    dict(reduction="length_alpha", alpha=0.5, pg_loss="cispo"),
    dict(tis_type="tis", tis_ratio_max=1.5),
    dict(tis_type="icepop", tis_ratio_min=0.6, tis_ratio_max=1.4, pg_loss="cispo"),
    dict(tis_type="tis", tis_ratio_min=0.2, tis_ratio_max=2.0, dual_clip_c=2.0),
    dict(is_only=True),
]


@pytest.mark.parametrize("kw", VARIANTS, ids=lambda d: "-".join(f"{k}={v}" for k, v in d.items()))
def test_variants_against_independent_autograd(kw):
    kw = dict(kw)
    use_gen = kw.pop("is_only", False) or "tis_type" in kw
    cfg = LossConfig(beta=0.3, **kw)
    for seed in range(3):
        rng = np.random.default_rng(1000 + seed)
        x, y, ids, old, mask, r = _case(rng)
        gen = old + rng.normal(0, 0.6, old.shape) if use_gen else None
        res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2), cfg=cfg,
                                    gen_logps=gen)
        tot, pol, klv, grad = _torch_loss(x, y, ids, old, mask, r, 2, cfg, gen)
        assert abs(res.loss - tot) < 1e-12 * max(1, abs(tot))
        assert abs(res.policy_loss - pol) < 1e-12 * max(1, abs(pol))
        assert abs(res.kl - klv) < 1e-12 * max(1, abs(klv))
        np.testing.assert_allclose(res.grad, grad, atol=1e-14, rtol=1e-10)


def _loss_value(x, y, ids, old, mask, r, cfg, gen=None):
    return orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2), cfg=cfg,
                                 want_grad=False, gen_logps=gen).loss


@pytest.mark.parametrize("kw", [
    dict(pg_loss="clip", dual_clip_c=2.0),
    dict(pg_loss="sapo", sapo_tau_pos=1.5, sapo_tau_neg=0.7),
    dict(pg_loss="reinforce", kl_estimator="k1"),
    dict(kl_estimator="k2", kl_input_clamp=0.4),
    dict(kl_output_clamp=0.02),
], ids=str)
def test_variants_finite_differences(kw):
    """Where no stop-gradient is involved the gradient is the derivative of the
    loss value itself."""
    cfg = LossConfig(beta=0.3, **kw)
    rng = np.random.default_rng(5)
    x, y, ids, old, mask, r = _case(rng, B=2, T=3, V=4, ratio_noise=0.7)
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2), cfg=cfg)
    # keep away from kinks (clip bounds, dual bound, clamp bounds)
    rho, d = res.tok["rho"][mask], res.tok["d"][mask]
    kinks = [1 - cfg.eps_low, 1 + cfg.eps_high] + ([cfg.dual_clip_c] if cfg.dual_clip_c else [])
    assert min(abs(rho[:, None] - np.array(kinks)[None]).ravel()) > 1e-4
    if cfg.kl_input_clamp:
        assert min(abs(abs(d) - cfg.kl_input_clamp)) > 1e-4
    h = 1e-6
    fd = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (_loss_value(xp, y, ids, old, mask, r, cfg) - _loss_value(xm, y, ids, old, mask, r, cfg)) / (2 * h)
    np.testing.assert_allclose(res.grad, fd, atol=3e-9)


def test_k1_and_k2_closed_forms_and_expectations():
    rng = np.random.default_rng(11)
    V = 40
    logp = rng.normal(0, 1, V)
    logp -= scipy.special.logsumexp(logp)
    logq = rng.normal(0, 1, V)
    logq -= scipy.special.logsumexp(logq)
    p = np.exp(logp)
    t1 = orc.token_terms(logp, logp, logq, np.zeros(V), LossConfig(kl_estimator="k1"))
    t2 = orc.token_terms(logp, logp, logq, np.zeros(V), LossConfig(kl_estimator="k2"))
    # k1 = log(p/q): E_p[k1] = KL(p || q)
    assert abs(np.sum(p * t1["kl"]) - np.sum(scipy.special.rel_entr(p, np.exp(logq)))) < 1e-12
    np.testing.assert_allclose(t1["kl"], logp - logq, rtol=1e-15)
    assert np.all(t1["dkl"] == 1.0)
    np.testing.assert_allclose(t2["kl"], 0.5 * (logp - logq) ** 2, rtol=1e-14)
    np.testing.assert_allclose(t2["dkl"], logp - logq, rtol=1e-14)


def test_kl_clamps_closed_form():
    d = np.array([-1.0, -0.25, 0.0, 0.25, 1.0])
    z = np.zeros(5)
    t = orc.token_terms(z, z, d, z, LossConfig(kl_estimator="k1", kl_input_clamp=0.5))
    np.testing.assert_array_equal(t["kl"], [0.5, 0.25, 0.0, -0.25, -0.5])
    np.testing.assert_array_equal(t["dkl"], [0.0, 1.0, 1.0, 1.0, 0.0])
    t = orc.token_terms(z, z, d, z, LossConfig(kl_estimator="k2", kl_output_clamp=0.1))
    np.testing.assert_allclose(t["kl"], [0.1, 0.03125, 0.0, 0.03125, 0.1])
    np.testing.assert_allclose(t["dkl"], [0.0, 0.25, 0.0, -0.25, 0.0])


def test_dual_clip_closed_form():
    """A = -1, c = 3: rho = 5 gives min(-5, -1.2) = -5 below -3, so the
    objective is -3 (loss 3) and the surrogate gradient is cut; rho = 2
    stays at -2 with gradient -A rho = 2."""
    cfg = LossConfig(dual_clip_c=3.0, beta=0.0)
    A = np.array([-1.0, -1.0, 1.0])
    logp = np.log(np.array([5.0, 2.0, 5.0]))
    t = orc.token_terms(logp, np.zeros(3), None, A, cfg)
    np.testing.assert_allclose(t["loss"], [3.0, 2.0, -1.2])
    np.testing.assert_allclose(t["dloss"], [0.0, 2.0, 0.0])
    assert list(t["clipped"]) == [True, False, True]


def test_cispo_sapo_reinforce_on_policy_closed_forms():
    A = np.array([2.0, -1.0])
    logp = np.log(np.array([1.5, 0.5]))           # old = 0: rho = 1.5, 0.5
    z = np.zeros(2)
    c = orc.token_terms(logp, z, None, A, LossConfig(pg_loss="cispo", beta=0.0))
    np.testing.assert_allclose(c["loss"], [-2.0 * 1.2 * math.log(1.5), 1.0 * 0.8 * math.log(0.5)])
    np.testing.assert_allclose(c["dloss"], [-2.4, 0.8])
    assert list(c["clipped"]) == [True, True]
    s = orc.token_terms(np.zeros(2), z, None, A, LossConfig(pg_loss="sapo", sapo_tau_pos=2.0,
                                                             sapo_tau_neg=0.5, beta=0.0))
    # rho = 1: f_tau(1) = 2 / tau, gradient -A (as the clipped surrogate at rho = 1)
    np.testing.assert_allclose(s["loss"], [-2.0 / 2.0 * 2.0, 2.0 / 0.5 * 1.0])
    np.testing.assert_allclose(s["dloss"], -A)
    rf = orc.token_terms(logp, z, None, A, LossConfig(pg_loss="reinforce", beta=0.0))
    np.testing.assert_allclose(rf["loss"], -A * logp)
    np.testing.assert_allclose(rf["dloss"], -A)
    op = orc.token_terms(logp, z, None, A, LossConfig(pg_loss="on_policy", beta=0.0))
    np.testing.assert_allclose(op["loss"], -A)
    np.testing.assert_allclose(op["dloss"], -A)


def test_fixed_constant_normaliser():
    mask = np.array([[1, 1, 0], [1, 0, 0], [0, 0, 0]], dtype=bool)
    L, N, w = orc.sequence_weights(mask, "fixed_constant", norm_constant=8.0)
    assert np.all(w == 0.125) and N == 3
    full = np.ones((2, 4), dtype=bool)
    _, _, wt = orc.sequence_weights(full, "token_mean")
    _, _, wf = orc.sequence_weights(full, "fixed_constant", norm_constant=8.0)
    assert np.array_equal(wt, wf)


def test_variant_validation():
    x, y, ids, old, mask, r = _case(np.random.default_rng(0), B=2, T=2, V=3)
    g = dict(samples_per_prompt=2)
    for bad in (dict(pg_loss="cispo", dual_clip_c=3.0), dict(dual_clip_c=1.0),
                dict(pg_loss="sapo", sapo_tau_pos=0.0), dict(kl_input_clamp=-1.0),
                dict(reduction="fixed_constant"), dict(pg_loss="nope"), dict(kl_estimator="k9")):
        with pytest.raises(orc.OracleInputError):
            orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=LossConfig(**bad))


def test_is_weight_with_gen_equal_old_changes_nothing():
    """exp(old - gen) = 1 exactly: every output is bit-identical to the call
    without the correction (also under truncation bounds around 1)."""
    rng = np.random.default_rng(21)
    x, y, ids, old, mask, r = _case(rng)
    g = dict(samples_per_prompt=2)
    base = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=LossConfig(beta=0.2))
    for extra in (dict(), dict(tis_type="tis", tis_ratio_max=1.0),
                  dict(tis_type="icepop", tis_ratio_min=1.0, tis_ratio_max=3.0)):
        res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g,
                                    cfg=LossConfig(beta=0.2, **extra), gen_logps=old.copy())
        assert res.loss == base.loss and np.array_equal(res.grad, base.grad)


def test_is_weight_closed_forms():
    old = np.log(np.array([5.0, 0.25, 1.0]))
    gen = np.zeros(3)
    np.testing.assert_allclose(orc.is_weights(old, gen, LossConfig()), [5.0, 0.25, 1.0], rtol=1e-15)
    np.testing.assert_allclose(orc.is_weights(old, gen, LossConfig(tis_type="tis", tis_ratio_max=2.0)),
                               [2.0, 0.25, 1.0], rtol=1e-15)
    np.testing.assert_allclose(
        orc.is_weights(old, gen, LossConfig(tis_type="icepop", tis_ratio_min=0.5, tis_ratio_max=2.0)),
        [2.0, 0.5, 1.0], rtol=1e-15)
    # the weight scales the policy loss and its gradient, not the KL
    A = np.array([1.0, -1.0, 2.0])
    logp = np.log(np.array([1.1, 0.9, 1.0])) + old
    cfg = LossConfig(tis_type="tis", tis_ratio_max=2.0, beta=0.5)
    t0 = orc.token_terms(logp, old, logp + 0.1, A, LossConfig(beta=0.5))
    t1 = orc.token_terms(logp, old, logp + 0.1, A, cfg, gen)
    np.testing.assert_allclose(t1["loss"], t0["loss"] * [2.0, 0.25, 1.0], rtol=1e-15)
    np.testing.assert_allclose(t1["dloss"], t0["dloss"] * [2.0, 0.25, 1.0], rtol=1e-15)
    assert np.array_equal(t1["kl"], t0["kl"]) and np.array_equal(t1["dkl"], t0["dkl"])


def test_is_finite_differences():
    """The weight depends on no logit, so the gradient is the derivative of
    the loss value."""
    cfg = LossConfig(beta=0.3, tis_type="icepop", tis_ratio_min=0.7, tis_ratio_max=1.3)
    rng = np.random.default_rng(8)
    x, y, ids, old, mask, r = _case(rng, B=2, T=3, V=4, ratio_noise=0.7)
    gen = old + rng.normal(0, 0.5, old.shape)
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2), cfg=cfg,
                                gen_logps=gen)
    rho = res.tok["rho"][mask]
    assert min(abs(rho[:, None] - np.array([0.8, 1.2])[None]).ravel()) > 1e-4
    h = 1e-6
    fd = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = (_loss_value(xp, y, ids, old, mask, r, cfg, gen)
                   - _loss_value(xm, y, ids, old, mask, r, cfg, gen)) / (2 * h)
    np.testing.assert_allclose(res.grad, fd, atol=3e-9)


def test_is_validation():
    x, y, ids, old, mask, r = _case(np.random.default_rng(0), B=2, T=2, V=3)
    g = dict(samples_per_prompt=2)
    bad = [(dict(tis_type="tis", tis_ratio_max=2.0), None),            # no generating log-probs
           (dict(tis_type="icepop", tis_ratio_max=2.0), old),          # icepop without a minimum
           (dict(tis_type="tis", tis_ratio_min=3.0, tis_ratio_max=2.0), old),
           (dict(tis_type="tis"), old),
           (dict(tis_type="clip", tis_ratio_max=2.0), old)]
    for kw, gen in bad:
        with pytest.raises(orc.OracleInputError):
            orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=LossConfig(**kw), gen_logps=gen)
