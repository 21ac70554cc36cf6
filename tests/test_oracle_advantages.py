"""Pins for the oracle's token-level advantage estimators (Relax REINFORCE++
page: REINFORCE++, REINFORCE++-baseline, Global masked normalization; PPO and
KL reduction), GDPO multi-reward advantages and the advantage clamp
(dockyard_rl, Advantage estimation), and the loss fed precomputed token
advantages.  Each against closed forms, numpy/torch library routines or an
independent torch autograd formulation of the whole recipe."""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as orc
from oracle import LossConfig, OracleInputError


def _mask(rng, B, T, holes=False):
    lens = rng.integers(1, T + 1, B)
    m = np.arange(T)[None, :] < lens[:, None]
    if holes:
        m &= rng.random((B, T)) > 0.2
        m[np.arange(B), 0] = True
    return m


def test_returns_terminal_reward_reaches_every_valid_token():
    """beta = 0, gamma = 1: every valid token's return is the response's reward."""
    rng = np.random.default_rng(0)
    B, T = 6, 9
    m = _mask(rng, B, T, holes=True)
    R = rng.normal(size=B)
    old = rng.normal(size=(B, T))
    r = orc.reinforce_pp_token_rewards(R, old, old + 1.0, m, 0.0)
    G = orc.discounted_returns(r, m, 1.0)
    np.testing.assert_array_equal(G, np.where(m, R[:, None], 0.0))


def test_returns_are_kl_to_go_with_zero_reward():
    """R = 0, gamma = 1: G_t = -beta * (sum over valid u >= t of d_u), checked
    with numpy's cumulative sum of the reversed row."""
    rng = np.random.default_rng(1)
    B, T = 5, 12
    m = _mask(rng, B, T, holes=True)
    old = rng.normal(size=(B, T))
    ref = old + rng.normal(0, 0.3, (B, T))
    beta = 0.07
    G = orc.discounted_returns(orc.reinforce_pp_token_rewards(np.zeros(B), old, ref, m, beta), m, 1.0)
    d = np.where(m, old - ref, 0.0)
    togo = np.cumsum(d[:, ::-1], axis=1)[:, ::-1]
    np.testing.assert_allclose(G, np.where(m, -beta * togo, 0.0), rtol=1e-13, atol=1e-15)


def test_returns_geometric_closed_form():
    """Prefix mask of length L, constant d and reward R, gamma < 1:
    G_t = -beta d (1 - gamma^(L - t)) / (1 - gamma) + gamma^(L - 1 - t) R."""
    B, T, L = 1, 10, 7
    m = np.arange(T)[None, :] < L
    old = np.full((B, T), 0.3)
    ref = np.full((B, T), 0.1)
    beta, gamma, R = 0.5, 0.9, 2.0
    G = orc.discounted_returns(orc.reinforce_pp_token_rewards([R], old, ref, m, beta), m, gamma)
    d = 0.2
    for t in range(L):
        want = -beta * d * (1 - gamma ** (L - t)) / (1 - gamma) + gamma ** (L - 1 - t) * R
        assert G[0, t] == pytest.approx(want, rel=1e-13)
    assert np.all(G[0, L:] == 0.0)


def test_returns_discount_counts_positions_across_holes():
    """The discount exponent is the position distance u - t, so a masked hole
    between two valid tokens still costs one factor of gamma."""
    m = np.array([[True, False, True]])
    r = orc.reinforce_pp_token_rewards([1.0], np.zeros((1, 3)), np.zeros((1, 3)), m, 0.0)
    G = orc.discounted_returns(r, m, 0.5)
    assert G[0, 2] == 1.0 and G[0, 1] == 0.0 and G[0, 0] == 0.25


def test_masked_slots_are_never_read():
    rng = np.random.default_rng(2)
    B, T = 4, 8
    m = _mask(rng, B, T, holes=True)
    old = rng.normal(size=(B, T))
    ref = old + 0.1
    R = rng.normal(size=B)
    a = orc.token_advantages("reinforce_pp", R, old, ref, m, kl_coef=0.1)
    old2, ref2 = old.copy(), ref.copy()
    old2[~m] = np.nan
    ref2[~m] = np.inf
    b = orc.token_advantages("reinforce_pp", R, old2, ref2, m, kl_coef=0.1)
    np.testing.assert_array_equal(a, b)


def test_baseline_is_inclusive_group_mean_without_std():
    rng = np.random.default_rng(3)
    B, T, n = 12, 5, 4
    m = _mask(rng, B, T)
    R = rng.normal(size=B)
    A = orc.token_advantages("reinforce_pp_baseline", R, None, None, m,
                             groups=dict(samples_per_prompt=n), normalize=False)
    C = (R.reshape(-1, n) - R.reshape(-1, n).mean(axis=1, keepdims=True)).ravel()
    np.testing.assert_allclose(A, np.where(m, C[:, None], 0.0), rtol=1e-14, atol=1e-15)
    with pytest.raises(OracleInputError):     # one sample per prompt collapses to zero
        orc.token_advantages("reinforce_pp_baseline", R, None, None, m,
                             groups=dict(samples_per_prompt=1))


def test_global_masked_normalization_moments_and_edges():
    rng = np.random.default_rng(4)
    B, T = 7, 11
    m = _mask(rng, B, T, holes=True)
    A = rng.normal(3.0, 2.0, (B, T))
    An = orc.global_masked_normalize(A, m)
    vals = An[m]
    assert abs(np.mean(vals)) < 1e-14
    assert np.var(vals) == pytest.approx(1.0, rel=1e-13)        # population variance (ddof 0)
    assert np.all(An[~m] == 0.0)
    # the floor is on the variance: var 1e-10 divides by sqrt(1e-8) = 1e-4
    tiny = np.where(m, 5.0 + 1e-5 * rng.choice([-1.0, 1.0], (B, T)), 0.0)
    vt = np.var(tiny[m])
    assert vt < 1e-8
    out = orc.global_masked_normalize(tiny, m)
    np.testing.assert_allclose(out[m], (tiny[m] - tiny[m].mean()) / 1e-4, rtol=1e-8, atol=1e-12)
    # zero variance, a single valid token, an empty mask: finite zeros
    assert np.all(orc.global_masked_normalize(np.full((B, T), 2.5), m) == 0.0)
    one = np.zeros((B, T), dtype=bool)
    one[2, 3] = True
    assert np.all(orc.global_masked_normalize(A, one) == 0.0)
    assert np.all(orc.global_masked_normalize(A, np.zeros((B, T), dtype=bool)) == 0.0)


def test_gdpo_two_identical_components_equal_normalized_loo():
    """Summing two copies of a component doubles it; the batch renormalisation
    removes the factor, leaving the normalized leave-one-out GRPO advantage."""
    rng = np.random.default_rng(5)
    B, n = 16, 4
    r = rng.integers(0, 2, B).astype(np.float64)
    r[:n] = [1.0, 0.0, 0.0, 1.0]
    g = dict(samples_per_prompt=n, leave_one_out=True, scale_by_std=True)
    A = orc.gdpo_advantages(np.stack([r, r]), groups=g)
    rr = r.reshape(-1, n)
    mean = rr.mean(axis=1, keepdims=True)
    sd = np.maximum(rr.std(axis=1, keepdims=True), 1e-6)
    loo = ((rr - (rr.sum(axis=1, keepdims=True) - rr) / (n - 1)) / sd).ravel()
    want = (loo - loo.mean()) / loo.std()
    np.testing.assert_allclose(A, want, rtol=1e-12, atol=1e-13)
    assert abs(A.mean()) < 1e-14 and A.std() == pytest.approx(1.0, rel=1e-13)
    with pytest.raises(OracleInputError):
        orc.gdpo_advantages(r[None, :], groups=g)


def test_gdpo_component_scale_and_constant_components():
    rng = np.random.default_rng(6)
    B, n = 12, 3
    a = rng.normal(size=B)
    b = rng.integers(0, 2, B).astype(np.float64)
    g = dict(samples_per_prompt=n, leave_one_out=True, scale_by_std=True)
    base = orc.gdpo_advantages(np.stack([a, b]), groups=g)
    # per-component std normalisation: an affine change of one component is invisible
    np.testing.assert_allclose(orc.gdpo_advantages(np.stack([7.0 * a - 3.0, b]), groups=g), base,
                               rtol=1e-10, atol=1e-12)
    # a component constant across every sample adds nothing
    c = np.full(B, 0.42)
    np.testing.assert_allclose(orc.gdpo_advantages(np.stack([a, b, c]), groups=g), base,
                               rtol=1e-12, atol=1e-13)


def test_advantage_clamp():
    rng = np.random.default_rng(7)
    B, n = 16, 4
    r = rng.normal(size=B)
    g = dict(samples_per_prompt=n)
    free = orc.grpo_advantages(r, groups=g)
    cl = orc.grpo_advantages(r, groups=dict(g, adv_clip_low=-0.5, adv_clip_high=0.75))
    np.testing.assert_array_equal(cl, np.clip(free, -0.5, 0.75))
    assert np.any(free < -0.5) and np.any(free > 0.75)
    with pytest.raises(OracleInputError):
        orc.grpo_advantages(r, groups=dict(g, adv_clip_low=1.0, adv_clip_high=0.0))


def _logits_case(rng, B=8, T=6, V=9):
    x = rng.normal(0, 1.5, (B, T, V))
    y = x + rng.normal(0, 0.4, (B, T, V))
    ids = rng.integers(0, V, (B, T))
    lse = scipy.special.logsumexp(x, axis=-1)
    old = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse + rng.normal(0, 0.4, (B, T))
    m = _mask(rng, B, T)
    return x, y, ids, old, m


def test_broadcast_advantages_reproduce_the_rewards_path():
    rng = np.random.default_rng(8)
    x, y, ids, old, m = _logits_case(rng)
    r = rng.integers(0, 2, 8).astype(np.float64)
    g = dict(samples_per_prompt=4, adv_clip_low=-1.0, adv_clip_high=1.0)
    for cfg in (LossConfig(beta=0.2), LossConfig(beta=0.2, pg_loss="cispo", reduction="sequence_mean")):
        a = orc.grpo_loss_fwd_bwd(x, y, ids, old, m, r, groups=g, cfg=cfg)
        At = np.broadcast_to(a.advantages[:, None], (8, 6)).copy()
        b = orc.grpo_loss_fwd_bwd(x, y, ids, old, m, None, groups=None, cfg=cfg, advantages=At)
        assert a.loss == b.loss
        np.testing.assert_array_equal(a.grad, b.grad)


def _torch_rpp_loss(x, ids, old, ref_lp, m, R, cfg, *, estimator, beta_r, spp):
    """Independent torch formulation of the whole recipe: token advantages
    with torch ops (group view/mean, flip + cumsum for the return-to-go,
    masked_select moments), then the PPO clip with those advantages under the
    response-mean reduction and the optional k2 loss, differentiated by
    autograd."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    mt = torch.tensor(m)
    oldt = torch.tensor(old, dtype=torch.float64)
    reft = torch.tensor(ref_lp, dtype=torch.float64)
    Rt = torch.tensor(R, dtype=torch.float64)
    B, T = mt.shape
    z = torch.zeros(B, T, dtype=torch.float64)
    if estimator == "reinforce_pp":
        last = torch.tensor([int(np.nonzero(m[i])[0][-1]) for i in range(B)])
        term = torch.zeros(B, T, dtype=torch.float64)
        term[torch.arange(B), last] = Rt
        r = torch.where(mt, -beta_r * (oldt - reft) + term, z)
        A = torch.where(mt, torch.flip(torch.cumsum(torch.flip(r, [1]), 1), [1]), z)
    else:
        C = (Rt.view(-1, spp) - Rt.view(-1, spp).mean(1, keepdim=True)).reshape(-1, 1)
        A = torch.where(mt, C.expand(B, T), z)
    vals = torch.masked_select(A, mt)
    mu = vals.mean()
    var = ((vals - mu) ** 2).mean()
    A = torch.where(mt, (A - mu) / torch.sqrt(torch.clamp(var, min=1e-8)), z)
    logp = torch.log_softmax(xt, -1).gather(-1, torch.tensor(ids)[..., None])[..., 0]
    ratio = torch.exp(logp - oldt)
    pg = torch.maximum(-ratio * A, -ratio.clamp(1 - cfg.eps_low, 1 + cfg.eps_high) * A)
    L = mt.sum(1).double()
    w = 1.0 / (B * L.clamp_min(1))
    pol = (w[:, None] * torch.where(mt, pg, z)).sum()
    k2 = 0.5 * (logp - reft) ** 2
    klv = (w[:, None] * torch.where(mt, k2, z)).sum()
    tot = pol + cfg.beta * klv
    tot.backward()
    return tot.item(), A.numpy(), xt.grad.numpy()


@pytest.mark.parametrize("estimator", ["reinforce_pp", "reinforce_pp_baseline"])
def test_recipes_against_independent_autograd(estimator):
    """REINFORCE++: KL in the reward (beta_r = 0.01), no KL loss;
    REINFORCE++-baseline: inclusive baseline, separate k2 loss (coef 0.01);
    both with the global normalization and the response-mean PPO loss."""
    for seed in range(3):
        rng = np.random.default_rng(900 + seed)
        x, y, ids, old, m = _logits_case(rng)
        lq = np.take_along_axis(y, ids[..., None], -1)[..., 0] - scipy.special.logsumexp(y, axis=-1)
        R = rng.integers(0, 2, 8).astype(np.float64)
        if estimator == "reinforce_pp":
            A = orc.token_advantages(estimator, R, old, lq, m, kl_coef=0.01, gamma=1.0)
            cfg = LossConfig(beta=0.0, reduction="sequence_mean")
            res = orc.grpo_loss_fwd_bwd(x, None, ids, old, m, None, groups=None, cfg=cfg, advantages=A)
        else:
            A = orc.token_advantages(estimator, R, None, None, m, groups=dict(samples_per_prompt=4))
            cfg = LossConfig(beta=0.01, kl_estimator="k2", reduction="sequence_mean")
            res = orc.grpo_loss_fwd_bwd(x, y, ids, old, m, None, groups=None, cfg=cfg, advantages=A)
        tot, At, grad = _torch_rpp_loss(x, ids, old, lq, m, R, cfg, estimator=estimator,
                                        beta_r=0.01, spp=4)
        np.testing.assert_allclose(A, At, rtol=1e-12, atol=1e-13)
        assert res.loss == pytest.approx(tot, rel=1e-12, abs=1e-15)
        np.testing.assert_allclose(res.grad, grad, rtol=1e-10, atol=1e-14)


def test_token_advantage_contract():
    rng = np.random.default_rng(10)
    x, y, ids, old, m = _logits_case(rng)
    A = rng.normal(size=(8, 6))
    with pytest.raises(OracleInputError):        # both sources
        orc.grpo_loss_fwd_bwd(x, y, ids, old, m, np.ones(8), groups=dict(samples_per_prompt=4),
                              cfg=LossConfig(), advantages=A)
    with pytest.raises(OracleInputError):        # sequence-level losses take [B] advantages
        orc.grpo_loss_fwd_bwd(x, y, ids, old, m, None, groups=None,
                              cfg=LossConfig(pg_loss="gspo", reduction="sequence_mean"), advantages=A)
    with pytest.raises(OracleInputError):
        orc.token_advantages("reinforce_pp", np.ones(8), old, None, m, kl_coef=0.1)
    with pytest.raises(OracleInputError):
        orc.token_advantages("reinforce_pp", np.ones(8), old, old, m, gamma=0.0)


def test_gdpo_leave_one_out_with_unequal_groups():
    """With groups of different sizes the leave-one-out factor n/(n - 1)
    differs between groups, so it survives the batch renormalisation; the
    expected values come from a numpy formulation per group."""
    rng = np.random.default_rng(11)
    sizes = [2, 4, 6]
    bounds = np.concatenate([[0], np.cumsum(sizes)])
    B = int(bounds[-1])
    comps = np.stack([rng.normal(size=B), rng.integers(0, 2, B).astype(np.float64)])
    comps[1, :2] = [0.0, 1.0]
    g = dict(group_boundaries=list(bounds), leave_one_out=True, scale_by_std=True)
    total = np.zeros(B)
    for c in comps:
        for s, e in zip(bounds[:-1], bounds[1:]):
            v = c[s:e]
            n = e - s
            loo = (v.sum() - v) / (n - 1)
            total[s:e] += (v - loo) / max(v.std(), 1e-6)
    want = (total - total.mean()) / total.std()
    np.testing.assert_allclose(orc.gdpo_advantages(comps, groups=g), want, rtol=1e-12, atol=1e-13)
