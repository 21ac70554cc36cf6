"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test checks the oracle against something other than itself: a library
routine (scipy / numpy / torch autograd), a closed form worked out by hand
from the definitions, finite differences, or an invariant the mathematics
fixes.  They are chosen so that a dropped term, a flipped sign, a wrong index
or a transposed operand in the oracle fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle as orc
from oracle import LossConfig

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, B=4, T=3, V=5, spp=2, ragged=True, scale=1.0, old_noise=0.2, ref_noise=0.3):
    x = rng.normal(0, scale, (B, T, V))
    y = x + rng.normal(0, ref_noise, (B, T, V))
    ids = rng.integers(0, V, (B, T))
    lse = scipy.special.logsumexp(x, axis=-1)
    old = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse + rng.normal(0, old_noise, (B, T))
    if ragged:
        lens = rng.integers(1, T + 1, B)
        mask = np.arange(T)[None, :] < lens[:, None]
    else:
        mask = np.ones((B, T), dtype=bool)
    rewards = rng.integers(0, 2, B).astype(float)
    # avoid all groups degenerate for a meaningful check
    rewards[::spp] = 1.0
    rewards[1::spp] = 0.0
    return x, y, ids, old, mask, rewards


# ---------------------------------------------------------------------------
# log-sum-exp
# ---------------------------------------------------------------------------

def test_row_logsumexp_matches_scipy():
    rng = np.random.default_rng(0)
    for V in (1, 2, 7, 32, 1000, 4097):
        x = rng.normal(0, 5, (6, V))
        np.testing.assert_allclose(orc.row_logsumexp(x), scipy.special.logsumexp(x, axis=-1),
                                   rtol=1e-14, atol=1e-13)


def test_row_logsumexp_brute_force_tiny():
    rng = np.random.default_rng(1)
    for V in (1, 3, 16, 64):
        x = rng.normal(0, 2, V)
        brute = math.log(math.fsum(math.exp(v) for v in x))
        assert abs(orc.row_logsumexp(x[None])[0] - brute) <= 1e-14 * max(1.0, abs(brute))


def test_row_logsumexp_neg_inf_entries():
    x = np.array([[0.0, -np.inf, math.log(3.0), -np.inf]])
    assert abs(orc.row_logsumexp(x)[0] - math.log(4.0)) < 1e-15


def test_shift_invariance_of_logits():
    rng = np.random.default_rng(2)
    x, y, ids, old, mask, r = _rand_case(rng)
    cfg = LossConfig(beta=0.04)
    g = dict(samples_per_prompt=2)
    a = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=cfg)
    b = orc.grpo_loss_fwd_bwd(x + 7.25, y - 3.5, ids, old, mask, r, groups=g, cfg=cfg)
    assert abs(a.loss - b.loss) < 1e-13
    np.testing.assert_allclose(a.grad, b.grad, atol=1e-14)


# ---------------------------------------------------------------------------
# k3 reference KL
# ---------------------------------------------------------------------------

def test_k3_expectation_is_kl_divergence():
    """E_{a ~ p_theta}[k3(a)] = KL(p_theta || p_ref) fixes the direction of d."""
    rng = np.random.default_rng(3)
    for V in (2, 5, 50):
        xt = rng.normal(0, 1.5, V)
        yr = rng.normal(0, 1.5, V)
        logp = xt - scipy.special.logsumexp(xt)
        logq = yr - scipy.special.logsumexp(yr)
        terms = orc.token_terms(logp, np.zeros(V), logq, np.zeros(V), LossConfig())
        p = np.exp(logp)
        expect = np.sum(scipy.special.rel_entr(p, np.exp(logq)))
        assert abs(np.sum(p * terms["kl"]) - expect) < 1e-12
        # the opposite direction must NOT match (the test would catch a swapped d)
        wrong = np.sum(scipy.special.rel_entr(np.exp(logq), p))
        assert abs(np.sum(p * terms["kl"]) - wrong) > 1e-6


def test_k3_nonnegative_and_zero_at_zero():
    d = np.linspace(-5, 5, 101)
    t = orc.token_terms(np.zeros_like(d), np.zeros_like(d), d, np.zeros_like(d), LossConfig())
    assert np.all(t["kl"] >= 0)
    t0 = orc.token_terms(np.array([0.3]), np.array([0.0]), np.array([0.3]), np.array([1.0]), LossConfig())
    assert t0["kl"][0] == 0.0 and t0["dkl"][0] == 0.0


# ---------------------------------------------------------------------------
# advantages
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("n", [2, 3, 4, 8, 16])
def test_advantages_bernoulli_closed_form(n):
    """k ones among n: A(1) = sqrt((n-k)/k), A(0) = -sqrt(k/(n-k)); the
    leave-one-out version is n/(n-1) times that."""
    rng = np.random.default_rng(n)
    for k in range(1, n):
        r = np.zeros(n)
        r[rng.permutation(n)[:k]] = 1.0
        off = orc.group_offsets(n, samples_per_prompt=n)
        A = orc.group_advantages(r, off)
        np.testing.assert_allclose(A[r == 1], math.sqrt((n - k) / k), rtol=1e-14)
        np.testing.assert_allclose(A[r == 0], -math.sqrt(k / (n - k)), rtol=1e-14)
        Al = orc.group_advantages(r, off, leave_one_out=True)
        np.testing.assert_allclose(Al, n / (n - 1) * A, rtol=1e-14)
        An = orc.group_advantages(r, off, scale_by_std=False)
        np.testing.assert_allclose(An, r - k / n, rtol=1e-15, atol=1e-16)


def test_advantages_against_numpy_group_stats():
    rng = np.random.default_rng(4)
    sizes = [4, 8, 16, 4, 2, 5]
    off = np.concatenate([[0], np.cumsum(sizes)])
    r = rng.normal(0.3, 2.0, off[-1])
    A = orc.group_advantages(r, off)
    for g in range(len(sizes)):
        s, e = off[g], off[g + 1]
        ref = (r[s:e] - np.mean(r[s:e])) / max(np.std(r[s:e], ddof=0), 1e-6)
        np.testing.assert_allclose(A[s:e], ref, rtol=1e-12)


def test_advantages_affine_invariance():
    rng = np.random.default_rng(5)
    r = rng.normal(0, 1, 24)
    off = orc.group_offsets(24, samples_per_prompt=8)
    for loo in (False, True):
        a = orc.group_advantages(r, off, leave_one_out=loo)
        b = orc.group_advantages(2.5 * r - 1.75, off, leave_one_out=loo)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_degenerate_group_zero_advantage_and_gradient():
    rng = np.random.default_rng(6)
    x, y, ids, old, mask, r = _rand_case(rng, B=4, spp=2)
    r[:2] = 1.0   # group 0 all equal
    g = dict(samples_per_prompt=2)
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=LossConfig(beta=0.0))
    assert np.all(res.advantages[:2] == 0.0)
    assert np.all(res.grad[:2] == 0.0)
    assert np.any(res.grad[2:] != 0.0)
    res2 = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=LossConfig(beta=0.1))
    # only the KL part remains in group 0: G = w * beta * (1 - e^d)
    G = res2.tok["G"][:2]
    expect = res2.seq_weight[:2, None] * 0.1 * (-np.expm1(res2.tok["d"][:2])) * mask[:2]
    np.testing.assert_allclose(G, expect, rtol=1e-14, atol=0)


def test_group_spec_csr_example():
    """The page's CSR example (three groups of eight) equals uniform groups of 8."""
    with open(os.path.join(GOLDEN, "group_spec_example.json")) as f:
        case = json.load(f)
    B = case["B"]
    rng = np.random.default_rng(7)
    r = rng.integers(0, 2, B).astype(float)
    a = orc.grpo_advantages(r, groups=dict(group_boundaries=case["group_boundaries"]))
    b = orc.grpo_advantages(r, groups=dict(samples_per_prompt=case["samples_per_prompt"]))
    assert np.array_equal(a, b)


def test_group_spec_errors():
    with pytest.raises(orc.OracleInputError):
        orc.group_offsets(8)
    with pytest.raises(orc.OracleInputError):
        orc.group_offsets(8, samples_per_prompt=4, group_boundaries=[0, 4, 8])
    with pytest.raises(orc.OracleInputError):
        orc.group_offsets(10, samples_per_prompt=4)
    with pytest.raises(orc.OracleInputError):
        orc.group_offsets(8, group_boundaries=[0, 4, 7])
    with pytest.raises(orc.OracleInputError):
        orc.group_offsets(8, group_boundaries=[0, 4, 3, 8])
    with pytest.raises(orc.OracleInputError):
        orc.group_offsets(8, group_boundaries=[0, 1, 8])     # singleton group
    with pytest.raises(orc.OracleInputError):
        orc.group_offsets(8, samples_per_prompt=1)


# ---------------------------------------------------------------------------
# reductions
# ---------------------------------------------------------------------------

def test_reduction_weight_relations():
    rng = np.random.default_rng(8)
    full = np.ones((6, 9), dtype=bool)
    _, _, wt = orc.sequence_weights(full, "token_mean")
    _, _, ws = orc.sequence_weights(full, "sequence_mean")
    assert np.array_equal(wt, ws)
    lens = rng.integers(1, 10, 6)
    ragged = np.arange(9)[None, :] < lens[:, None]
    L, N, ws = orc.sequence_weights(ragged, "sequence_mean")
    _, _, w0 = orc.sequence_weights(ragged, "length_alpha", alpha=0.0)
    _, _, w1 = orc.sequence_weights(ragged, "length_alpha", alpha=1.0)
    _, _, wh = orc.sequence_weights(ragged, "length_alpha", alpha=0.5)
    _, _, wt = orc.sequence_weights(ragged, "token_mean")
    assert np.array_equal(L, lens) and N == lens.sum()
    assert np.array_equal(w0, ws)
    assert np.all(w1 == 1.0 / 6)
    np.testing.assert_allclose(wh * lens, np.sqrt(lens) / 6, rtol=1e-15)
    assert np.all(wt == 1.0 / lens.sum())
    # total weight per response: token mean L_i / N, sequence mean 1 / B, alpha L^a / B
    np.testing.assert_allclose(wt * lens, lens / lens.sum(), rtol=1e-15)
    np.testing.assert_allclose(ws * lens, 1.0 / 6, rtol=1e-15)
    # empty sequence
    ragged[2] = False
    L, N, wa = orc.sequence_weights(ragged, "length_alpha", alpha=0.5)
    assert wa[2] == 0.0
    L, N, ws = orc.sequence_weights(ragged, "sequence_mean")
    assert ws[2] == 1.0 / 6


def test_per_sequence_then_mean_weights():
    """The live-sequence mean ("GRPO Loss", Normalizer semantics): every
    sequence with an active token carries total weight 1 / B_live, an empty
    one 0; with no empty sequence it equals the sequence mean; the scalar is
    the plain mean over live sequences of each sequence's token mean."""
    rng = np.random.default_rng(21)
    lens = rng.integers(1, 10, 7)
    ragged = np.arange(9)[None, :] < lens[:, None]
    _, _, wl = orc.sequence_weights(ragged, "per_sequence_then_mean")
    _, _, ws = orc.sequence_weights(ragged, "sequence_mean")
    assert np.array_equal(wl, ws)
    ragged[[1, 4]] = False
    L, N, wl = orc.sequence_weights(ragged, "per_sequence_then_mean")
    assert wl[1] == 0.0 and wl[4] == 0.0
    live = L > 0
    np.testing.assert_allclose((wl * L)[live], 1.0 / 5, rtol=1e-15)
    assert abs(float(np.sum(wl * L)) - 1.0) < 1e-15
    # no active token anywhere: every weight is 0
    _, N0, w0 = orc.sequence_weights(np.zeros((3, 4), dtype=bool), "per_sequence_then_mean")
    assert N0 == 0 and np.all(w0 == 0.0)
    # the token loss with these weights is the mean over live sequences of
    # the per-sequence mean token loss (brute force from the token values)
    T = 9
    logp = np.log(rng.uniform(0.05, 1.0, (7, T)))
    old = logp + rng.normal(0, 0.3, (7, T))
    ref = logp + rng.normal(0, 0.3, (7, T))
    r = np.array([1, 0, 1, 1, 0, 0, 1], dtype=np.float64)
    cfg = LossConfig(eps_low=0.2, eps_high=0.2, beta=0.0, reduction="per_sequence_then_mean")
    res = orc.grpo_token_loss(logp, old, ref, ragged, r, groups=dict(group_boundaries=[0, 3, 7]),
                              cfg=cfg)
    per_seq = [np.mean(res.tok["loss"][i][ragged[i]]) for i in range(7) if ragged[i].any()]
    assert abs(res.policy_loss - float(np.mean(per_seq))) < 1e-14


# ---------------------------------------------------------------------------
# closed-form tiny cases (worked out by hand from the definitions)
# ---------------------------------------------------------------------------

def test_closed_form_two_sequence_case():
    """One group of two with rewards (1, 0): mean 1/2, population std 1/2, so
    A = (+1, -1).  T = 1, V = 2, token mean over N = 2, eps = 0.2, beta = 0.04.

    seq 0: x = (ln 3, 0) -> p = (3/4, 1/4); a = 0; old = ln(1/2) -> rho = 3/2,
           above 1 + eps with A > 0: clipped, token loss -1.2, no surrogate
           gradient.  y = (0, 0) -> q_a = 1/2, d = ln(2/3),
           k3 = 2/3 - ln(2/3) - 1.  G = (1/2) * 0.04 * (1 - 2/3) = 0.02/3,
           grad = G * (1 - 3/4, -1/4).
    seq 1: x = (0, 0) -> p = (1/2, 1/2); a = 1; old = ln(1/4) -> rho = 2; A = -1
           so min(-2, -1.2) = -2: token loss 2, unclipped, d loss/d logp =
           -A*rho = 2.  y = (0, ln 3) -> q_a = 3/4, d = ln(3/2),
           k3 = 1/2 - ln(3/2).  G = (1/2) * (2 + 0.04 * (1 - 3/2)) = 0.99,
           grad = 0.99 * (-1/2, 1/2).
    policy_loss = (-1.2 + 2) / 2 = 0.4, kl = (1/6) / 2 = 1/12,
    loss = 0.4 + 0.04 / 12.
    """
    x = np.array([[[math.log(3.0), 0.0]], [[0.0, 0.0]]])
    y = np.array([[[0.0, 0.0]], [[0.0, math.log(3.0)]]])
    ids = np.array([[0], [1]])
    old = np.array([[math.log(0.5)], [math.log(0.25)]])
    mask = np.ones((2, 1), dtype=bool)
    r = np.array([1.0, 0.0])
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2),
                                cfg=LossConfig(eps_low=0.2, eps_high=0.2, beta=0.04))
    assert np.allclose(res.advantages, [1.0, -1.0], rtol=0, atol=1e-15)
    assert res.clipped == 1 and bool(res.tok["clipped"][0, 0]) and not res.tok["clipped"][1, 0]
    assert abs(res.policy_loss - 0.4) < 1e-14
    assert abs(res.kl - 1.0 / 12.0) < 1e-14
    assert abs(res.loss - (0.4 + 0.04 / 12.0)) < 1e-14
    np.testing.assert_allclose(res.seq_kl, [2 / 3 - math.log(2 / 3) - 1, 0.5 - math.log(1.5)], atol=1e-15)
    G0 = 0.02 / 3.0
    np.testing.assert_allclose(res.grad[0, 0], [G0 * 0.25, -G0 * 0.25], rtol=1e-13)
    np.testing.assert_allclose(res.grad[1, 0], [-0.495, 0.495], rtol=1e-13)


def test_closed_form_leave_one_out_asymmetric_clip():
    """Group of three, rewards (1, 0, 0): mean 1/3, var = (4/9 + 1/9 + 1/9)/3 =
    2/9, std = sqrt(2)/3.  Leave-one-out baselines 0, 1/2, 1/2, so
    A = (3/sqrt(2), -3/(2 sqrt(2)), -3/(2 sqrt(2))).
    V = 1 (p = 1, logp = 0 whatever the logit) with T = 2, sequence mean over
    B = 3, beta = 0, eps_low = 0.1, eps_high = 0.3.  old sets rho per token:
      seq 0 (A > 0): rho = 1.25 (inside), rho = 1.5 (clipped at 1.3)
      seq 1 (A < 0): rho = 0.8 (clipped at 0.9, since A < 0 and rho < 0.9)
      seq 2 (A < 0), only one active token: rho = 1.5 (unclipped, -min(1.5A, 1.3A) = -1.5A)
    Token losses: seq 0: -1.25 A0, -1.3 A0; seq 1: -0.9 A1; seq 2: -1.5 A2.
    """
    s2 = math.sqrt(2.0)
    A = [3 / s2, -3 / (2 * s2), -3 / (2 * s2)]
    rhos = np.array([[1.25, 1.5], [0.8, 1.0], [1.5, 1.0]])
    x = np.zeros((3, 2, 1))
    ids = np.zeros((3, 2), dtype=np.int64)
    old = -np.log(rhos)
    mask = np.array([[1, 1], [1, 0], [1, 0]], dtype=bool)
    r = np.array([1.0, 0.0, 0.0])
    cfg = LossConfig(eps_low=0.1, eps_high=0.3, beta=0.0, reduction="sequence_mean")
    res = orc.grpo_loss_fwd_bwd(x, None, ids, old, mask, r,
                                groups=dict(group_boundaries=[0, 3], leave_one_out=True), cfg=cfg)
    np.testing.assert_allclose(res.advantages, A, rtol=1e-15)
    P = [-1.25 * A[0] - 1.3 * A[0], -0.9 * A[1], -1.5 * A[2]]
    np.testing.assert_allclose(res.seq_policy, P, rtol=1e-14)
    assert res.clipped == 2
    w = [1 / 6, 1 / 3, 1 / 3]
    assert abs(res.policy_loss - sum(wi * Pi for wi, Pi in zip(w, P))) < 1e-14
    # V = 1: every gradient is zero (softmax of one logit is constant)
    assert np.all(res.grad == 0.0)
    # d loss / d logp (token level): -A*rho unless clipped
    tl = orc.grpo_token_loss(np.zeros((3, 2)), old, None, mask, r,
                             groups=dict(group_boundaries=[0, 3], leave_one_out=True), cfg=cfg)
    expect = np.array([[w[0] * -A[0] * 1.25, 0.0], [0.0, 0.0], [w[2] * -A[2] * 1.5, 0.0]])
    np.testing.assert_allclose(tl.grad, expect, rtol=1e-14, atol=1e-300)


def test_tie_at_clip_bound_keeps_gradient():
    """At rho exactly 1 + eps (A > 0) the token is not clipped: the inclusive
    clamp passes the gradient and the tie of the minimum sums to -A*rho."""
    hi = 1.25                    # exactly representable; exp(log(1.25)) == 1.25 in binary64
    lp = math.log(hi)
    assert math.exp(lp) == hi
    t = orc.token_terms(np.array([lp]), np.array([0.0]), None, np.array([2.0]),
                        LossConfig(eps_low=0.2, eps_high=0.25, beta=0.0))
    assert not t["clipped"][0]
    assert t["dloss"][0] == -2.0 * hi
    # torch autograd on the same expression gives the same split
    lpt = torch.tensor([lp], dtype=torch.float64, requires_grad=True)
    rho = torch.exp(lpt - 0.0)
    obj = -torch.minimum(rho * 2.0, torch.clamp(rho, 0.8, hi) * 2.0)
    obj.sum().backward()
    assert abs(lpt.grad.item() - t["dloss"][0]) < 1e-15


# ---------------------------------------------------------------------------
# identities
# ---------------------------------------------------------------------------

def test_identity_ref_equals_policy_and_old_equals_logp():
    rng = np.random.default_rng(9)
    x, _, ids, old, mask, r = _rand_case(rng, B=8, T=5, V=7, spp=4)
    g = dict(samples_per_prompt=4)
    first = orc.grpo_loss_fwd_bwd(x, x, ids, old, mask, r, groups=g, cfg=LossConfig())
    old_eq = first.tok["logp"].copy()
    for eps in (0.1, 0.2, 0.45):
        res = orc.grpo_loss_fwd_bwd(x, x, ids, old_eq, mask, r, groups=g,
                                    cfg=LossConfig(eps_low=eps, eps_high=eps))
        assert np.all(res.tok["rho"][mask] == 1.0)
        assert res.kl == 0.0 and np.all(res.seq_kl == 0.0)
        expect = -sum(res.seq_weight[i] * res.seq_tokens[i] * res.advantages[i] for i in range(8))
        assert abs(res.policy_loss - expect) <= 1e-15 * max(1.0, abs(expect))
        # token mean: loss = -masked mean of A
        mm = -np.sum(np.where(mask, res.advantages[:, None], 0.0)) / mask.sum()
        assert abs(res.loss - mm) < 1e-15


def test_gradient_rows_sum_to_zero():
    rng = np.random.default_rng(10)
    x, y, ids, old, mask, r = _rand_case(rng, B=4, T=4, V=33)
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2), cfg=LossConfig())
    s = res.grad.sum(axis=-1)
    assert np.all(np.abs(s) <= 1e-16 * 40 + 1e-15 * np.abs(res.tok["G"]))


def test_masked_slots_never_read():
    rng = np.random.default_rng(11)
    x, y, ids, old, mask, r = _rand_case(rng, B=4, T=6, V=9)
    g = dict(samples_per_prompt=2)
    cfg = LossConfig(beta=0.05)
    a = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=cfg)
    x2, y2, ids2, old2 = x.copy(), y.copy(), ids.copy(), old.copy()
    x2[~mask] = np.nan
    y2[~mask] = np.inf
    ids2[~mask] = -7
    old2[~mask] = -np.inf
    b = orc.grpo_loss_fwd_bwd(x2, y2, ids2, old2, mask, r, groups=g, cfg=cfg)
    assert a.loss == b.loss and a.kl == b.kl and a.policy_loss == b.policy_loss
    assert np.array_equal(a.grad, b.grad)
    # token level too
    ref_lp = a.tok["logp"] + a.tok["d"]
    ta = orc.grpo_token_loss(a.tok["logp"], old, ref_lp, mask, r, groups=g, cfg=cfg)
    lp2 = a.tok["logp"].copy()
    lp2[~mask] = np.nan
    ref2 = ref_lp.copy()
    ref2[~mask] = -np.inf
    tb = orc.grpo_token_loss(lp2, old2, ref2, mask, r, groups=g, cfg=cfg)
    assert ta.policy_loss == tb.policy_loss and ta.kl == tb.kl
    assert np.array_equal(ta.grad, tb.grad)


def test_token_loss_agrees_with_logits_path():
    rng = np.random.default_rng(12)
    x, y, ids, old, mask, r = _rand_case(rng, B=4, T=5, V=11)
    g = dict(samples_per_prompt=2)
    for red, alpha in (("token_mean", None), ("sequence_mean", None), ("length_alpha", 0.5)):
        cfg = LossConfig(eps_low=0.2, eps_high=0.28, beta=0.03, reduction=red, alpha=alpha)
        big = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=cfg)
        lse = scipy.special.logsumexp(x, -1)
        lse_y = scipy.special.logsumexp(y, -1)
        logp = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse
        logq = np.take_along_axis(y, ids[..., None], -1)[..., 0] - lse_y
        tl = orc.grpo_token_loss(logp, old, logq, mask, r, groups=g, cfg=cfg)
        assert abs(big.loss - tl.loss) < 1e-13
        # chain rule: d loss/d x_v = dlogp * (onehot - softmax)
        p = np.exp(x - lse[..., None])
        onehot = np.eye(x.shape[-1])[ids]
        np.testing.assert_allclose(big.grad, tl.grad[..., None] * (onehot - p), atol=1e-15)


# ---------------------------------------------------------------------------
# finite differences and an independent autograd formulation
# ---------------------------------------------------------------------------

def _loss_only(x, y, ids, old, mask, r, g, cfg):
    return orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=cfg, want_grad=False).loss


def _far_from_bounds(res, cfg, mask, margin=1e-3):
    rho = res.tok["rho"][mask]
    return np.all(np.abs(rho - (1 + cfg.eps_high)) > margin) and np.all(np.abs(rho - (1 - cfg.eps_low)) > margin)


@pytest.mark.parametrize("red,alpha,loo,eps_lo,eps_hi,beta", [
    ("token_mean", None, False, 0.2, 0.2, 0.04),
    ("sequence_mean", None, True, 0.2, 0.28, 0.01),
    ("length_alpha", 0.5, True, 0.1, 0.3, 0.2),
    ("length_alpha", 0.3, False, 0.2, 0.2, 0.0),
])
def test_finite_differences(red, alpha, loo, eps_lo, eps_hi, beta):
    rng = np.random.default_rng(13)
    cfg = LossConfig(eps_low=eps_lo, eps_high=eps_hi, beta=beta, reduction=red, alpha=alpha)
    g = dict(group_boundaries=[0, 2, 5], leave_one_out=loo)
    for _ in range(20):
        x, y, ids, old, mask, r = _rand_case(rng, B=5, T=3, V=4, spp=1, old_noise=0.4)
        r[[0, 2]] = 1.0
        r[[1, 3]] = 0.0
        res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=cfg)
        if _far_from_bounds(res, cfg, mask):
            break
    assert res.clipped > 0 or True
    h = 1e-6
    fd = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        xp = x.copy()
        xp[idx] += h
        xm = x.copy()
        xm[idx] -= h
        fd[idx] = (_loss_only(xp, y, ids, old, mask, r, g, cfg) - _loss_only(xm, y, ids, old, mask, r, g, cfg)) / (2 * h)
    np.testing.assert_allclose(res.grad, fd, atol=2e-9)
    # token-level dlogp by finite differences on logp
    lse = scipy.special.logsumexp(x, -1)
    lse_y = scipy.special.logsumexp(y, -1)
    logp = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse
    logq = np.take_along_axis(y, ids[..., None], -1)[..., 0] - lse_y
    tl = orc.grpo_token_loss(logp, old, logq, mask, r, groups=g, cfg=cfg)
    fd2 = np.zeros_like(logp)
    for idx in np.ndindex(*logp.shape):
        lp, lm = logp.copy(), logp.copy()
        lp[idx] += h
        lm[idx] -= h
        fp_ = orc.grpo_token_loss(lp, old, logq, mask, r, groups=g, cfg=cfg).loss
        fm_ = orc.grpo_token_loss(lm, old, logq, mask, r, groups=g, cfg=cfg).loss
        fd2[idx] = (fp_ - fm_) / (2 * h)
    np.testing.assert_allclose(tl.grad, fd2, atol=2e-9)


def test_clipped_tokens_carry_only_the_kl_gradient():
    rng = np.random.default_rng(14)
    x, y, ids, _, mask, r = _rand_case(rng, B=2, T=2, V=6, ragged=False)
    r[:] = [1.0, 0.0]   # A = (+1, -1)
    lse = scipy.special.logsumexp(x, -1)
    logp = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse
    # seq 0 (A > 0): rho = 2 (clipped above); seq 1 (A < 0): rho = 0.5 (clipped below)
    old = logp - np.log(np.array([[2.0, 2.0], [0.5, 0.5]]))
    g = dict(samples_per_prompt=2)
    res0 = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=LossConfig(beta=0.0))
    assert res0.clipped == 4 and np.all(res0.grad == 0.0)
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=LossConfig(beta=0.3))
    expect_G = res.seq_weight[:, None] * 0.3 * (-np.expm1(res.tok["d"]))
    np.testing.assert_allclose(res.tok["G"], expect_G, rtol=1e-14)
    h = 1e-6
    for idx in [(0, 0, 1), (1, 1, 3), (0, 1, int(ids[0, 1]))]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd = (_loss_only(xp, y, ids, old, mask, r, g, LossConfig(beta=0.3)) -
              _loss_only(xm, y, ids, old, mask, r, g, LossConfig(beta=0.3))) / (2 * h)
        assert abs(fd - res.grad[idx]) < 1e-9


def _torch_objective(x, y, ids, old, mask, r, offsets, cfg, loo, scale_std, std_eps=1e-6):
    """Independent formulation with torch autograd (fp64, CPU)."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y, dtype=torch.float64)
    idt = torch.tensor(ids, dtype=torch.int64)[..., None]
    mt = torch.tensor(mask, dtype=torch.bool)
    oldt = torch.tensor(old, dtype=torch.float64)
    rt = torch.tensor(r, dtype=torch.float64)
    B = rt.shape[0]
    adv = torch.zeros(B, dtype=torch.float64)
    for s, e in zip(offsets[:-1], offsets[1:]):
        grp = rt[s:e]
        n = e - s
        sd = torch.sqrt(torch.mean((grp - grp.mean()) ** 2))
        base = (grp.sum() - grp) / (n - 1) if loo else grp.mean()
        a = grp - base
        adv[s:e] = a / torch.clamp(sd, min=std_eps) if scale_std else a
    logp = torch.gather(xt, -1, idt)[..., 0] - torch.logsumexp(xt, -1)
    logq = torch.gather(yt, -1, idt)[..., 0] - torch.logsumexp(yt, -1)
    ratio = torch.exp(logp - oldt)
    A = adv[:, None].expand_as(ratio)
    per_tok = -torch.minimum(ratio * A, torch.clamp(ratio, 1 - cfg.eps_low, 1 + cfg.eps_high) * A)
    dd = logq - logp
    kl = torch.exp(dd) - dd - 1
    L = mt.sum(1).to(torch.float64)
    if cfg.reduction == "token_mean":
        w = torch.full((B,), 1.0 / max(float(L.sum()), 1.0), dtype=torch.float64)
    elif cfg.reduction == "sequence_mean":
        w = 1.0 / (B * torch.clamp(L, min=1.0))
    elif cfg.reduction == "per_sequence_then_mean":
        n_live = float((L > 0).sum())
        w = torch.where(L > 0, 1.0 / (max(n_live, 1.0) * torch.clamp(L, min=1.0)), torch.zeros_like(L))
    else:
        w = torch.where(L > 0, L ** cfg.alpha / (B * torch.clamp(L, min=1.0)), torch.zeros_like(L))
    zero = torch.zeros_like(per_tok)
    pol = (w[:, None] * torch.where(mt, per_tok, zero)).sum()
    klv = (w[:, None] * torch.where(mt, kl, zero)).sum()
    total = pol + cfg.beta * klv
    total.backward()
    return total.item(), pol.item(), klv.item(), xt.grad.numpy()


@pytest.mark.parametrize("seed", range(8))
def test_against_independent_autograd(seed):
    rng = np.random.default_rng(100 + seed)
    red, alpha = [("token_mean", None), ("sequence_mean", None), ("length_alpha", 0.5),
                  ("per_sequence_then_mean", None)][seed % 4]
    loo = bool(seed % 2)
    cfg = LossConfig(eps_low=0.2, eps_high=0.28 if seed % 2 else 0.2, beta=0.04, reduction=red, alpha=alpha)
    sizes = [2, 4, 2] if seed < 3 else [4, 4]
    offsets = list(np.concatenate([[0], np.cumsum(sizes)]))
    B = offsets[-1]
    x, y, ids, old, mask, r = _rand_case(rng, B=B, T=6, V=13, spp=2, scale=2.0, old_noise=0.3)
    if red == "per_sequence_then_mean":
        mask[1] = False   # an empty sequence: the live count differs from B
    g = dict(group_boundaries=offsets, leave_one_out=loo)
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=g, cfg=cfg)
    tot, pol, klv, grad = _torch_objective(x, y, ids, old, mask, r, offsets, cfg, loo, True)
    assert abs(res.loss - tot) < 1e-13
    assert abs(res.policy_loss - pol) < 1e-13
    assert abs(res.kl - klv) < 1e-13
    np.testing.assert_allclose(res.grad, grad, atol=1e-15, rtol=1e-11)
