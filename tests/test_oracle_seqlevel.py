"""Pins for the oracle's sequence-level objectives: the GSPO sequence ratio
(Relax REINFORCE++ page, Formula-level comparison; dockyard_rl, One loss many
algorithms), the REAL loss (ms-swift REAL blog: REAL formalisation, source
walkthrough) and sequence-masked truncated importance sampling (dockyard_rl,
Off-policy correction (async GRPO)).

Each is checked against something other than the oracle: torch autograd of
independent formulations (the REAL one follows the blog's log-sum-exp with an
appended zero and -inf masking rather than the oracle's loops), central
finite differences, closed forms, the gradient bound the blog states, and
reductions to the token-level objectives where the definitions coincide."""

import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle as orc
from oracle import LossConfig, OracleInputError


def _case(rng, B=6, T=5, V=7, ratio_noise=0.4, seq_shift=0.3, spp=3):
    x = rng.normal(0, 1.5, (B, T, V))
    y = x + rng.normal(0, 0.5, (B, T, V))
    ids = rng.integers(0, V, (B, T))
    lse = scipy.special.logsumexp(x, axis=-1)
    logp = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse
    # a per-sequence shift moves whole sequences across the clip band
    old = logp + rng.normal(0, ratio_noise, (B, T)) + rng.uniform(-seq_shift, seq_shift, (B, 1))
    lens = rng.integers(1, T + 1, B)
    mask = np.arange(T)[None, :] < lens[:, None]
    r = rng.integers(0, 2, B).astype(np.float64)
    r[:spp] = [1.0, 0.0, 1.0][:spp]          # group 0 has both labels
    return x, y, ids, old, mask, r


def _weights_t(mt, cfg):
    L = mt.sum(1).double()
    B = mt.shape[0]
    if cfg.reduction == "token_mean":
        return torch.full((B,), 1.0 / float(max(L.sum(), 1)), dtype=torch.float64)
    if cfg.reduction == "sequence_mean":
        return 1.0 / (B * L.clamp_min(1))
    if cfg.reduction == "fixed_constant":
        return torch.full((B,), 1.0 / cfg.norm_constant, dtype=torch.float64)
    return torch.where(L > 0, L ** cfg.alpha / (B * L.clamp_min(1)), torch.zeros_like(L))


def _adv_t(r, spp):
    rt = torch.tensor(r, dtype=torch.float64).view(-1, spp)
    return ((rt - rt.mean(1, keepdim=True)) /
            rt.std(1, keepdim=True, unbiased=False).clamp_min(1e-6)).reshape(-1)


def _kl_t(lr, cfg):
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
    return kl


def _torch_gspo(x, y, ids, old, mask, r, spp, cfg, gen=None):
    """GSPO with torch autograd: the masked-mean log-ratio per sequence, the
    clipped surrogate on its exponential, expanded to the sequence's tokens."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    idt = torch.tensor(ids)[..., None]
    mt = torch.tensor(mask)
    oldt = torch.tensor(old, dtype=torch.float64)
    A = _adv_t(r, spp)
    logp = torch.log_softmax(xt, -1).gather(-1, idt)[..., 0]
    logq = torch.log_softmax(torch.tensor(y, dtype=torch.float64), -1).gather(-1, idt)[..., 0]
    z = torch.zeros_like(logp)
    L = mt.sum(1).double()
    s = torch.where(mt, logp - oldt, z).sum(1) / L.clamp_min(1)
    rho = torch.exp(s)
    lo, hi = 1 - cfg.eps_low, 1 + cfg.eps_high
    pg_seq = -torch.minimum(rho * A, rho.clamp(lo, hi) * A)
    pg = pg_seq[:, None].expand_as(logp)
    if gen is not None:
        wis = torch.exp(oldt - torch.tensor(gen, dtype=torch.float64))
        if cfg.tis_type is not None:
            wis = wis.clamp(cfg.tis_ratio_min or 0.0, cfg.tis_ratio_max)
        pg = pg * wis
    kl = _kl_t(logq - logp, cfg)
    w = _weights_t(mt, cfg)
    pol = (w[:, None] * torch.where(mt, pg, z)).sum()
    klv = (w[:, None] * torch.where(mt, kl, z)).sum()
    tot = pol + cfg.beta * klv
    tot.backward()
    return tot.item(), pol.item(), klv.item(), xt.grad.numpy(), s.detach().numpy()


def _torch_real(x, y, ids, old, mask, r, spp, cfg):
    """REAL as the blog's source walkthrough lays it out: masked-mean scores
    and advantages per sequence, a view into groups, positive/negative masks
    by sign, -inf filling and a log-sum-exp over the scores with a zero
    column appended, summed over valid groups and divided by the number of
    groups; the KL term as a masked token mean."""
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    idt = torch.tensor(ids)[..., None]
    mt = torch.tensor(mask)
    md = mt.double()
    oldt = torch.tensor(old, dtype=torch.float64)
    logp = torch.log_softmax(xt, -1).gather(-1, idt)[..., 0]
    logq = torch.log_softmax(torch.tensor(y, dtype=torch.float64), -1).gather(-1, idt)[..., 0]
    tau = cfg.real_tau
    scores = ((logp - oldt) * md).sum(-1) / md.sum(-1).clamp(min=1.0)
    adv_tok = _adv_t(r, spp)[:, None].expand_as(logp)
    seq_adv = (adv_tok * md).sum(-1) / md.sum(-1).clamp(min=1.0)
    gs = scores.view(-1, spp)
    ga = seq_adv.view(-1, spp)
    pos = ga > 0
    neg = ga < 0
    valid = (pos.sum(1) != 0) & (neg.sum(1) != 0)
    zero = torch.zeros(int(valid.sum()), 1, dtype=torch.float64)
    sc = gs[valid] / tau
    neg_in = sc.masked_fill(~neg[valid], float("-inf"))
    pos_in = (-sc).masked_fill(~pos[valid], float("-inf"))
    neg_loss = torch.logsumexp(torch.cat([neg_in, zero], 1), 1)
    pos_loss = torch.logsumexp(torch.cat([pos_in, zero], 1), 1)
    pol = (neg_loss + pos_loss).sum() / ga.size(0)
    kl = _kl_t(logq - logp, cfg)
    klv = (kl * md).sum() / md.sum().clamp(min=1.0)
    tot = pol + cfg.beta * klv
    tot.backward()
    return tot.item(), pol.item(), klv.item(), xt.grad.numpy(), scores.detach().numpy()


GSPO_CASES = [
    dict(reduction="sequence_mean"),
    dict(reduction="sequence_mean", eps_low=0.2, eps_high=0.28, kl_estimator="k2"),
    dict(reduction="length_alpha", alpha=0.5),
    dict(reduction="fixed_constant", norm_constant=23.0, kl_estimator="k1"),
    dict(reduction="sequence_mean", tis_type="tis", tis_ratio_max=1.3),
    dict(reduction="sequence_mean", tis_type="icepop", tis_ratio_min=0.7, tis_ratio_max=1.4,
         kl_input_clamp=0.3),
    dict(reduction="sequence_mean", is_only=True),
]


@pytest.mark.parametrize("kw", GSPO_CASES, ids=lambda d: "-".join(f"{k}={v}" for k, v in d.items()))
def test_gspo_against_independent_autograd(kw):
    kw = dict(kw)
    use_gen = kw.pop("is_only", False) or "tis_type" in kw
    cfg = LossConfig(beta=0.3, pg_loss="gspo", **kw)
    n_clipped = 0
    for seed in range(4):
        rng = np.random.default_rng(2000 + seed)
        x, y, ids, old, mask, r = _case(rng)
        gen = old + rng.normal(0, 0.4, old.shape) if use_gen else None
        res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3),
                                    cfg=cfg, gen_logps=gen)
        tot, pol, klv, grad, s = _torch_gspo(x, y, ids, old, mask, r, 3, cfg, gen)
        assert abs(res.loss - tot) < 1e-12 * max(1, abs(tot))
        assert abs(res.policy_loss - pol) < 1e-12 * max(1, abs(pol))
        assert abs(res.kl - klv) < 1e-12 * max(1, abs(klv))
        np.testing.assert_allclose(res.seq_logratio, s, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(res.grad, grad, atol=1e-14, rtol=1e-10)
        n_clipped += res.clipped
    assert n_clipped > 0          # the cases do cross the clip band


def test_gspo_single_token_sequences_equal_token_clip():
    """With one active token per sequence the sequence ratio is the token
    ratio, so GSPO and the token-level clipped surrogate coincide."""
    rng = np.random.default_rng(7)
    x, y, ids, old, _, r = _case(rng, T=1, ratio_noise=0.5)
    mask = np.ones((6, 1), dtype=bool)
    for red in ("sequence_mean", "length_alpha"):
        g = LossConfig(beta=0.2, pg_loss="gspo", reduction=red, alpha=0.5, eps_high=0.28)
        t = LossConfig(beta=0.2, pg_loss="clip", reduction=red, alpha=0.5, eps_high=0.28)
        a = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=g)
        b = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=t)
        assert a.loss == pytest.approx(b.loss, rel=1e-14, abs=1e-16)
        assert a.clipped == b.clipped
        np.testing.assert_allclose(a.grad, b.grad, rtol=1e-12, atol=1e-16)


def test_gspo_uniform_log_ratio_equals_token_clip():
    """When every token of a sequence has the same log-ratio, each token's
    ratio equals the sequence ratio: the loss and the gradient of GSPO equal
    the token-level clipped surrogate's (w_i * L_i/L_i * dl/ds = w_i * dl/dlogp)."""
    rng = np.random.default_rng(11)
    x, y, ids, _, mask, r = _case(rng)
    lse = scipy.special.logsumexp(x, axis=-1)
    logp = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse
    shift = rng.uniform(-0.5, 0.5, (6, 1))
    old = logp - shift                                 # log-ratio = shift for every token
    g = LossConfig(beta=0.1, pg_loss="gspo", reduction="sequence_mean")
    t = LossConfig(beta=0.1, pg_loss="clip", reduction="sequence_mean")
    a = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=g)
    b = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=t)
    assert a.clipped == b.clipped and a.clipped > 0
    assert a.loss == pytest.approx(b.loss, rel=1e-12)
    np.testing.assert_allclose(a.grad, b.grad, rtol=1e-9, atol=1e-15)


def _fd_check(cfg, seed, gen_noise=None, h=1e-6):
    rng = np.random.default_rng(seed)
    x, y, ids, old, mask, r = _case(rng, B=6, T=3, V=4)
    gen = None if gen_noise is None else old + rng.normal(0, gen_noise, old.shape)
    kw = dict(groups=dict(samples_per_prompt=3), cfg=cfg, gen_logps=gen)
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, **kw)
    checked = 0
    for idx in np.ndindex(*x.shape):
        xp = x.copy()
        xm = x.copy()
        xp[idx] += h
        xm[idx] -= h
        lp = orc.grpo_loss_fwd_bwd(xp, y, ids, old, mask, r, want_grad=False, **kw)
        lm = orc.grpo_loss_fwd_bwd(xm, y, ids, old, mask, r, want_grad=False, **kw)
        if lp.clipped != res.clipped or lm.clipped != res.clipped:
            continue                   # a clip decision flips inside the step
        fd = (lp.loss - lm.loss) / (2 * h)
        assert fd == pytest.approx(res.grad[idx], rel=1e-5, abs=1e-8), idx
        checked += 1
    assert checked > x.size // 2


@pytest.mark.parametrize("kw", [
    dict(pg_loss="gspo", reduction="sequence_mean"),
    dict(pg_loss="gspo", reduction="length_alpha", alpha=0.5, eps_low=0.1, eps_high=0.3),
    dict(pg_loss="real"),
    dict(pg_loss="real", real_tau=0.2, kl_estimator="k2"),
])
def test_sequence_level_finite_differences(kw):
    cfg = LossConfig(beta=0.25, **kw)
    _fd_check(cfg, 3100)


def test_gspo_finite_differences_with_is_weights():
    cfg = LossConfig(beta=0.25, pg_loss="gspo", reduction="sequence_mean", tis_type="tis",
                     tis_ratio_max=1.2)
    _fd_check(cfg, 3200, gen_noise=0.3)


def test_gspo_clipped_sequences_carry_only_the_kl_gradient():
    rng = np.random.default_rng(5)
    x, y, ids, old, mask, r = _case(rng, seq_shift=0.8)
    cfg = LossConfig(beta=0.3, pg_loss="gspo", reduction="sequence_mean")
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=cfg)
    # with all advantages zero only the KL part of the gradient is left
    nopol = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, np.zeros(6), groups=dict(samples_per_prompt=3),
                                  cfg=cfg)
    rho = np.exp(res.seq_logratio)
    A = res.advantages
    clipped = ((A > 0) & (rho > 1.2)) | ((A < 0) & (rho < 0.8))
    assert clipped.any() and not clipped.all()
    assert res.clipped == int(res.seq_tokens[clipped].sum())
    np.testing.assert_array_equal(res.grad[clipped], nopol.grad[clipped])
    assert np.any(res.grad[~clipped] != nopol.grad[~clipped])
    # with the band wide open nothing is clipped
    wide = LossConfig(beta=0.3, pg_loss="gspo", reduction="sequence_mean", eps_low=0.999,
                      eps_high=1e9)
    assert orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3),
                                 cfg=wide).clipped == 0


REAL_CASES = [
    dict(),
    dict(real_tau=0.2),
    dict(real_tau=1.5, kl_estimator="k1"),
    dict(kl_output_clamp=0.05),
]


@pytest.mark.parametrize("kw", REAL_CASES, ids=lambda d: "-".join(f"{k}={v}" for k, v in d.items()) or "default")
def test_real_against_independent_autograd(kw):
    cfg = LossConfig(beta=0.3, pg_loss="real", **kw)
    for seed in range(4):
        rng = np.random.default_rng(4000 + seed)
        x, y, ids, old, mask, r = _case(rng)
        res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=cfg)
        tot, pol, klv, grad, s = _torch_real(x, y, ids, old, mask, r, 3, cfg)
        assert abs(res.loss - tot) < 1e-12 * max(1, abs(tot))
        assert abs(res.policy_loss - pol) < 1e-12 * max(1, abs(pol))
        assert abs(res.kl - klv) < 1e-12 * max(1, abs(klv))
        np.testing.assert_allclose(res.seq_logratio, s, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(res.grad, grad, atol=1e-14, rtol=1e-10)


def test_real_two_member_group_closed_form():
    """One positive and one negative sequence: loss = softplus(-s1/tau) +
    softplus(s2/tau) over G = 1 group; the positive member's weight is
    -sigmoid(-s1/tau)/tau."""
    tau = 0.5
    s = np.array([0.3, -0.7])
    A = np.array([1.0, -1.0])
    gl, dpol, pol = orc.real_terms(s, A, np.array([4, 2]), np.array([0, 2]), tau)
    sp = lambda v: math.log1p(math.exp(v))
    assert pol == pytest.approx(sp(-0.3 / tau) + sp(-0.7 / tau), rel=1e-15)
    assert dpol[0] == pytest.approx(-(1 / tau) * scipy.special.expit(-0.3 / tau), rel=1e-14)
    assert dpol[1] == pytest.approx((1 / tau) * scipy.special.expit(-0.7 / tau), rel=1e-14)


def test_real_weight_bounded_and_monotone():
    """The blog states the gradient weight is bounded by 1/tau in magnitude and
    grows for a positive sample as its score falls."""
    rng = np.random.default_rng(9)
    tau = 0.5
    for _ in range(20):
        n = 8
        s = rng.normal(0, 3, n)
        A = np.where(rng.integers(0, 2, n) > 0, 1.0, -1.0)
        A[0], A[1] = 1.0, -1.0
        _, dpol, _ = orc.real_terms(s, A, np.full(n, 3), np.array([0, n]), tau)
        assert np.all(np.abs(dpol) <= 1.0 / tau + 1e-15)
        s2 = s.copy()
        s2[0] -= 0.5                                   # the positive sample looks less likely
        _, dpol2, _ = orc.real_terms(s2, A, np.full(n, 3), np.array([0, n]), tau)
        assert abs(dpol2[0]) > abs(dpol[0])


def test_real_single_label_groups_and_empty_sequences_contribute_nothing():
    s = np.array([0.1, -0.2, 0.3, 0.4, 0.5, -0.6])
    A = np.array([1.0, 1.0, 0.0, 0.5, -0.5, 0.2])
    L = np.array([3, 3, 3, 2, 0, 5])          # sequence 4 has no active token
    gl, dpol, pol = orc.real_terms(s, A, L, np.array([0, 3, 6]), 0.5)
    # group 0: no negative -> invalid; group 1: the only negative is empty -> invalid
    assert gl[0] == 0.0 and gl[1] == 0.0 and pol == 0.0
    assert np.all(dpol == 0.0)
    # an empty positive sequence is not a label: only members 2 (pos) and 1 (neg) count
    s2 = np.array([0.9, -0.2, 0.3])
    gl2, dpol2, pol2 = orc.real_terms(s2, np.array([1.0, -1.0, 1.0]), np.array([0, 3, 2]),
                                      np.array([0, 3]), 0.5)
    sp = lambda v: math.log1p(math.exp(v))
    assert pol2 == pytest.approx(sp(-0.3 / 0.5) + sp(-0.2 / 0.5), rel=1e-15)
    assert dpol2[0] == 0.0


def test_real_degenerate_batch_leaves_only_kl():
    rng = np.random.default_rng(13)
    x, y, ids, old, mask, _ = _case(rng)
    r = np.ones(6)
    cfg = LossConfig(beta=0.3, pg_loss="real")
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=cfg)
    assert res.policy_loss == 0.0
    assert res.loss == pytest.approx(0.3 * res.kl, rel=1e-15)
    assert np.all(res.tok["loss"] == 0.0)


def test_seq_mask_keep_closed_form_and_limits():
    rng = np.random.default_rng(17)
    x, y, ids, old, mask, r = _case(rng)
    gen = old + rng.normal(0, 0.5, old.shape) + rng.uniform(-0.4, 0.4, (6, 1))
    lo, hi = 0.8, 1.25
    cfg = LossConfig(beta=0.2, tis_type="seq_mask", tis_ratio_min=lo, tis_ratio_max=hi)
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=cfg,
                                gen_logps=gen)
    # keep flags straight from the definition: geometric mean of the token weights
    for i in range(6):
        m = mask[i]
        ratio = float(np.prod(np.exp(old[i, m] - gen[i, m])) ** (1.0 / m.sum()))
        assert res.seq_keep[i] == (lo <= ratio <= hi)
    assert res.seq_keep.any() and not res.seq_keep.all()
    # wide bounds keep everything: identical to the untruncated weight
    wide = LossConfig(beta=0.2, tis_type="seq_mask", tis_ratio_min=0.0, tis_ratio_max=1e9)
    plain = LossConfig(beta=0.2)
    a = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=wide,
                              gen_logps=gen)
    b = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=plain,
                              gen_logps=gen)
    assert a.loss == b.loss
    np.testing.assert_array_equal(a.grad, b.grad)
    # empty bounds mask every sequence: no policy term, gradient of the KL alone
    none = LossConfig(beta=0.2, tis_type="seq_mask", tis_ratio_min=1e6, tis_ratio_max=1e9)
    c = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=none,
                              gen_logps=gen)
    assert c.policy_loss == 0.0
    d = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, np.zeros(6), groups=dict(samples_per_prompt=3),
                              cfg=plain, gen_logps=gen)
    np.testing.assert_array_equal(c.grad, d.grad)


def test_seq_mask_against_independent_autograd():
    rng = np.random.default_rng(19)
    x, y, ids, old, mask, r = _case(rng)
    gen = old + rng.normal(0, 0.5, old.shape) + rng.uniform(-0.4, 0.4, (6, 1))
    lo, hi = 0.8, 1.25
    cfg = LossConfig(beta=0.2, tis_type="seq_mask", tis_ratio_min=lo, tis_ratio_max=hi,
                     reduction="sequence_mean")
    res = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=cfg,
                                gen_logps=gen)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    idt = torch.tensor(ids)[..., None]
    mt = torch.tensor(mask)
    md = mt.double()
    oldt = torch.tensor(old, dtype=torch.float64)
    gent = torch.tensor(gen, dtype=torch.float64)
    A = _adv_t(r, 3)[:, None]
    logp = torch.log_softmax(xt, -1).gather(-1, idt)[..., 0]
    logq = torch.log_softmax(torch.tensor(y, dtype=torch.float64), -1).gather(-1, idt)[..., 0]
    seq_ratio = torch.exp(((oldt - gent) * md).sum(1) / md.sum(1))
    keep = ((seq_ratio >= lo) & (seq_ratio <= hi)).double()[:, None]
    wis = torch.exp(oldt - gent) * keep
    ratio = torch.exp(logp - oldt)
    pg = -torch.minimum(ratio * A, ratio.clamp(0.8, 1.2) * A) * wis
    kl = torch.exp(logq - logp) - (logq - logp) - 1
    w = 1.0 / (6 * md.sum(1))
    tot = (w[:, None] * (pg + 0.2 * kl) * md).sum()
    tot.backward()
    assert res.loss == pytest.approx(tot.item(), rel=1e-12)
    np.testing.assert_allclose(res.grad, xt.grad.numpy(), rtol=1e-10, atol=1e-14)


def test_token_path_equals_logits_path_for_sequence_losses():
    """grpo_token_loss on the log-probs of the logits gives the logits path's
    loss, and its dlogp is the G that the logits path spreads over the row."""
    rng = np.random.default_rng(23)
    x, y, ids, old, mask, r = _case(rng)
    lse = scipy.special.logsumexp(x, axis=-1)
    lp = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse
    lq = np.take_along_axis(y, ids[..., None], -1)[..., 0] - scipy.special.logsumexp(y, axis=-1)
    for cfg in (LossConfig(beta=0.2, pg_loss="gspo", reduction="sequence_mean"),
                LossConfig(beta=0.2, pg_loss="real")):
        a = orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3), cfg=cfg)
        b = orc.grpo_token_loss(lp, old, lq, mask, r, groups=dict(samples_per_prompt=3), cfg=cfg)
        assert b.loss == pytest.approx(a.loss, rel=1e-12)
        np.testing.assert_allclose(b.seq_logratio, a.seq_logratio, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(b.grad, a.tok["G"], rtol=1e-10, atol=1e-15)


@pytest.mark.parametrize("kw,gen", [
    (dict(pg_loss="gspo"), False),                                       # token mean
    (dict(pg_loss="real", reduction="sequence_mean"), False),
    (dict(pg_loss="real"), True),                                         # no off-policy weights
    (dict(pg_loss="real", real_tau=0.0), False),
    (dict(pg_loss="gspo", reduction="sequence_mean", dual_clip_c=2.0), False),
    (dict(tis_type="seq_mask", tis_ratio_max=2.0), True),                 # needs a lower bound
    (dict(pg_loss="gspo", reduction="sequence_mean", tis_type="seq_mask", tis_ratio_min=0.5,
          tis_ratio_max=2.0), True),
    (dict(tis_type="seq_mask", tis_ratio_min=0.5, tis_ratio_max=2.0), False),  # needs gen
])
def test_sequence_level_invalid_combinations(kw, gen):
    rng = np.random.default_rng(29)
    x, y, ids, old, mask, r = _case(rng)
    with pytest.raises(OracleInputError):
        orc.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=3),
                              cfg=LossConfig(**kw), gen_logps=old + 0.1 if gen else None)
