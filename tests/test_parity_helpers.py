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
    dict(tis_type="seq_mask", tis_ratio_min=0.8, tis_ratio_max=1.25),
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


# --- sequence-level losses ----------------------------------------------------

SEQ_VARIANTS = [
    dict(pg_loss="gspo", reduction="sequence_mean"),
    dict(pg_loss="gspo", reduction="length_alpha", alpha=0.5, kl_estimator="k2"),
    dict(pg_loss="gspo", reduction="sequence_mean", tis_type="tis", tis_ratio_max=1.3),
    dict(pg_loss="real"),
    dict(pg_loss="real", real_tau=0.2, kl_input_clamp=0.2),
]


def _seq_case(seed, shift=0.4):
    x, y, ids, old, mask, r = _case(seed, old_std=0.3)
    old = old + np.random.default_rng(seed + 100).uniform(-shift, shift, (old.shape[0], 1))
    return x, y, ids, old, mask, r


def _seq_as_result(ref, grad_dtype=torch.float32):
    res = _as_result(ref, grad_dtype)
    res.seq_logratio = torch.tensor(ref.seq_logratio, dtype=torch.float32)
    return res


def _seq_run(kw, seed):
    from _parity import compare_seq_outputs, seq_branches  # noqa: F401
    cfg = oracle.LossConfig(beta=0.1, **kw)
    x, y, ids, old, mask, r = _seq_case(seed)
    gen = old + np.random.default_rng(seed + 9).normal(0, 0.4, old.shape) if "tis_type" in kw else None
    groups = dict(samples_per_prompt=2)
    ref = oracle.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=groups, cfg=cfg, gen_logps=gen)
    h = dict(old_logps=old, gen_logps=gen)
    return cfg, x, ids, mask, ref, h, groups


@pytest.mark.parametrize("kw", SEQ_VARIANTS, ids=str)
def test_seq_helpers_accept_rounded_oracle(kw):
    from _parity import GRAD16_BAR, compare_seq_outputs, seq_branches
    cfg, x, ids, mask, ref, h, groups = _seq_run(kw, 11)
    if kw["pg_loss"] == "gspo":
        assert ref.clipped > 0
    for dt, gdt in ((torch.float32, "f32"), (torch.bfloat16, "bf16"), (torch.float16, "f16")):
        res = _seq_as_result(ref, dt)
        compare_seq_outputs(res, ref, cfg, mask, h, groups, 1e-5)
        base = GRAD16_BAR.get(gdt, (1e-5, 0))[0]
        br = seq_branches(ref, cfg, mask, h, groups, base)
        compare_logits_grad(res.grad.double().numpy(), ref, cfg, mask, gdt, branches=br)


@pytest.mark.parametrize("kw", [SEQ_VARIANTS[0], SEQ_VARIANTS[3]], ids=str)
def test_seq_helpers_reject_planted_mistakes(kw):
    from _parity import compare_seq_outputs, seq_branches
    cfg, x, ids, mask, ref, h, groups = _seq_run(kw, 12)
    res = _seq_as_result(ref)
    res.loss = torch.tensor(ref.loss * (1 + 1e-3) + 1e-6, dtype=torch.float32)
    with pytest.raises(AssertionError):
        compare_seq_outputs(res, ref, cfg, mask, h, groups, 1e-5)
    res = _seq_as_result(ref)
    res.seq_logratio = res.seq_logratio + 1e-4
    with pytest.raises(AssertionError):
        compare_seq_outputs(res, ref, cfg, mask, h, groups, 1e-5)
    res = _seq_as_result(ref)
    res.policy_loss = torch.tensor(ref.policy_loss * 1.01 + 1e-6, dtype=torch.float32)
    with pytest.raises(AssertionError):
        compare_seq_outputs(res, ref, cfg, mask, h, groups, 1e-5)
    # one gradient row off by 5 %
    i, t = [int(v[0]) for v in np.nonzero(mask & (np.abs(ref.tok["G"]) > 1e-3))]
    g = ref.grad.copy()
    g[i, t] *= 1.05
    br = seq_branches(ref, cfg, mask, h, groups, 2.0 ** -7)
    with pytest.raises(AssertionError):
        compare_logits_grad(g, ref, cfg, mask, "bf16", branches=br)


def test_seq_branch_flip_rejected_away_from_bounds_accepted_at_a_bound():
    from _parity import SEQ_ABS_ERR, seq_branches
    kw = dict(pg_loss="gspo", reduction="sequence_mean")
    cfg = oracle.LossConfig(beta=0.0, **kw)
    x, _, ids, _, mask, _ = _seq_case(13)
    groups = dict(samples_per_prompt=2)
    r = np.tile([0.0, 1.0], 4)
    lse = scipy.special.logsumexp(x, axis=-1)
    logp = np.take_along_axis(x, ids[..., None], -1)[..., 0] - lse
    A = oracle.group_advantages(r, oracle.group_offsets(8, 2))
    k = int(np.nonzero(A > 0)[0][0])

    def run(shift_k):
        old = logp.copy()
        old[k] = logp[k] - shift_k               # sequence k's log-ratio is shift_k exactly
        ref = oracle.grpo_loss_fwd_bwd(x, None, ids, old, mask, r, groups=groups, cfg=cfg)
        return ref, dict(old_logps=old, gen_logps=None)

    def unclipped_rows(ref, g):
        rho = np.exp(ref.seq_logratio[k])
        for t in np.nonzero(mask[k])[0]:
            p = scipy.special.softmax(x[k, t])
            onehot = np.zeros_like(p)
            onehot[ids[k, t]] = 1.0
            g[k, t] = -ref.seq_weight[k] * A[k] * rho * (onehot - p)
        return g

    # far above the band (rho = e^0.5): flipping the sequence to unclipped is caught
    ref, h = run(0.5)
    assert ref.clipped == ref.seq_tokens[k]
    br = seq_branches(ref, cfg, mask, h, groups, 1e-5)
    with pytest.raises(AssertionError):
        compare_logits_grad(unclipped_rows(ref, ref.grad.copy()), ref, cfg, mask, "f32", policy=x,
                            ids=ids, branches=br)
    # a hair above the upper bound: either branch is right
    ref2, h2 = run(np.log(1.2) + SEQ_ABS_ERR / 4)
    assert ref2.clipped == ref2.seq_tokens[k]
    br2 = seq_branches(ref2, cfg, mask, h2, groups, 1e-5)
    assert br2[0][k][mask[k]].all()
    stats = compare_logits_grad(unclipped_rows(ref2, ref2.grad.copy()), ref2, cfg, mask, "f32",
                                policy=x, ids=ids, branches=br2)
    assert stats["ambiguous"] >= 1


def _bf16_case(seed=5):
    """A small bf16 batch in the shape of the full-size inputs (torch tensors)."""
    x, y, ids, old, mask, r = _case(seed, B=8, T=10, V=300)
    t = dict(policy=torch.tensor(x, dtype=torch.bfloat16), ref=torch.tensor(y, dtype=torch.bfloat16),
             action_ids=torch.tensor(ids), old_logps=torch.tensor(old, dtype=torch.float32),
             mask=torch.tensor(mask), rewards=torch.tensor(r, dtype=torch.float32))
    return t


def test_stream_oracle_accepts_rounded_oracle_and_rejects_a_bad_row():
    """The whole-batch streaming comparison (tests/_fullsize.py) equals the
    in-memory oracle, accepts the oracle's own gradient rounded to bf16 and
    rejects one row off by 5 %."""
    from _fullsize import masked_rows_zero, stream_oracle
    t = _bf16_case()
    cfg = oracle.LossConfig(eps_low=0.2, eps_high=0.28, beta=0.04)
    groups = dict(samples_per_prompt=4)
    h = {k: (v.float().numpy() if v.is_floating_point() else v.numpy()) for k, v in t.items()}
    want = oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"],
                                    h["mask"], h["rewards"], groups=groups, cfg=cfg)
    grad = torch.tensor(want.grad).to(torch.bfloat16)
    wl = SimpleNamespace()
    got, st = stream_oracle(t, grad, wl, cfg, groups, chunk=3, workers=3, announce=lambda m: None)
    assert got.loss == want.loss and np.array_equal(got.tok["G"], want.tok["G"])
    assert st["rows"] == int(h["mask"].sum())
    assert masked_rows_zero(grad, t["mask"])
    i, tt = np.argwhere(h["mask"])[len(np.argwhere(h["mask"])) // 2]
    bad = grad.clone()
    bad[i, tt] = (bad[i, tt].float() * 1.05).to(torch.bfloat16)
    with pytest.raises(AssertionError):
        stream_oracle(t, bad, wl, cfg, groups, chunk=3, workers=3, announce=lambda m: None)
    # a nonzero masked row is caught
    mi, mt = np.argwhere(~h["mask"])[0]
    bad = grad.clone()
    bad[mi, mt, 0] = 1.0
    assert not masked_rows_zero(bad, t["mask"])


def test_loss_bar_is_strict_for_the_clipped_surrogate():
    """A loss 2e-4 off in relative terms fails the bf16 bar of the default
    objective, however large the propagated log-prob error would be; CISPO
    (value linear in logp) may still fall back to that propagated bound."""
    x, y, ids, old, mask, r = _case(4)
    for pg, ok in (("clip", False), ("cispo", True)):
        cfg = oracle.LossConfig(beta=0.1, pg_loss=pg)
        ref = oracle.grpo_loss_fwd_bwd(x, y, ids, old, mask, r, groups=dict(samples_per_prompt=2),
                                       cfg=cfg)
        res = _as_result(ref)
        res.loss = torch.tensor(ref.loss * (1 + 2e-4), dtype=torch.float32)
        # a huge log-prob error budget would cover the 2e-4 for either objective
        if ok:
            compare_scalars(res, ref, cfg, 1e-4, e_logp=1e-2, e_d=1e-2)
        else:
            with pytest.raises(AssertionError):
                compare_scalars(res, ref, cfg, 1e-4, e_logp=1e-2, e_d=1e-2)


def test_stream_oracle_sequence_level():
    """The streaming comparison of a sequence-level loss (GSPO): the second
    pass's gradient rows, rounded to bf16, pass; one row off by 5 % fails."""
    from _fullsize import stream_oracle
    t = _bf16_case(seed=6)
    cfg = oracle.LossConfig(eps_low=0.2, eps_high=0.2, beta=0.04, pg_loss="gspo",
                            reduction="sequence_mean")
    groups = dict(samples_per_prompt=4)
    h = {k: (v.float().numpy() if v.is_floating_point() else v.numpy()) for k, v in t.items()}
    want = oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"],
                                    h["mask"], h["rewards"], groups=groups, cfg=cfg)
    grad = torch.tensor(want.grad).to(torch.bfloat16)
    got, st = stream_oracle(t, grad, None, cfg, groups, chunk=5, workers=2, announce=lambda m: None)
    assert got.loss == want.loss and np.array_equal(got.seq_logratio, want.seq_logratio)
    i, tt = np.argwhere(h["mask"])[3]
    bad = grad.clone()
    bad[i, tt] = (bad[i, tt].float() * 1.05).to(torch.bfloat16)
    with pytest.raises(AssertionError):
        stream_oracle(t, bad, None, cfg, groups, chunk=5, workers=2, announce=lambda m: None)


def test_token_grad_other_branch_only_at_a_clip_bound():
    """compare_token_grad: the oracle's float32 dlogp passes; a token whose
    ratio sits on a clip bound may take the other branch; the same flip at a
    token away from the bounds fails, and so does a nonzero masked token."""
    from _parity import compare_token_grad
    rng = np.random.default_rng(5)
    B, T = 8, 64
    logp = np.log(rng.uniform(1e-3, 1.0, (B, T))).astype(np.float32)
    old = (logp + rng.normal(0, 0.3, (B, T))).astype(np.float32)
    # two tokens per sequence exactly on the bounds 1 + eps and 1 - eps (in float32)
    old[:, 3] = (logp[:, 3].astype(np.float64) - np.log(1.2)).astype(np.float32)
    old[:, 5] = (logp[:, 5].astype(np.float64) - np.log(0.8)).astype(np.float32)
    ref_lp = (logp + rng.normal(0, 0.3, (B, T))).astype(np.float32)
    mask = np.arange(T)[None, :] < rng.integers(8, T + 1, B)[:, None]
    r = np.array([0, 1, 1, 0, 1, 0, 0, 1], dtype=np.float32)
    cfg = oracle.LossConfig(eps_low=0.2, eps_high=0.2, beta=0.04, reduction="sequence_mean")
    ref = oracle.grpo_token_loss(logp, old, ref_lp, mask, r, groups=dict(samples_per_prompt=4),
                                 cfg=cfg)
    g = ref.grad.astype(np.float32).astype(np.float64)
    assert compare_token_grad(g, ref, cfg, mask, 1e-5, "oracle")[1] == 0
    adv = ref.advantages[:, None]
    rho = ref.tok["rho"]
    w = ref.seq_weight[:, None]
    # flip the bound tokens to the other branch: the unclipped value is -A rho w
    # plus the KL part, the clipped one the KL part alone
    flip = g.copy()
    for t in (3, 5):
        kl_part = g[:, t] - np.where(ref.tok["clipped"][:, t], 0.0, -adv[:, 0] * rho[:, t] * w[:, 0])
        flip[:, t] = np.where(ref.tok["clipped"][:, t], kl_part - adv[:, 0] * rho[:, t] * w[:, 0],
                              kl_part)
    n_amb, n_other = compare_token_grad(flip, ref, cfg, mask, 1e-5, "flipped at bounds")
    assert n_amb >= 2 * B and n_other > 0
    # the same flip away from a bound fails
    far = g.copy()
    t = 10
    i = int(np.argmax(mask[:, t] & (adv[:, 0] != 0) & ~ref.tok["clipped"][:, t]))
    assert mask[i, t] and adv[i, 0] != 0
    far[i, t] = g[i, t] + adv[i, 0] * rho[i, t] * w[i, 0]
    with pytest.raises(AssertionError):
        compare_token_grad(far, ref, cfg, mask, 1e-5, "flipped away")
    bad = g.copy()
    mi, mt = np.argwhere(~mask)[0]
    bad[mi, mt] = 1e-3
    with pytest.raises(AssertionError):
        compare_token_grad(bad, ref, cfg, mask, 1e-5, "masked")
