"""Parity of the sequence-level losses on the HIP path, through the C ABI,
against the fp64 oracle: the GSPO sequence ratio (Relax REINFORCE++ page,
Formula-level comparison; dockyard_rl, One loss many algorithms), the REAL
in-group classification loss (ms-swift REAL blog) and sequence-masked
truncated importance sampling (dockyard_rl, Off-policy correction).

Logits entry point on each row-kernel width (64, 256 and 1024 threads per
row, ragged scalar tails), the log-prob token entry point (vector and scalar
paths), the split forward/backward used by autograd, grad_scale, masked
NaN/Inf and bitwise repeats.  Inputs shift whole sequences' log-ratios so
that GSPO sequences fall on both sides of the clip band and seq-mask masks
some sequences."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from _parity import (GRAD16_BAR, cfg_from, compare_exact_parts, compare_logits_grad,
                     compare_scalars, compare_seq_outputs, compare_token_values, gpu_kwargs,
                     host_inputs, seq_branches, to_np)
from workloads import (LogitsWorkload, TokenWorkload, make_gen_logps, make_logits_inputs,
                       make_token_inputs, poison_masked, shift_by_sequence)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

SEQ_CASES = [
    dict(pg_loss="gspo", reduction="sequence_mean"),
    dict(pg_loss="gspo", reduction="length_alpha", alpha=0.5, kl_estimator="k2"),
    dict(pg_loss="gspo", reduction="sequence_mean", tis_type="tis", tis_ratio_max=1.3),
    dict(pg_loss="gspo", reduction="fixed_constant", norm_constant=300.0, is_only=True),
    dict(pg_loss="gspo", reduction="per_sequence_then_mean"),
    dict(pg_loss="real"),
    dict(pg_loss="real", real_tau=0.2, kl_input_clamp=0.2),
    dict(tis_type="seq_mask", tis_ratio_min=0.8, tis_ratio_max=1.25),
    dict(tis_type="seq_mask", tis_ratio_min=0.8, tis_ratio_max=1.25, pg_loss="cispo",
         reduction="sequence_mean"),
]


def _id(kw):
    return "-".join(f"{k}={v}" for k, v in kw.items() if v is not None)


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _wl(V, dtype, T=16, sizes=(4, 4, 4, 4), **kw):
    base = dict(name=f"seq_V{V}_{dtype}", group_sizes=sizes, T=T, V=V, dtype=dtype,
                logit_std=2.0, ref_noise_std=math.sqrt(0.1), old_noise_std=0.3, reward_p=0.5,
                len_range=(1, T), beta=0.1)
    base.update(kw)
    return LogitsWorkload(**base)


def _split(kw):
    kw = dict(kw)
    red = kw.pop("reduction", None)
    alpha = kw.pop("alpha", None)
    use_gen = kw.pop("is_only", False) or "tis_type" in kw
    return red, alpha, use_gen, kw


def _inputs(wl, seed, use_gen):
    inp = make_logits_inputs(wl, device="cpu", seed=seed)
    inp["old_logps"] = shift_by_sequence(inp["old_logps"], seed=seed, spread=0.4)
    if use_gen:
        inp["gen_logps"] = shift_by_sequence(make_gen_logps(inp["old_logps"], seed=seed),
                                             seed=seed + 1, spread=0.3)
    return inp


def check_seq_logits(rpl, wl, kw, seed=0, grad_dtype=None):
    red, alpha, use_gen, obj = _split(kw)
    if alpha is not None:
        wl = dataclasses.replace(wl, alpha=alpha)
    announce(f"sequence-level logits {wl.name} {_id(kw)} seed={seed}")
    inp_cpu = _inputs(wl, seed, use_gen)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    gkw = gpu_kwargs(wl, red, **obj)
    res = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                inp["rewards"], inp["mask"], per_token=True,
                                gen_logps=inp.get("gen_logps"), grad_dtype=grad_dtype, **gkw)
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    cfg = cfg_from(wl, red, **obj)
    groups = wl.groups_kwargs()
    ref = oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"],
                                   h["mask"], h["rewards"], groups=groups, cfg=cfg,
                                   gen_logps=h.get("gen_logps"))
    gdt = {None: wl.dtype, torch.float32: "f32"}[grad_dtype]
    rtol = 1e-5 if wl.dtype == "f32" else 1e-4
    compare_exact_parts(res, ref, wl.name)
    seqlv = cfg.pg_loss in oracle.SEQUENCE_PG
    if seqlv:
        amb_seq = compare_seq_outputs(res, ref, cfg, h["mask"], h, groups, rtol, wl.name)
        base = GRAD16_BAR.get(gdt, (1e-5, 0))[0]
        br = seq_branches(ref, cfg, h["mask"], h, groups, base)
        stats = compare_logits_grad(to_np(res.grad), ref, cfg, h["mask"], gdt, wl.name,
                                    policy=h["policy"], ids=h["action_ids"], branches=br)
        amb_tokens = int(br[0].sum())
    else:
        rel, kappa, _ = compare_scalars(res, ref, cfg, rtol, wl.name)
        compare_token_values(res, ref, cfg, h["mask"], rtol)
        stats = compare_logits_grad(to_np(res.grad), ref, cfg, h["mask"], gdt, wl.name,
                                    policy=h["policy"], ids=h["action_ids"])
        amb_seq, amb_tokens = 0, stats["ambiguous"]
        # the masking flag of each sequence is an exact binary64 decision
        assert ref.seq_keep is not None and ref.seq_keep.any() and not ref.seq_keep.all()
    clipped = int(to_np(res.counts)[1])
    assert abs(clipped - ref.clipped) <= amb_tokens, (clipped, ref.clipped, stats)
    assert int(to_np(res.status)[0]) == 0
    if cfg.pg_loss == "gspo":
        assert 0 < ref.clipped < ref.num_tokens, "the inputs must clip some sequences, not all"
    print(f"  stats={stats} clipped={clipped}/{ref.clipped} ambiguous_seq={amb_seq}", flush=True)
    return res, ref, inp


@pytest.mark.parametrize("kw", SEQ_CASES, ids=_id)
@pytest.mark.parametrize("V,dtype", [(1000, "f32"), (4097, "bf16")])
def test_seq_logits_small_rows(gpu_lib, kw, V, dtype):
    """64 threads per row (V = 1000 f32) and 256 (V = 4097 bf16, scalar tail)."""
    check_seq_logits(gpu_lib, _wl(V, dtype), kw)


@pytest.mark.parametrize("kw", [SEQ_CASES[0], SEQ_CASES[2], SEQ_CASES[4], SEQ_CASES[6]], ids=_id)
@pytest.mark.parametrize("V", [32000, 151936])
def test_seq_logits_long_rows(gpu_lib, kw, V):
    """256 threads per row (V = 32000 bf16) and 1024 (V = 151936 bf16)."""
    check_seq_logits(gpu_lib, _wl(V, "bf16", T=6, sizes=(4, 4)), kw, seed=2)


def test_seq_real_csr_leave_one_out(gpu_lib):
    """REAL over CSR groups of unequal size with leave-one-out advantages and
    one all-equal group (contributes nothing)."""
    wl = _wl(2048, "bf16", T=12, sizes=(4, 8, 2, 6), csr=True, leave_one_out=True,
             degenerate_groups=1)
    check_seq_logits(gpu_lib, wl, dict(pg_loss="real"), seed=3)


@pytest.mark.parametrize("kw", [SEQ_CASES[0], SEQ_CASES[4], SEQ_CASES[6]], ids=_id)
@pytest.mark.parametrize("V", [4097, 20000])
def test_seq_logits_f16(gpu_lib, V, kw):
    """IEEE half logits and gradient through the sequence-level losses (the
    forward-only kernel, then the gradient-only kernel: 256 threads per row
    with a scalar tail at V = 4097, 1024 at V = 20000) and the
    sequence-masked truncated IS (the fused kernel)."""
    check_seq_logits(gpu_lib, _wl(V, "f16", T=8), kw, seed=6)


def test_seq_gspo_f32_gradient_from_bf16(gpu_lib):
    check_seq_logits(gpu_lib, _wl(4097, "bf16"), SEQ_CASES[0], seed=4, grad_dtype=torch.float32)


@pytest.mark.parametrize("kw", [SEQ_CASES[0], SEQ_CASES[4]], ids=_id)
def test_seq_split_backward_and_grad_scale(gpu_lib, kw):
    """The autograd split (forward only, then backward with grad_scale) equals
    the fused call bitwise; grad_scale = 0.5 halves the fused gradient
    exactly; a repeat is bit-identical."""
    rpl = gpu_lib
    wl = _wl(4097, "bf16")
    red, _, _, obj = _split(kw)
    inp = {k: v.to(DEV) for k, v in _inputs(wl, 5, False).items()}
    gkw = gpu_kwargs(wl, red, **obj)
    args = (inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"], inp["rewards"],
            inp["mask"])
    announce(f"sequence-level split/scale {_id(kw)}")
    fused = rpl.grpo_loss_fwd_bwd(*args, **gkw)
    again = rpl.grpo_loss_fwd_bwd(*args, **gkw)
    half = torch.tensor([0.5], dtype=torch.float32, device=DEV)
    scaled = rpl.grpo_loss_fwd_bwd(*args, grad_scale=half, **gkw)
    pol = inp["policy"].clone().requires_grad_(True)
    loss, _, _ = rpl.grpo_loss(pol, *args[1:], **gkw)
    loss.backward(torch.tensor(1.0, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(fused.grad.view(torch.int16), again.grad.view(torch.int16))
    assert torch.equal(fused.scalars.view(torch.int32), again.scalars.view(torch.int32))
    assert torch.equal(fused.seq_logratio.view(torch.int32), again.seq_logratio.view(torch.int32))
    assert torch.equal((fused.grad.float() * 0.5).to(torch.bfloat16).view(torch.int16),
                       scaled.grad.view(torch.int16))
    assert torch.equal(pol.grad.view(torch.int16), fused.grad.view(torch.int16))
    assert float(loss.detach()) == float(fused.loss)


@pytest.mark.parametrize("kw", [SEQ_CASES[0], SEQ_CASES[4]], ids=_id)
@pytest.mark.parametrize("V,dtype,T", [(1000, "f32", 2048), (2600, "bf16", 1400)])
def test_seq_large_csr_split_bitwise(gpu_lib, kw, V, dtype, T):
    """Sequence-level losses over a larger batch of unequal CSR groups
    (4, 8, 2, 6, 4) with T = 2048 (64 threads and four rows per block) and
    T = 1400 (256 threads per row): against the oracle, and bitwise against
    the autograd split (the forward pass alone, then the backward pass)."""
    rpl = gpu_lib
    wl = _wl(V, dtype, T=T, sizes=(4, 8, 2, 6, 4), csr=True)
    res, _, inp = check_seq_logits(rpl, wl, kw, seed=6)
    red, _, _, obj = _split(kw)
    gkw = gpu_kwargs(wl, red, **obj)
    args = (inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"], inp["rewards"],
            inp["mask"])
    fused = rpl.grpo_loss_fwd_bwd(*args, **gkw)
    pol = inp["policy"].clone().requires_grad_(True)
    loss, _, _ = rpl.grpo_loss(pol, *args[1:], **gkw)
    loss.backward(torch.tensor(1.0, device=DEV))
    torch.cuda.synchronize()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(pol.grad.view(bits), fused.grad.view(bits))
    assert torch.equal(fused.grad.view(bits), res.grad.view(bits))
    assert float(loss.detach()) == float(fused.loss)


@pytest.mark.parametrize("kw", [SEQ_CASES[0], SEQ_CASES[4], SEQ_CASES[6]], ids=_id)
def test_seq_masked_slots_never_read(gpu_lib, kw):
    rpl = gpu_lib
    wl = _wl(1000, "f32")
    red, _, use_gen, obj = _split(kw)
    inp = {k: v.to(DEV) for k, v in _inputs(wl, 6, use_gen).items()}
    bad = poison_masked(inp, V=wl.V)
    if use_gen:
        g = inp["gen_logps"].clone()
        g[~inp["mask"]] = float("nan")
        bad["gen_logps"] = g
    gkw = gpu_kwargs(wl, red, **obj)
    announce(f"sequence-level masked NaN/Inf {_id(kw)}")
    outs = []
    for d in (inp, bad):
        r = rpl.grpo_loss_fwd_bwd(d["policy"], d["ref"], d["action_ids"], d["old_logps"],
                                  d["rewards"], d["mask"], gen_logps=d.get("gen_logps"),
                                  per_token=True, **gkw)
        outs.append(r)
    torch.cuda.synchronize()
    a, b = outs
    for name in ("scalars", "seq_policy", "seq_kl", "seq_logratio", "tok_loss", "tok_kl"):
        assert torch.equal(getattr(a, name).view(torch.int32), getattr(b, name).view(torch.int32)), name
    assert torch.equal(a.grad.view(torch.int32), b.grad.view(torch.int32))
    assert int(b.status[0]) == 0


def _tok_wl(T):
    return TokenWorkload(name=f"seq_tok_T{T}", group_size=4, num_groups=6, T=T,
                         old_noise_std=0.3, ref_noise_std=math.sqrt(0.1), reward_p=0.5,
                         len_range=(1, T), beta=0.1)


@pytest.mark.parametrize("kw", SEQ_CASES, ids=_id)
@pytest.mark.parametrize("T", [256, 203])
def test_seq_token_loss(gpu_lib, kw, T):
    """Log-prob entry point: vector path (T = 256) and scalar path (T = 203)."""
    rpl = gpu_lib
    wl = _tok_wl(T)
    red, alpha, use_gen, obj = _split(kw)
    red = red or "token_mean"
    announce(f"sequence-level token loss T={T} {_id(kw)}")
    inp = make_token_inputs(wl, device="cpu", seed=7)
    inp["old_logps"] = shift_by_sequence(inp["old_logps"], seed=7, spread=0.4)
    if use_gen:
        inp["gen_logps"] = shift_by_sequence(make_gen_logps(inp["old_logps"], seed=7), seed=8,
                                             spread=0.3)
    d = {k: v.to(DEV) for k, v in inp.items()}
    res = rpl.grpo_token_loss(d["logp"], d["old_logps"], d["ref_logp"], d["rewards"], d["mask"],
                              gen_logps=d.get("gen_logps"), eps_low=wl.eps_low,
                              eps_high=wl.eps_high, beta=wl.beta, samples_per_prompt=wl.group_size,
                              reduction=red, alpha=alpha, per_token=True, **obj)
    torch.cuda.synchronize()
    h = host_inputs(inp)
    cfg = oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=red,
                            alpha=alpha, **obj)
    groups = dict(samples_per_prompt=wl.group_size)
    ref = oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"], h["rewards"],
                                 groups=groups, cfg=cfg, gen_logp=h.get("gen_logps"))
    compare_exact_parts(res, ref, wl.name)
    g = to_np(res.grad)
    if cfg.pg_loss in oracle.SEQUENCE_PG:
        # the token path's log-probs are exact inputs: s_i carries only rounding
        amb_seq = compare_seq_outputs(res, ref, cfg, h["mask"], h, groups, 1e-5, wl.name)
        br = seq_branches(ref, cfg, h["mask"], h, groups, 1e-5)
        ok = np.abs(g - ref.grad) <= 1e-5 * np.max(np.abs(ref.grad)) + 1e-30
        amb = br[1]
        for C in br[2][1:]:
            ok |= amb & (np.abs(g - C) <= 1e-5 * np.max(np.abs(ref.grad)) + 1e-30)
        assert ok.all(), f"dlogp: {int((~ok).sum())} tokens out of tolerance"
        assert np.all(g[~h["mask"]] == 0.0)
    else:
        compare_scalars(res, ref, cfg, 1e-5, wl.name)
        ok = np.abs(g - ref.grad) <= 1e-5 * np.max(np.abs(ref.grad)) + 1e-30
        assert ok.all(), f"dlogp: {int((~ok).sum())} tokens out of tolerance"
    if cfg.pg_loss == "gspo":
        assert 0 < ref.clipped < ref.num_tokens
