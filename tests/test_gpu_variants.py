"""Parity of the objective variants (policy-loss forms, KL estimators, KL
clamps, the fixed-constant normaliser, the truncated off-policy importance
weight) on the HIP path, through the C ABI,
against the fp64 oracle: logits entry point on each row-kernel path (wave per
row, resident row, streaming row) and the log-prob token entry point."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from _parity import (branch_ambiguity, cfg_from, compare_exact_parts, compare_logits_grad,
                     compare_scalars, compare_token_values, gpu_kwargs, host_inputs, to_np)
from workloads import (TOKEN_WORKLOADS, LogitsWorkload, make_gen_logps, make_logits_inputs,
                       make_token_inputs)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# ratio spread wide enough that both clip bounds, the dual-clip bound and
# both KL clamps are crossed by many tokens
VARIANTS = [
    dict(dual_clip_c=1.5),
    dict(pg_loss="cispo"),
    dict(pg_loss="cispo", kl_estimator="k2"),
    dict(pg_loss="sapo", sapo_tau_pos=1.0, sapo_tau_neg=1.05),
    dict(pg_loss="sapo", sapo_tau_pos=2.0, sapo_tau_neg=0.5, kl_estimator="k1"),
    dict(pg_loss="reinforce"),
    dict(pg_loss="on_policy"),
    dict(kl_estimator="k1"),
    dict(kl_estimator="k2"),
    dict(kl_input_clamp=0.2),
    dict(kl_estimator="k2", kl_output_clamp=0.05),
    dict(kl_input_clamp=0.3, kl_output_clamp=0.02),
    dict(reduction="fixed_constant", norm_constant=4096.0),
    dict(reduction="length_alpha", alpha=0.5, pg_loss="cispo"),
    # off-policy importance weight (the generating policy's log-probs are an input)
    dict(is_only=True),
    dict(tis_type="tis", tis_ratio_max=1.3),
    dict(tis_type="icepop", tis_ratio_min=0.8, tis_ratio_max=1.25, pg_loss="cispo"),
    dict(tis_type="tis", tis_ratio_min=0.5, tis_ratio_max=2.0, dual_clip_c=1.5, kl_estimator="k2"),
]


def _id(kw):
    return "-".join(f"{k}={v}" for k, v in kw.items() if v is not None)


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _wl(V, dtype, T=16, sizes=(4, 4, 4, 4), **kw):
    base = dict(name=f"variant_V{V}_{dtype}", group_sizes=sizes, T=T, V=V, dtype=dtype,
                logit_std=2.0, ref_noise_std=math.sqrt(0.1), old_noise_std=0.7, reward_p=0.5,
                len_range=(1, T), beta=0.1)
    base.update(kw)
    return LogitsWorkload(**base)


def _split(kw):
    """(reduction, alpha, whether the case takes generating log-probs, objective keywords)"""
    kw = dict(kw)
    red = kw.pop("reduction", None)
    alpha = kw.pop("alpha", None)
    use_gen = kw.pop("is_only", False) or "tis_type" in kw
    return red, alpha, use_gen, kw


def check_variant_logits(rpl, wl, kw, seed=0):
    red, alpha, use_gen, obj = _split(kw)
    if alpha is not None:
        wl = dataclasses.replace(wl, alpha=alpha)
    announce(f"variant logits {wl.name} {_id(kw)} seed={seed}")
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=seed)
    if use_gen:
        inp_cpu["gen_logps"] = make_gen_logps(inp_cpu["old_logps"], seed=seed)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    gkw = gpu_kwargs(wl, red, **obj)
    res = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                inp["rewards"], inp["mask"], per_token=True,
                                gen_logps=inp.get("gen_logps"), **gkw)
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    cfg = cfg_from(wl, red, **obj)
    ref = oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"],
                                   h["mask"], h["rewards"], groups=wl.groups_kwargs(), cfg=cfg,
                                   gen_logps=h.get("gen_logps"))
    bf16 = wl.dtype == "bf16"
    rtol = 1e-4 if bf16 else 1e-5
    compare_exact_parts(res, ref, wl.name)
    rel, kappa, propagated = compare_scalars(res, ref, cfg, rtol, wl.name)
    compare_token_values(res, ref, cfg, h["mask"], rtol)
    stats = compare_logits_grad(to_np(res.grad), ref, cfg, h["mask"], bf16, wl.name,
                                policy=h["policy"], ids=h["action_ids"])
    clipped = int(to_np(res.counts)[1])
    assert abs(clipped - ref.clipped) <= stats["ambiguous"], (clipped, ref.clipped, stats)
    assert int(to_np(res.status)[0]) == 0
    print(f"  rel={rel:.3g} propagated={propagated} stats={stats} clipped={clipped}/{ref.clipped}",
          flush=True)
    return res, ref


@pytest.mark.parametrize("kw", VARIANTS, ids=_id)
@pytest.mark.parametrize("V,dtype", [(1000, "f32"), (4097, "bf16")])
def test_variant_logits_small_rows(gpu_lib, kw, V, dtype):
    """Wave-per-row (V = 1000 f32) and block-per-row (V = 4097 bf16, scalar tail)."""
    check_variant_logits(gpu_lib, _wl(V, dtype), kw)


@pytest.mark.parametrize("kw", [VARIANTS[0], VARIANTS[2], VARIANTS[4], VARIANTS[11], VARIANTS[16]],
                         ids=_id)
@pytest.mark.parametrize("V", [32000, 151936])
def test_variant_logits_long_rows(gpu_lib, kw, V):
    """Resident-row kernel (V = 32000 bf16) and streaming kernel (V = 151936 bf16)."""
    check_variant_logits(gpu_lib, _wl(V, "bf16", T=6, sizes=(4, 4)), kw, seed=2)


def test_variant_autograd_split_passes(gpu_lib):
    """grpo_loss (forward-only pass, then the gradient pass from the stashed
    per-row weights) equals the fused call for CISPO with the k2 estimator
    and a KL input clamp, through autograd."""
    wl = _wl(3000, "bf16")
    announce("variant autograd split")
    inp = {k: v.to(DEV) for k, v in make_logits_inputs(wl, device="cpu", seed=4).items()}
    kw = gpu_kwargs(wl, pg_loss="cispo", kl_estimator="k2", kl_input_clamp=0.25)
    fused = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"],
                                      inp["old_logps"], inp["rewards"], inp["mask"], **kw)
    x = inp["policy"].clone().requires_grad_(True)
    loss, pol, kl = gpu_lib.grpo_loss(x, inp["ref"], inp["action_ids"], inp["old_logps"],
                                      inp["rewards"], inp["mask"], **kw)
    (2.0 * loss).backward()
    torch.cuda.synchronize()
    assert float(loss.detach()) == float(fused.loss)
    # scaling by 2 is exact, so the two paths agree to bf16 rounding
    assert torch.allclose(x.grad.float(), 2.0 * fused.grad.float(), rtol=2 ** -7, atol=0)


# ---------------------------------------------------------------------------
# log-prob token entry point
# ---------------------------------------------------------------------------

def check_variant_tokens(rpl, kw, B=64, T=257, seed=0):
    red, alpha, use_gen, obj = _split(kw)
    base = TOKEN_WORKLOADS["token_loss_ragged"]
    wl = dataclasses.replace(base, old_noise_std=0.7, beta=0.1)
    announce(f"variant tokens {_id(kw)} B={B} T={T}")
    inp_cpu = make_token_inputs(wl, device="cpu", seed=seed, B=B, T=T)
    if use_gen:
        inp_cpu["gen_logps"] = make_gen_logps(inp_cpu["old_logps"], seed=seed)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    red = red or wl.reduction
    res = rpl.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                              inp["mask"], gen_logps=inp.get("gen_logps"), eps_low=wl.eps_low,
                              eps_high=wl.eps_high, beta=wl.beta,
                              samples_per_prompt=wl.group_size, reduction=red, alpha=alpha,
                              per_token=True, **obj)
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    cfg = oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
                            reduction=red, alpha=alpha, **obj)
    ref = oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"],
                                 h["rewards"], groups=dict(samples_per_prompt=wl.group_size),
                                 cfg=cfg, gen_logp=h.get("gen_logps"))
    # float32 inputs: only the float32 arithmetic of the kernel separates it
    # from the oracle (a few ulp in the ratio and in d)
    e = 2.0 ** -21
    compare_exact_parts(res, ref)
    compare_scalars(res, ref, cfg, 1e-5, e_logp=e, e_d=e)
    compare_token_values(res, ref, cfg, h["mask"], 1e-5, e_logp=e, e_d=e)
    g = to_np(res.grad)
    flag, anyb, cands = branch_ambiguity(ref, cfg, h["mask"], e_logp=4 * e, e_d=4 * e)
    gmax = float(np.max(np.abs(ref.grad)))
    ok = np.abs(g - ref.grad) <= 1e-5 * gmax
    for C in cands[1:]:
        ok |= anyb & (np.abs(g - C) <= 1e-5 * gmax)
    bad = ~ok & h["mask"]
    assert not bad.any(), f"{int(bad.sum())} dlogp values out of tolerance"
    assert np.all(g[~h["mask"]] == 0.0)
    clipped = int(to_np(res.counts)[1])
    assert abs(clipped - ref.clipped) <= int(flag.sum())


@pytest.mark.parametrize("kw", VARIANTS, ids=_id)
def test_variant_tokens_vector_path(gpu_lib, kw):
    check_variant_tokens(gpu_lib, kw, T=256)


@pytest.mark.parametrize("kw", [VARIANTS[0], VARIANTS[3], VARIANTS[11], VARIANTS[17]], ids=_id)
def test_variant_tokens_scalar_path(gpu_lib, kw):
    check_variant_tokens(gpu_lib, kw, B=32, T=131, seed=1)
