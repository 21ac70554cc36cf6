"""Full-size workloads, in the launch configuration bench.py times, compared
whole against the fp64 oracle.

The logits workloads (10^10 vocabulary entries) are streamed through the
oracle a chunk of rows at a time on the host's cores (tests/_fullsize.py):
  * advantages, weights, token counts: bit-exact against the oracle;
  * the three scalars against the oracle's own scalars at the stated bar
    (bf16 logits: loss relative error <= 1e-4), per-sequence totals, every
    active token's log-prob, loss and k3;
  * every active gradient row against the oracle's row at 2^-7 per element
    (rows at a clip bound may match either branch, ill-conditioned rows
    their propagated bound; both are counted and printed);
  * every masked gradient row is exactly zero, every row sums to ~0;
  * a second call is bit-identical.
The token-loss workload (4,194,304 tokens) is compared whole as well.
"""

import numpy as np
import pytest
import torch

import oracle
from _fullsize import masked_rows_zero, stream_oracle
from _parity import (LOGP_ABS_ERR, assert_grad_rows_sum_to_zero, branch_ambiguity, cfg_from,
                     compare_exact_parts, compare_scalars, compare_token_grad, compare_token_values,
                     gpu_kwargs, to_np)
from workloads import TOKEN_WORKLOADS, WORKLOADS, make_logits_inputs, make_token_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


@pytest.mark.parametrize("name,reduction", [
    ("logits_v32000", None),
    ("logits_v151936", None),
    ("logits_csr_v128256", "token_mean"),
    ("logits_csr_v128256", "sequence_mean"),
    ("logits_csr_v128256", "length_alpha"),
])
def test_fullsize_logits(gpu_lib, name, reduction):
    rpl = gpu_lib
    wl = WORKLOADS[name]
    red = reduction or wl.reductions[0]
    what = f"{name} {red}"
    announce(f"full size {what}: generating")
    inp = make_logits_inputs(wl, device=DEV, seed=0)
    B, T, V = wl.B, wl.T, wl.V
    kw = gpu_kwargs(wl, red)
    grad = torch.empty((B, T, V), dtype=inp["policy"].dtype, device=DEV)
    announce(f"full size {what}: run 1")
    res = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                inp["rewards"], inp["mask"], grad_out=grad, per_token=True, **kw)
    torch.cuda.synchronize()
    assert int(res.status[0]) == 0

    cfg = cfg_from(wl, red)
    mask = inp["mask"].cpu().numpy().astype(bool)
    ref, st = stream_oracle(inp, grad, wl, cfg, wl.groups_kwargs(), announce=announce)
    announce(f"full size {what}: oracle done, {st}")
    compare_exact_parts(res, ref, what)
    compare_scalars(res, ref, cfg, 1e-4, what)
    compare_token_values(res, ref, cfg, mask, 1e-4)
    glp = to_np(res.tok_logp)
    assert np.all(np.abs(glp - ref.tok["logp"])[mask] <= LOGP_ABS_ERR), what
    flag, _, _ = branch_ambiguity(ref, cfg, mask)
    clipped = int(res.counts[1])
    assert abs(clipped - ref.clipped) <= int(flag.sum()), (clipped, ref.clipped, int(flag.sum()))
    announce(f"full size {what}: clipped gpu={clipped} oracle={ref.clipped} "
             f"ambiguous={int(flag.sum())}")

    assert masked_rows_zero(grad, inp["mask"]), what
    # every gradient row sums to ~0: G * (1 - sum p); bf16 rounding bounds the rest
    announce(f"full size {what}: row sums")
    assert_grad_rows_sum_to_zero(grad.view(B * T, V))

    # bit-identical second run
    announce(f"full size {what}: run 2")
    grad2 = torch.empty_like(grad)
    res2 = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                 inp["rewards"], inp["mask"], grad_out=grad2, **kw)
    torch.cuda.synchronize()
    assert torch.equal(res.scalars.view(torch.int32), res2.scalars.view(torch.int32))
    assert torch.equal(grad.view(torch.int16), grad2.view(torch.int16))


@pytest.mark.parametrize("name", ["token_loss_full", "token_loss_ragged"])
def test_fullsize_token_loss(gpu_lib, name):
    """B = 1024 sequences x T = 4096 = 4,194,304 tokens, groups of 16, sequence
    mean: compared whole against the oracle."""
    wl = TOKEN_WORKLOADS[name]
    announce(f"full size {name}")
    inp = make_token_inputs(wl, device=DEV, seed=0)
    res = gpu_lib.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                                  inp["mask"], eps_low=wl.eps_low, eps_high=wl.eps_high,
                                  beta=wl.beta, samples_per_prompt=wl.group_size,
                                  reduction=wl.reduction, per_token=True)
    torch.cuda.synchronize()
    h = {k: v.cpu().numpy() for k, v in inp.items()}
    cfg = oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
                            reduction=wl.reduction)
    ref = oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"], h["rewards"],
                                 groups=dict(samples_per_prompt=wl.group_size), cfg=cfg)
    compare_exact_parts(res, ref, name)
    compare_scalars(res, ref, cfg, 1e-5, name)
    compare_token_values(res, ref, cfg, h["mask"].astype(bool), 1e-5)
    n_amb, _ = compare_token_grad(to_np(res.grad), ref, cfg, h["mask"].astype(bool), 1e-5, name)
    clipped = int(res.counts[1])
    assert abs(clipped - ref.clipped) <= n_amb
    res2 = gpu_lib.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                                   inp["mask"], eps_low=wl.eps_low, eps_high=wl.eps_high,
                                   beta=wl.beta, samples_per_prompt=wl.group_size,
                                   reduction=wl.reduction)
    torch.cuda.synchronize()
    assert torch.equal(res.scalars.view(torch.int32), res2.scalars.view(torch.int32))
    assert torch.equal(res.grad.view(torch.int32), res2.grad.view(torch.int32))
