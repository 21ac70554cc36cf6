"""Full-size workloads, in the launch configuration bench.py times.

The logits workloads are far too large for the fp64 oracle to redo whole
(10^10 vocabulary entries), so each check uses what the oracle can compute
one row at a time plus properties that hold at any size:
  * advantages, weights, token counts: bit-exact against the oracle;
  * sampled rows (first, last, every group, random): log-prob, token loss,
    k3 and the whole gradient row against the oracle;
  * the scalars against the fp64 fixed-order sum of the kernel's own
    per-token outputs (checks the two reduction stages at full size);
  * every gradient row sums to ~0 (softmax rows sum to one);
  * a second call is bit-identical.
The token-loss workload (4,194,304 tokens) is compared whole.
"""

import numpy as np
import pytest
import torch

import oracle
from _parity import (LOGP_ABS_ERR, assert_grad_rows_sum_to_zero, cfg_from, compare_exact_parts,
                     compare_scalars, gpu_kwargs, sample_rows, to_np)
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
    announce(f"full size {name} {red}: generating")
    inp = make_logits_inputs(wl, device=DEV, seed=0)
    B, T, V = wl.B, wl.T, wl.V
    kw = gpu_kwargs(wl, red)
    grad = torch.empty((B, T, V), dtype=inp["policy"].dtype, device=DEV)
    announce(f"full size {name} {red}: run 1")
    res = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                inp["rewards"], inp["mask"], grad_out=grad, per_token=True, **kw)
    torch.cuda.synchronize()
    assert int(res.status[0]) == 0

    mask = inp["mask"].cpu().numpy()
    rewards = inp["rewards"].cpu().numpy()
    cfg = cfg_from(wl, red)
    groups = wl.groups_kwargs()
    off = oracle.group_offsets(B, groups.get("samples_per_prompt"), groups.get("group_boundaries"))
    A = oracle.group_advantages(rewards, off, wl.leave_one_out, wl.scale_by_std)
    L, N, w = oracle.sequence_weights(mask, cfg.reduction, cfg.alpha)
    gA = to_np(res.advantages)
    assert np.array_equal(gA.astype(np.float32).view(np.uint32), A.astype(np.float32).view(np.uint32))
    assert np.array_equal(to_np(res.seq_weight).astype(np.float32).view(np.uint32),
                          w.astype(np.float32).view(np.uint32))
    assert np.array_equal(to_np(res.seq_tokens), L) and int(res.counts[0]) == N

    # scalars against the fixed-order fp64 sum of the kernel's per-token values
    tl = to_np(res.tok_loss)
    tk = to_np(res.tok_kl)
    P = tl.sum(axis=1)
    K = tk.sum(axis=1)
    pl = float(np.sum(w * P))
    kl = float(np.sum(w * K))
    for got, want in ((float(res.policy_loss), pl), (float(res.kl), kl),
                      (float(res.loss), pl + wl.beta * kl)):
        assert abs(got - want) <= 2e-7 * max(abs(want), 1e-30) + 1e-12, (got, want)
    assert np.allclose(to_np(res.seq_policy), P, rtol=1e-6, atol=1e-9)
    assert np.allclose(to_np(res.seq_kl), K, rtol=1e-6, atol=1e-9)

    # sampled rows against the oracle
    rng = np.random.default_rng(1)
    rows = sample_rows(B, T, mask, rng)
    announce(f"full size {name} {red}: {len(rows)} sampled rows")
    pol = inp["policy"].view(B * T, V)
    ref = inp["ref"].view(B * T, V)
    ids = inp["action_ids"].view(-1).cpu().numpy()
    old = inp["old_logps"].view(-1).cpu().numpy()
    g2 = grad.view(B * T, V)
    mflat = mask.reshape(-1)
    glp = to_np(res.tok_logp).reshape(-1)
    for r in rows:
        i = r // T
        g_row = g2[r].double().cpu().numpy()
        if not mflat[r]:
            assert np.all(g_row == 0.0) and tl.reshape(-1)[r] == 0.0
            continue
        x = pol[r].float().cpu().numpy()[None]
        y = ref[r].float().cpu().numpy()[None]
        o = oracle.logits_rows(x, y, ids[r:r + 1], old[r:r + 1], A[i:i + 1], w[i:i + 1], cfg)
        assert abs(glp[r] - o["logp"][0]) <= LOGP_ABS_ERR, (r, glp[r], o["logp"][0])
        lo, hi = 1 - cfg.eps_low, 1 + cfg.eps_high
        rho = o["rho"][0]
        ambiguous = min(abs(rho - lo), abs(rho - hi)) <= rho * 4 * LOGP_ABS_ERR
        if ambiguous:
            continue
        # token loss / k3 within the propagated float32 log-prob error
        assert abs(tl.reshape(-1)[r] - o["loss"][0]) <= 2 * LOGP_ABS_ERR * abs(A[i]) * rho + 1e-6
        assert abs(tk.reshape(-1)[r] - o["kl"][0]) <= 2 * LOGP_ABS_ERR * abs(np.expm1(o["d"][0])) + 1e-7
        # gradient row, bf16 criterion (with the ill-conditioned-G allowance)
        G = o["G"][0]
        dG = abs(w[i]) * (abs(A[i]) * rho + 2 * cfg.beta * np.exp(o["d"][0])) * 2 * LOGP_ABS_ERR
        tol = max(2.0 ** -7, dG / abs(G)) if G != 0 else 0.0
        gr = o["grad"][0]
        err = np.abs(g_row - gr)
        assert np.all(err <= tol * np.abs(gr) + 2.0 ** -126), (r, float(np.max(err / (np.abs(gr) + 1e-300))))

    # every gradient row sums to ~0: G * (1 - sum p); bf16 rounding bounds the rest
    announce(f"full size {name} {red}: row sums")
    assert_grad_rows_sum_to_zero(g2)

    # bit-identical second run
    announce(f"full size {name} {red}: run 2")
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
    g = to_np(res.grad)
    rho = ref.tok["rho"]
    lo, hi = 1 - wl.eps_low, 1 + wl.eps_high
    amb = (np.abs(rho - hi) <= 4e-7 * rho) | (np.abs(rho - lo) <= 4e-7 * rho)
    err = np.abs(g - ref.grad)
    bad = (err > 1e-5 * np.max(np.abs(ref.grad))) & ~amb
    assert not bad.any(), int(bad.sum())
    clipped = int(res.counts[1])
    assert abs(clipped - ref.clipped) <= int((amb & h["mask"]).sum())
    res2 = gpu_lib.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                                   inp["mask"], eps_low=wl.eps_low, eps_high=wl.eps_high,
                                   beta=wl.beta, samples_per_prompt=wl.group_size,
                                   reduction=wl.reduction)
    torch.cuda.synchronize()
    assert torch.equal(res.scalars.view(torch.int32), res2.scalars.view(torch.int32))
    assert torch.equal(res.grad.view(torch.int32), res2.grad.view(torch.int32))
