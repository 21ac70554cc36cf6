"""Full-size parity of the sequence-level losses (GSPO sequence ratio, REAL
in-group classification) and of sequence-masked truncated importance
sampling, through the C ABI, in the launch configuration bench.py times
(forward pass, sequence phase, gradient pass).

Both full-size batches are compared whole: the fp64 oracle streams every
active row a chunk at a time on the host's cores (tests/_fullsize.py), its
second pass forming every gradient row once the sequences' log-ratios are
known, and each is compared with the GPU's row as it is formed.

logits_v32000 (B = 64 in 8 groups of 8, T = 1024, V = 32,000 bf16, ragged
lengths 64..1024: about 35 K active rows): GSPO, REAL and seq-mask-tis;
every per-token and per-sequence value, the scalars, the REAL coupling
within groups and every gradient row.

logits_v151936 (B = 32, T = 2048, V = 151,936 bf16, full mask: 65,536
rows): GSPO and REAL compared whole in the same way; GSPO is also checked
on every sequence by properties (s_i is the mean of the sequence's own
per-token log-ratios, the token loss is constant along a sequence), on three
sequences the oracle recomputes alone, every gradient row sums to ~0 and a
second call is bit-identical.

Old log-probs are shifted per sequence so that GSPO clips some sequences on
both sides of the band and seq-mask drops some sequences.
"""

import math
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import oracle
from _parity import (GRAD16_BAR, LOGP_ABS_ERR, SEQ_ABS_ERR, assert_grad_rows_sum_to_zero,
                     cfg_from, check_grad_row, compare_exact_parts, compare_scalars,
                     compare_seq_outputs, compare_token_values, gpu_kwargs, host_inputs,
                     sample_rows, seq_branches, to_np, token_branches)
from _fullsize import masked_rows_zero, stream_oracle
from workloads import WORKLOADS, make_gen_logps, make_logits_inputs, shift_by_sequence

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_BASE = GRAD16_BAR["bf16"][0]


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _id(kw):
    return "-".join(f"{k}={v}" for k, v in kw.items())


def _rerun_bitwise(rpl, inp, grad, res, kw, gen):
    grad2 = torch.empty_like(grad)
    res2 = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                 inp["rewards"], inp["mask"], grad_out=grad2, gen_logps=gen, **kw)
    torch.cuda.synchronize()
    assert torch.equal(res.scalars.view(torch.int32), res2.scalars.view(torch.int32))
    assert torch.equal(grad.view(torch.int16), grad2.view(torch.int16))


@pytest.fixture(scope="module")
def v32k():
    wl = WORKLOADS["logits_v32000"]
    announce("full size logits_v32000: generating")
    inp = make_logits_inputs(wl, device=DEV, seed=0)
    inp["old_logps"] = shift_by_sequence(inp["old_logps"], seed=0, spread=0.4)
    inp["gen_logps"] = shift_by_sequence(make_gen_logps(inp["old_logps"], seed=0), seed=1,
                                         spread=0.3)
    torch.cuda.synchronize()
    announce("full size logits_v32000: host copies")
    h = host_inputs(inp)
    yield wl, inp, h


V32_CASES = [
    dict(pg_loss="gspo", reduction="sequence_mean"),
    dict(pg_loss="real"),
    dict(tis_type="seq_mask", tis_ratio_min=0.8, tis_ratio_max=1.25),
]


@pytest.mark.parametrize("kw", V32_CASES, ids=_id)
def test_fullsize_v32000_whole(gpu_lib, v32k, kw):
    wl, inp, h_all = v32k
    obj = dict(kw)
    red = obj.pop("reduction", None)
    use_gen = "tis_type" in obj
    name = f"full size logits_v32000 {_id(kw)}"
    B, T, V = wl.B, wl.T, wl.V
    gkw = gpu_kwargs(wl, red, **obj)
    gen = inp["gen_logps"] if use_gen else None
    grad = torch.empty((B, T, V), dtype=torch.bfloat16, device=DEV)
    announce(f"{name}: run 1")
    res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"],
                                    inp["old_logps"], inp["rewards"], inp["mask"], grad_out=grad,
                                    per_token=True, gen_logps=gen, **gkw)
    torch.cuda.synchronize()
    assert int(res.status[0]) == 0

    h = {k: v for k, v in h_all.items() if k != "gen_logps" or use_gen}
    mask = h["mask"].astype(bool)
    cfg = cfg_from(wl, red, **obj)
    groups = wl.groups_kwargs()
    announce(f"{name}: oracle over {int(mask.sum())} active rows, every gradient row compared")
    ref, st = stream_oracle(inp, grad, wl, cfg, groups, announce=announce,
                            gen_logps=h.get("gen_logps"))
    announce(f"{name}: oracle done, {st}")
    compare_exact_parts(res, ref, name)
    glp = to_np(res.tok_logp)
    assert np.all(np.abs(glp - ref.tok["logp"])[mask] <= LOGP_ABS_ERR), name + " tok_logp"
    assert np.all(glp[~mask] == 0.0)
    if cfg.pg_loss in oracle.SEQUENCE_PG:
        amb_seq = compare_seq_outputs(res, ref, cfg, mask, h, groups, 1e-4, name)
        br = seq_branches(ref, cfg, mask, h, groups, BF16_BASE)
    else:
        amb_seq = 0
        compare_scalars(res, ref, cfg, 1e-4, name)
        compare_token_values(res, ref, cfg, mask, 1e-4)
        br = token_branches(ref, cfg, mask, BF16_BASE)
        # each sequence's masking flag is an exact binary64 decision
        assert ref.seq_keep.any() and not ref.seq_keep.all()
    if cfg.pg_loss == "gspo":
        assert 0 < ref.clipped < ref.num_tokens, "the inputs must clip some sequences, not all"
    clipped = int(res.counts[1])
    assert abs(clipped - ref.clipped) <= int(br[0].sum()), (clipped, ref.clipped)

    announce(f"{name}: masked rows, row sums (sequences at a clip bound: {amb_seq})")
    g2 = grad.view(B * T, V)
    assert masked_rows_zero(grad, inp["mask"]), name
    assert_grad_rows_sum_to_zero(g2)
    announce(f"{name}: run 2")
    _rerun_bitwise(gpu_lib, inp, grad, res, gkw, gen)


def _oracle_sequence(inp, i, A, L, w, cfg, chunk=256):
    """The oracle's per-token terms of every row of sequence i (full mask),
    row chunk by row chunk, plus its sequence-level policy terms."""
    T = inp["policy"].shape[1]
    ids = inp["action_ids"][i].cpu().numpy()
    old = inp["old_logps"][i].double().cpu().numpy()
    acc = {k: np.zeros(T) for k in ("logp", "d", "kl", "dkl")}
    for s in range(0, T, chunk):
        e = min(T, s + chunk)
        x = inp["policy"][i, s:e].float().cpu().numpy()
        y = inp["ref"][i, s:e].float().cpu().numpy()
        n = e - s
        out = oracle.logits_rows(x, y, ids[s:e], old[s:e], np.full(n, A[i]), np.full(n, w[i]), cfg,
                                 want_grad=False)
        for k in acc:
            acc[k][s:e] = out[k]
    sq = oracle.sequence_terms(1, np.zeros(T, dtype=np.int64), acc["logp"], old, None,
                               A[i:i + 1], L[i:i + 1], w[i:i + 1], np.array([0, 1]), cfg)
    return acc, sq, ids


def test_fullsize_gspo_headline(gpu_lib):
    wl = WORKLOADS["logits_v151936"]
    red = "sequence_mean"
    obj = dict(pg_loss="gspo")
    name = "full size logits_v151936 gspo sequence_mean"
    B, T, V = wl.B, wl.T, wl.V
    announce(f"{name}: generating")
    inp = make_logits_inputs(wl, device=DEV, seed=0)
    inp["old_logps"] = shift_by_sequence(inp["old_logps"], seed=0, spread=0.4)
    gkw = gpu_kwargs(wl, red, **obj)
    grad = torch.empty((B, T, V), dtype=torch.bfloat16, device=DEV)
    announce(f"{name}: run 1")
    res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"],
                                    inp["old_logps"], inp["rewards"], inp["mask"], grad_out=grad,
                                    per_token=True, **gkw)
    torch.cuda.synchronize()
    assert int(res.status[0]) == 0

    cfg = cfg_from(wl, red, **obj)
    mask = inp["mask"].cpu().numpy().astype(bool)
    rewards = inp["rewards"].cpu().numpy()
    groups = wl.groups_kwargs()
    off = oracle.group_offsets(B, groups.get("samples_per_prompt"), groups.get("group_boundaries"))
    A = oracle.group_advantages(rewards, off, wl.leave_one_out, wl.scale_by_std)
    L, N, w = oracle.sequence_weights(mask, cfg.reduction, cfg.alpha)
    assert np.array_equal(to_np(res.advantages).astype(np.float32).view(np.uint32),
                          A.astype(np.float32).view(np.uint32))
    assert np.array_equal(to_np(res.seq_weight).astype(np.float32).view(np.uint32),
                          w.astype(np.float32).view(np.uint32))
    assert np.array_equal(to_np(res.seq_tokens), L) and int(res.counts[0]) == N

    # properties on every sequence
    glp = to_np(res.tok_logp)
    old = inp["old_logps"].double().cpu().numpy()
    gs = to_np(res.seq_logratio)
    tl = to_np(res.tok_loss)
    tk = to_np(res.tok_kl)
    for i in range(B):
        s_own = math.fsum(glp[i] - old[i]) / max(int(L[i]), 1)
        assert abs(gs[i] - s_own) <= 2.0 ** -23 * abs(s_own) + 1e-12, (i, gs[i], s_own)
        assert np.all(tl[i] == tl[i, 0]), f"{name}: token loss varies along sequence {i}"
    rho = np.exp(gs)
    lo, hi = 1 - cfg.eps_low, 1 + cfg.eps_high
    assert np.any(rho < lo) and np.any(rho > hi) and np.any((rho > lo) & (rho < hi)), rho
    P = tl.sum(axis=1)
    K = tk.sum(axis=1)
    pl = float(np.sum(w * P))
    kl = float(np.sum(w * K))
    for got, want in ((float(res.policy_loss), pl), (float(res.kl), kl),
                      (float(res.loss), pl + wl.beta * kl)):
        assert abs(got - want) <= 2e-7 * max(abs(want), 1e-30) + 1e-12, (got, want)
    assert np.allclose(to_np(res.seq_policy), P, rtol=1e-6, atol=1e-9)
    assert np.allclose(to_np(res.seq_kl), K, rtol=1e-6, atol=1e-9)

    # whole sequences against the oracle: the first, the last and the first
    # one the kernel reports clipped (so that branch is checked too)
    clip_gpu = ((A > 0) & (rho > hi)) | ((A < 0) & (rho < lo))
    assert clip_gpu.any() and not clip_gpu.all()
    picks = sorted({0, B - 1, int(np.nonzero(clip_gpu)[0][0])})
    rng = np.random.default_rng(5)
    for i in picks:
        announce(f"{name}: sequence {i} through the oracle ({T} rows)")
        acc, sq, ids = _oracle_sequence(inp, i, A, L, w, cfg)
        assert np.all(np.abs(glp[i] - acc["logp"]) <= LOGP_ABS_ERR), (name, i)
        s = float(sq["seq_logratio"][0])
        assert abs(gs[i] - s) <= SEQ_ABS_ERR + 2.0 ** -23 * abs(s), (name, i, gs[i], s)
        _, l_c, _, clip_c = oracle.gspo_terms(np.array([s]), A[i:i + 1], cfg)
        flags = {bool(clip_c[0])}
        dl = 0.0
        for ds in (SEQ_ABS_ERR, -SEQ_ABS_ERR):
            _, l_p, _, clip_p = oracle.gspo_terms(np.array([s + ds]), A[i:i + 1], cfg)
            flags.add(bool(clip_p[0]))
            dl = max(dl, abs(float(l_p[0] - l_c[0])))
        lb = dl + 2.0 ** -22 * abs(float(l_c[0])) + 1e-30
        assert np.all(np.abs(tl[i] - sq["loss"]) <= lb), (name, i, tl[i, 0], sq["loss"][0])
        kb = 2 * LOGP_ABS_ERR * np.abs(np.expm1(acc["d"])) + 2.0 ** -22 * acc["kl"] + 1e-12
        assert np.all(np.abs(tk[i] - acc["kl"]) <= kb), (name, i)
        sub = SimpleNamespace(seq_logratio=np.array([s]), advantages=A[i:i + 1],
                              seq_tokens=L[i:i + 1], seq_weight=w[i:i + 1],
                              tok=dict(d=acc["d"][None], dkl=acc["dkl"][None]))
        br = seq_branches(sub, cfg, np.ones((1, T), dtype=bool), {}, groups, BF16_BASE)
        G0 = br[2][0][0]
        assert np.allclose(G0, sq["gpol"] + w[i] * (cfg.beta * acc["dkl"]), rtol=1e-14, atol=0)
        ts = sorted({0, T - 1} | set(int(v) for v in rng.integers(0, T, 6)))
        for t in ts:
            g = grad[i, t].double().cpu().numpy()
            x = inp["policy"][i, t].float().cpu().numpy()
            check_grad_row(g, x, ids[t], (0, t), br, "bf16", f"{name} seq {i}")
        if len(flags) == 1:
            assert flags == {bool(clip_gpu[i])}, (name, i, flags)
        print(f"  sequence {i}: s={s:.6f} clipped={sorted(flags)}", flush=True)

    announce(f"{name}: row sums")
    assert_grad_rows_sum_to_zero(grad.view(B * T, V))
    announce(f"{name}: run 2")
    _rerun_bitwise(gpu_lib, inp, grad, res, gkw, None)


@pytest.mark.parametrize("kw", [dict(pg_loss="gspo", reduction="sequence_mean"),
                                dict(pg_loss="real")], ids=_id)
def test_fullsize_headline_seqlevel_whole(gpu_lib, kw):
    """GSPO and REAL at V = 151,936 compared whole: every token's log-prob,
    loss and KL, every s_i and per-sequence total, the scalars and every
    gradient row, against the oracle streamed over all 65,536 rows."""
    wl = WORKLOADS["logits_v151936"]
    obj = dict(kw)
    red = obj.pop("reduction", None)
    name = f"full size logits_v151936 {_id(kw)} whole"
    B, T, V = wl.B, wl.T, wl.V
    announce(f"{name}: generating")
    inp = make_logits_inputs(wl, device=DEV, seed=0)
    inp["old_logps"] = shift_by_sequence(inp["old_logps"], seed=0, spread=0.4)
    gkw = gpu_kwargs(wl, red, **obj)
    grad = torch.empty((B, T, V), dtype=torch.bfloat16, device=DEV)
    announce(f"{name}: run")
    res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"],
                                    inp["old_logps"], inp["rewards"], inp["mask"], grad_out=grad,
                                    per_token=True, **gkw)
    torch.cuda.synchronize()
    assert int(res.status[0]) == 0
    cfg = cfg_from(wl, red, **obj)
    groups = wl.groups_kwargs()
    mask = inp["mask"].cpu().numpy().astype(bool)
    ref, st = stream_oracle(inp, grad, wl, cfg, groups, announce=announce)
    announce(f"{name}: oracle done, {st}")
    h = dict(old_logps=inp["old_logps"].cpu().numpy())
    compare_exact_parts(res, ref, name)
    glp = to_np(res.tok_logp)
    assert np.all(np.abs(glp - ref.tok["logp"])[mask] <= LOGP_ABS_ERR), name + " tok_logp"
    amb_seq = compare_seq_outputs(res, ref, cfg, mask, h, groups, 1e-4, name)
    br = seq_branches(ref, cfg, mask, h, groups, BF16_BASE)
    clipped = int(res.counts[1])
    assert abs(clipped - ref.clipped) <= int(br[0].sum()), (clipped, ref.clipped)
    announce(f"{name}: clipped gpu={clipped} oracle={ref.clipped}, sequences at a bound {amb_seq}")
