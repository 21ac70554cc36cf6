"""The entry points are capturable in a HIP graph: a call enqueues kernel
launches only (no host copy, no memset, no synchronisation), with uniform
or CSR groups (CSR offsets travel as kernel arguments).  Every replay is
checked bitwise against the eager result, with eager work,
synchronisations and input updates between replays."""

import math

import pytest
import torch

from _parity import gpu_kwargs
from workloads import TOKEN_WORKLOADS, LogitsWorkload, make_logits_inputs, make_token_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    return g


@pytest.mark.parametrize("groups", ["uniform", "csr"])
def test_token_loss_graph_replays(gpu_lib, groups):
    rpl = gpu_lib
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    announce(f"graph token loss {groups}")
    a = make_token_inputs(wl, device=DEV, seed=31, B=64, T=512)
    b = make_token_inputs(wl, device=DEV, seed=32, B=64, T=512)
    kw = dict(samples_per_prompt=16, reduction="sequence_mean", per_token=True)
    if groups == "csr":
        # 30 CSR groups of 2 and 4 samples summing to B = 64
        sizes = [2] * 27 + [4] * 2 + [2]
        kw = dict(group_boundaries=[0] + [int(v) for v in torch.tensor(sizes).cumsum(0)],
                  reduction="sequence_mean", per_token=True, leave_one_out=True)
        assert kw["group_boundaries"][-1] == 64
    static = {k: v.clone() for k, v in a.items()}
    box = {}

    def call():
        box["res"] = rpl.grpo_token_loss(static["logp"], static["old_logps"], static["ref_logp"],
                                         static["rewards"], static["mask"], out=box.get("res"),
                                         **kw)

    g = _capture(call)
    res = box["res"]
    eager_a = rpl.grpo_token_loss(a["logp"], a["old_logps"], a["ref_logp"], a["rewards"], a["mask"], **kw)
    eager_b = rpl.grpo_token_loss(b["logp"], b["old_logps"], b["ref_logp"], b["rewards"], b["mask"], **kw)
    torch.cuda.synchronize()
    for rep in range(6):
        src, ref = (a, eager_a) if rep % 2 == 0 else (b, eager_b)
        for k in static:
            static[k].copy_(src[k])
        g.replay()
        # eager work in between, on the same stream and workspace
        junk = rpl.grpo_token_loss(b["logp"], a["old_logps"], b["ref_logp"], a["rewards"], b["mask"], **kw)
        torch.cuda.synchronize()
        for name in ("scalars", "seq_policy", "seq_kl", "advantages", "seq_weight", "grad", "tok_loss"):
            assert torch.equal(_bits(getattr(res, name)), _bits(getattr(ref, name))), (rep, name)
        assert torch.equal(res.counts, ref.counts) and torch.equal(res.status, ref.status)
        del junk


@pytest.mark.parametrize("mode", ["uniform", "csr", "csr_noalloc"])
def test_logits_graph_replays(gpu_lib, mode):
    rpl = gpu_lib
    if mode == "uniform":
        wl = LogitsWorkload(name="graph", group_sizes=(4, 4), T=24, V=12000, dtype="bf16",
                            logit_std=2.0, ref_noise_std=math.sqrt(0.1),
                            old_noise_std=math.sqrt(0.05), reward_p=0.5, len_range=(1, 24))
    else:
        wl = LogitsWorkload(name="graph_csr", group_sizes=(4, 2, 6, 2, 2), T=24, V=12000,
                            dtype="bf16", logit_std=2.0, ref_noise_std=math.sqrt(0.1),
                            old_noise_std=math.sqrt(0.05), reward_p=0.5, len_range=(1, 24),
                            csr=True, leave_one_out=True, reductions=("sequence_mean",))
    entry = rpl.grpo_loss_fwd_bwd_noalloc if mode == "csr_noalloc" else rpl.grpo_loss_fwd_bwd
    announce(f"graph logits {mode}")
    a = make_logits_inputs(wl, device=DEV, seed=41)
    b = make_logits_inputs(wl, device=DEV, seed=42)
    kw = gpu_kwargs(wl)
    static = {k: v.clone() for k, v in a.items()}
    grad = torch.empty_like(static["policy"])
    box = {}

    def call():
        box["res"] = entry(static["policy"], static["ref"], static["action_ids"],
                           static["old_logps"], static["rewards"], static["mask"],
                           grad_out=grad, per_token=True, out=box.get("res"), **kw)

    g = _capture(call)
    res = box["res"]
    refs = []
    for src in (a, b):
        refs.append(rpl.grpo_loss_fwd_bwd(src["policy"], src["ref"], src["action_ids"], src["old_logps"],
                                          src["rewards"], src["mask"], per_token=True, **kw))
    torch.cuda.synchronize()
    for rep in range(6):
        src, ref = (a, refs[0]) if rep % 2 == 0 else (b, refs[1])
        for k in static:
            static[k].copy_(src[k])
        g.replay()
        torch.randn(1000, device=DEV).sum()  # unrelated eager work
        torch.cuda.synchronize()
        assert torch.equal(_bits(grad), _bits(ref.grad)), rep
        for name in ("scalars", "seq_policy", "seq_kl", "tok_logp", "tok_loss", "tok_kl"):
            assert torch.equal(_bits(getattr(res, name)), _bits(getattr(ref, name))), (rep, name)
