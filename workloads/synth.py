"""Seeded synthetic inputs for the GRPO loss workloads.

This module only draws random inputs; it holds none of the loss arithmetic.
The one place it touches the policy's distribution is input synthesis itself:
cached behaviour log-probs are the policy's log-softmax at the taken token
plus noise (computed with torch's own logsumexp), and "sampled" action ids
use the Gumbel-max trick.  Both sides of every parity test receive the same
tensors, so nothing here can hide a mistake in either of them.

Notation: the workload descriptions write N(0, s) with s a variance (they
write N(0, 2^2) for a standard deviation of 2), so N(0, 0.1) is drawn with
std sqrt(0.1) and N(0, 0.05) with std sqrt(0.05).

Workloads (sizes as stated by the GRPO loss workload list):
  tiny_logits        B=8 (2x4), T=16, V=32, fp32, ragged lengths 1..16
  token_loss         B=1024 (64x16), T=4096, per-token fp32 log-probs
  logits_v32000      B=64 (8x8), T=1024, V=32000, bf16, ragged 64..1024
  logits_v151936     B=32 (4x8), T=2048, V=151936, bf16 + one +8 spike per row,
                     ids sampled from the policy softmax, full mask
  logits_csr_v128256 B=96 in 12 CSR groups of {4,8,16}, T=1024, V=128256,
                     bf16, leave-one-out + std, one all-equal group,
                     asymmetric clip, ragged 1..1024, three reductions
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class LogitsWorkload:
    name: str
    group_sizes: tuple            # sizes of the reward groups, in order
    T: int
    V: int
    dtype: str                    # "f32" | "bf16" | "f16"
    logit_std: float
    ref_noise_std: float
    old_noise_std: float
    reward_p: float               # Bernoulli probability of reward 1
    len_range: tuple | None       # (lo, hi) prefix lengths, None = full mask
    ids: str = "uniform"          # "uniform" | "softmax"
    spike: float | None = None    # add this to one random id per row
    csr: bool = False             # pass groups as CSR boundaries
    degenerate_groups: int = 0    # force this many all-equal groups; redraw the others
    eps_low: float = 0.2
    eps_high: float = 0.2
    beta: float = 0.04
    reductions: tuple = ("token_mean",)
    alpha: float | None = None
    leave_one_out: bool = False
    scale_by_std: bool = True

    @property
    def B(self):
        return int(sum(self.group_sizes))

    def scaled(self, *, T=None, V=None, prompts=None):
        """Same recipe at a smaller size (for parity runs the oracle finishes fast)."""
        gs = self.group_sizes if prompts is None else tuple(self.group_sizes[:prompts])
        T2 = self.T if T is None else T
        lr = self.len_range
        if lr is not None and T is not None:
            # keep the same length mix relative to T
            lo = max(1, int(round(lr[0] * T2 / self.T)))
            lr = (min(lo, T2), T2)
        return replace(self, T=T2, V=self.V if V is None else V, group_sizes=gs,
                       len_range=lr, name=f"{self.name}[B{sum(gs)},T{T2},V{self.V if V is None else V}]")

    def groups_kwargs(self):
        d = dict(leave_one_out=self.leave_one_out, scale_by_std=self.scale_by_std)
        if self.csr:
            d["group_boundaries"] = [int(v) for v in np.concatenate([[0], np.cumsum(self.group_sizes)])]
        else:
            assert len(set(self.group_sizes)) == 1
            d["samples_per_prompt"] = int(self.group_sizes[0])
        return d


@dataclass(frozen=True)
class TokenWorkload:
    name: str
    group_size: int
    num_groups: int
    T: int
    old_noise_std: float
    ref_noise_std: float
    reward_p: float
    len_range: tuple | None
    eps_low: float = 0.2
    eps_high: float = 0.2
    beta: float = 0.04
    reduction: str = "sequence_mean"

    @property
    def B(self):
        return self.group_size * self.num_groups


def _csr_sizes(total, choices, count, seed):
    """`count` group sizes drawn i.i.d. from `choices`, all redrawn until they
    sum to `total` (seeded)."""
    rng = np.random.default_rng([seed, 7])
    while True:
        sizes = tuple(int(v) for v in rng.choice(choices, size=count))
        if sum(sizes) == total:
            return sizes


WORKLOADS = {
    "tiny_logits": LogitsWorkload(
        name="tiny_logits", group_sizes=(4, 4), T=16, V=32, dtype="f32", logit_std=1.0,
        ref_noise_std=math.sqrt(0.1), old_noise_std=math.sqrt(0.05), reward_p=0.5,
        len_range=(1, 16)),
    "logits_v32000": LogitsWorkload(
        name="logits_v32000", group_sizes=(8,) * 8, T=1024, V=32000, dtype="bf16",
        logit_std=2.0, ref_noise_std=math.sqrt(0.1), old_noise_std=math.sqrt(0.05),
        reward_p=0.3, len_range=(64, 1024)),
    "logits_v151936": LogitsWorkload(
        name="logits_v151936", group_sizes=(8,) * 4, T=2048, V=151936, dtype="bf16",
        logit_std=3.0, ref_noise_std=math.sqrt(0.1), old_noise_std=math.sqrt(0.05),
        reward_p=0.5, len_range=None, ids="softmax", spike=8.0),
    "logits_csr_v128256": LogitsWorkload(
        name="logits_csr_v128256", group_sizes=_csr_sizes(96, (4, 8, 16), 12, 0), T=1024,
        V=128256, dtype="bf16", logit_std=2.0, ref_noise_std=math.sqrt(0.1),
        old_noise_std=math.sqrt(0.05), reward_p=0.5, len_range=(1, 1024), csr=True,
        degenerate_groups=1, eps_low=0.2, eps_high=0.28, beta=0.01,
        reductions=("token_mean", "sequence_mean", "length_alpha"), alpha=0.5,
        leave_one_out=True, scale_by_std=True),
}

TOKEN_WORKLOADS = {
    "token_loss_full": TokenWorkload(
        name="token_loss_full", group_size=16, num_groups=64, T=4096,
        old_noise_std=math.sqrt(0.05), ref_noise_std=math.sqrt(0.1), reward_p=0.5,
        len_range=None),
    "token_loss_ragged": TokenWorkload(
        name="token_loss_ragged", group_size=16, num_groups=64, T=4096,
        old_noise_std=math.sqrt(0.05), ref_noise_std=math.sqrt(0.1), reward_p=0.5,
        len_range=(1, 4096)),
}


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _prefix_mask(B, T, len_range, g, device):
    if len_range is None:
        return torch.ones((B, T), dtype=torch.bool, device=device)
    lo, hi = len_range
    lens = torch.randint(lo, hi + 1, (B,), generator=g, device=device)
    return torch.arange(T, device=device)[None, :] < lens[:, None]


def _rewards(group_sizes, p, degenerate, g, device):
    """Bernoulli(p) rewards in {0, 1}.  With ``degenerate`` > 0 the first
    ``degenerate`` groups are forced all-equal (all 1) and every other group is
    redrawn until it holds both values."""
    out = []
    for k, n in enumerate(group_sizes):
        if k < degenerate:
            out.append(torch.ones(n, device=device))
            continue
        while True:
            r = (torch.rand(n, generator=g, device=device) < p).float()
            if degenerate == 0 or (0 < float(r.sum()) < n):
                break
        out.append(r)
    return torch.cat(out)


def make_logits_inputs(wl: LogitsWorkload, device="cpu", seed=0, row_chunk=None):
    """Draw one batch of inputs.  Returns a dict of tensors on ``device``:
    policy, ref [B, T, V] (fp32, bf16 or fp16), action_ids [B, T] int64,
    old_logps [B, T] fp32, rewards [B] fp32, mask [B, T] bool.
    Large batches are drawn in row chunks so no fp32 temporary exceeds about
    1 GiB."""
    B, T, V = wl.B, wl.T, wl.V
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.dtype]
    g = _gen(device, seed)
    rows = B * T
    if row_chunk is None:
        row_chunk = max(1, min(rows, (1 << 28) // V))
    policy = torch.empty((rows, V), dtype=dt, device=device)
    ref = torch.empty((rows, V), dtype=dt, device=device)
    ids = torch.empty(rows, dtype=torch.int64, device=device)
    old = torch.empty(rows, dtype=torch.float32, device=device)
    for s in range(0, rows, row_chunk):
        e = min(rows, s + row_chunk)
        n = e - s
        x = torch.randn((n, V), generator=g, device=device) * wl.logit_std
        if wl.spike is not None:
            sp = torch.randint(0, V, (n, 1), generator=g, device=device)
            x.scatter_add_(1, sp, torch.full((n, 1), wl.spike, device=device))
        xp = x.to(dt)
        policy[s:e] = xp
        xf = xp.float()
        y = xf + torch.randn((n, V), generator=g, device=device) * wl.ref_noise_std
        ref[s:e] = y.to(dt)
        del y
        if wl.ids == "softmax":
            u = torch.rand((n, V), generator=g, device=device).clamp_min_(1e-30)
            gumbel = -torch.log(-torch.log(u))
            a = torch.argmax(xf + gumbel, dim=1)
            del u, gumbel
        else:
            a = torch.randint(0, V, (n,), generator=g, device=device)
        ids[s:e] = a
        lse = torch.logsumexp(xf, dim=1)
        old[s:e] = xf.gather(1, a[:, None])[:, 0] - lse + \
            torch.randn(n, generator=g, device=device) * wl.old_noise_std
        del x, xf
    mask = _prefix_mask(B, T, wl.len_range, g, device)
    rewards = _rewards(wl.group_sizes, wl.reward_p, wl.degenerate_groups, g, device)
    return dict(policy=policy.view(B, T, V), ref=ref.view(B, T, V), action_ids=ids.view(B, T),
                old_logps=old.view(B, T), rewards=rewards, mask=mask)


def make_token_inputs(wl: TokenWorkload, device="cpu", seed=0, B=None, T=None):
    """Per-token inputs: logp = -Exp(1), old = logp + noise, ref = logp + noise."""
    B = wl.B if B is None else B
    T = wl.T if T is None else T
    g = _gen(device, seed)
    u = torch.rand((B, T), generator=g, device=device).clamp_min_(1e-12)
    logp = torch.log(u)                       # -Exp(1)
    old = logp + torch.randn((B, T), generator=g, device=device) * wl.old_noise_std
    ref = logp + torch.randn((B, T), generator=g, device=device) * wl.ref_noise_std
    lr = None if wl.len_range is None else (min(wl.len_range[0], T), min(wl.len_range[1], T))
    mask = _prefix_mask(B, T, lr, g, device)
    rewards = (torch.rand(B, generator=g, device=device) < wl.reward_p).float()
    return dict(logp=logp.float(), old_logps=old.float(), ref_logp=ref.float(),
                rewards=rewards, mask=mask)


def make_gen_logps(old_logps, seed=0, std=0.3):
    """Log-probs of a generating policy a little older than the one behind
    old_logps: old + N(0, std^2) per token, seeded."""
    g = _gen(old_logps.device, seed + 7919)
    noise = torch.randn(old_logps.shape, generator=g, device=old_logps.device) * std
    return (old_logps.float() + noise).contiguous()


def shift_by_sequence(t, seed=0, spread=0.4):
    """t [B, T] plus one offset per sequence drawn from U(-spread, spread),
    seeded: moves whole sequences' log-ratios across a clip band."""
    g = _gen(t.device, seed + 104729)
    off = (torch.rand((t.shape[0], 1), generator=g, device=t.device) * 2.0 - 1.0) * spread
    return (t.float() + off).contiguous()


def poison_masked(inputs, V=None):
    """Write NaN/+-Inf into every masked slot's logits rows and old log-probs
    and out-of-range ids into masked action ids (masked slots must never be
    read).  Works on the dicts returned above; returns a new dict."""
    out = dict(inputs)
    m = inputs["mask"]
    inv = ~m
    if "policy" in inputs:
        pol = inputs["policy"].clone()
        ref = inputs["ref"].clone()
        pol[inv] = float("nan")
        ref[inv] = float("inf")
        out["policy"], out["ref"] = pol, ref
        ids = inputs["action_ids"].clone()
        ids[inv] = -1 if V is None else V + 5
        out["action_ids"] = ids
    else:
        for k, val in (("logp", float("nan")), ("ref_logp", float("-inf"))):
            t = inputs[k].clone()
            t[inv] = val
            out[k] = t
    old = inputs["old_logps"].clone()
    old[inv] = float("-inf")
    out["old_logps"] = old
    return out
