"""Whole-batch oracle comparison at full size.

The fp64 oracle runs over every active row of a full-size logits batch, a
chunk of rows at a time on host threads (oracle.grpo_loss_rows with a thread
pool's map): rows are gathered on the GPU, copied to the host in their
storage type and widened there, and each chunk's oracle gradient rows are
compared with the GPU's rows as they are produced, so no [B, T, V] host array
is ever held.  Rows that miss the plain per-element bar are re-checked once
the whole batch's per-token values are known: rows at a branch point may
match any candidate G, ill-conditioned rows are held to their propagated
error bound (tests/_parity.py states both refinements).
"""

from __future__ import annotations

import os
import threading
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
from _parity import GRAD16_BAR, check_grad_row, seq_branches, token_branches


def host_workers():
    """Host threads for the oracle: the CPUs this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _to_host_f32(rows):
    """[n, V] device rows -> float32 numpy (16-bit storage widened exactly)."""
    h = rows.cpu()
    if h.dtype == torch.bfloat16:
        u = h.view(torch.int16).numpy().view(np.uint16)
        return (u.astype(np.uint32) << 16).view(np.float32)
    return h.float().numpy()


def _gdt_name(dtype):
    return {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[dtype]


def stream_oracle(inp, grad, wl, cfg, groups, *, chunk=32, workers=None, announce=print,
                  gen_logps=None):
    """Runs the oracle over the whole batch and compares every active gradient
    row.  Returns (oracle result without grad, stats).  ``grad`` is the GPU
    gradient [B, T, V] (or None to skip the gradient); ``gen_logps`` the
    host [B, T] generating log-probs of the off-policy weight, if any.  For
    the sequence-level losses the gradient rows come from the oracle's second
    pass, once every sequence's log-ratio is known."""
    B, T, V = inp["policy"].shape
    dev = inp["policy"].device
    pol = inp["policy"].reshape(B * T, V)
    ref = None if inp.get("ref") is None else inp["ref"].reshape(B * T, V)
    g2 = None if grad is None else grad.reshape(B * T, V)
    gdt = None if grad is None else _gdt_name(grad.dtype)
    base, floor = GRAD16_BAR.get(gdt, (None, None))
    mask = inp["mask"].cpu().numpy().astype(bool)
    n_active = int(mask.sum())
    lock = threading.Lock()
    state = dict(rows=0, failed=[], max_err=0.0, max_ref=0.0, next_report=0.1, t0=time.time())

    def fetch(ii, tt):
        idx = torch.from_numpy((ii * T + tt).astype(np.int64)).to(dev)
        x = _to_host_f32(pol.index_select(0, idx))
        y = None if ref is None else _to_host_f32(ref.index_select(0, idx))
        return x, y

    def sink(ii, tt, rows):
        idx = torch.from_numpy((ii * T + tt).astype(np.int64)).to(dev)
        g = _to_host_f32(g2.index_select(0, idx)).astype(np.float64)
        err = np.abs(g - rows)
        if base is not None:
            with np.errstate(invalid="ignore"):
                lim = np.where(np.abs(rows) > 0, base * np.abs(rows), 0.0) + floor
            bad = ~np.all(err <= lim, axis=1)
        else:
            bad = np.zeros(len(ii), dtype=bool)
        with lock:
            state["max_err"] = max(state["max_err"], float(err.max(initial=0.0)))
            state["max_ref"] = max(state["max_ref"], float(np.abs(rows).max(initial=0.0)))
            state["failed"].extend((int(i), int(t)) for i, t in zip(ii[bad], tt[bad]))
            state["rows"] += len(ii)
            if state["rows"] >= state["next_report"] * n_active:
                announce(f"  oracle rows {state['rows']}/{n_active} "
                         f"({time.time() - state['t0']:.0f} s)")
                state["next_report"] += 0.1

    h_ids = inp["action_ids"].cpu().numpy()
    h_old = inp["old_logps"].cpu().numpy()
    h_rew = inp["rewards"].cpu().numpy()
    w = workers or host_workers()
    announce(f"  oracle over {n_active} active rows on {w} host threads")
    with ThreadPoolExecutor(max_workers=w) as ex:
        res = oracle.grpo_loss_rows(fetch, (B, T, V), h_ids, h_old, mask, h_rew, groups=groups,
                                    cfg=cfg, have_ref=ref is not None, row_chunk=chunk,
                                    gen_logps=gen_logps,
                                    grad_sink=None if grad is None else sink, map_chunks=ex.map)
    stats = dict(rows=state["rows"], recheck=len(state["failed"]), seconds=time.time() - state["t0"],
                 workers=w)
    if grad is None:
        return res, stats
    if base is None:
        # float32 gradient: max|dg| <= 1e-5 max|g| over the whole batch
        assert state["max_err"] <= 1e-5 * state["max_ref"], (state["max_err"], state["max_ref"])
        return res, stats
    # rows that missed the plain bar: branch candidates and propagated bounds
    if state["failed"]:
        if cfg.pg_loss in oracle.SEQUENCE_PG:
            h = dict(old_logps=h_old, gen_logps=gen_logps)
            branches = seq_branches(res, cfg, mask, h, groups, base)
        else:
            branches = token_branches(res, cfg, mask, base)
        for (i, t) in state["failed"]:
            r = i * T + t
            x = _to_host_f32(pol[r:r + 1])[0]
            g = _to_host_f32(g2[r:r + 1])[0].astype(np.float64)
            check_grad_row(g, x, int(h_ids[i, t]), (i, t), branches, gdt, what=f"row ({i},{t})")
    return res, stats


def masked_rows_zero(grad, mask):
    """Every masked row of the GPU gradient is exactly zero (checked on the GPU)."""
    B, T, V = grad.shape
    g2 = grad.reshape(B * T, V)
    m = mask.reshape(-1).to(torch.bool)
    idx = torch.nonzero(~m).reshape(-1)
    for s in range(0, idx.numel(), 4096):
        blk = g2.index_select(0, idx[s:s + 4096])
        if bool((blk != 0).any()):
            return False
    return True
