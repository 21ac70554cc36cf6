"""The oracle's row-streaming form (grpo_loss_rows) is the in-memory logits
path with the rows fetched a chunk at a time: over the same inputs it gives
the same bits, whatever the chunk size and whatever order a thread pool
evaluates the chunks in."""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from workloads import WORKLOADS, make_logits_inputs


def _inputs(seed=0):
    wl = WORKLOADS["tiny_logits"]
    inp = make_logits_inputs(wl, device="cpu", seed=seed)
    return wl, {k: v.float().numpy() if v.is_floating_point() else v.numpy() for k, v in inp.items()}


@pytest.mark.parametrize("cfg", [
    oracle.LossConfig(eps_low=0.2, eps_high=0.28, beta=0.04),
    oracle.LossConfig(beta=0.04, reduction="length_alpha", alpha=0.5),
    oracle.LossConfig(beta=0.04, pg_loss="gspo", reduction="sequence_mean"),
], ids=["clip", "alpha", "gspo"])
@pytest.mark.parametrize("chunk", [1, 7, 4096])
def test_rows_form_matches_in_memory(cfg, chunk):
    wl, h = _inputs()
    groups = wl.groups_kwargs()
    want = oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"],
                                    h["mask"], h["rewards"], groups=groups, cfg=cfg)
    B, T, V = h["policy"].shape
    grad = np.full((B, T, V), np.nan)
    calls = []

    def fetch(ii, tt):
        calls.append(len(ii))
        return h["policy"][ii, tt], h["ref"][ii, tt]

    def sink(ii, tt, rows):
        grad[ii, tt] = rows

    with ThreadPoolExecutor(4) as ex:
        got = oracle.grpo_loss_rows(fetch, (B, T, V), h["action_ids"], h["old_logps"], h["mask"],
                                    h["rewards"], groups=groups, cfg=cfg, row_chunk=chunk,
                                    grad_sink=sink, map_chunks=ex.map)
    assert max(calls) <= chunk
    for name in ("loss", "policy_loss", "kl", "clipped", "num_tokens"):
        assert getattr(got, name) == getattr(want, name), name
    for name in ("seq_policy", "seq_kl", "seq_weight", "advantages"):
        assert np.array_equal(getattr(got, name), getattr(want, name)), name
    for name, v in want.tok.items():
        assert np.array_equal(got.tok[name], v), name
    m = h["mask"].astype(bool)
    assert np.array_equal(grad[m], want.grad[m])
    # masked rows are never handed to the sink
    assert np.all(np.isnan(grad[~m]))
    # the log-sum-exp of every active row, as the row's log-softmax defines it
    x = h["policy"].astype(np.float64)
    lse = np.log(np.sum(np.exp(x - x.max(axis=-1, keepdims=True)), axis=-1)) + x.max(axis=-1)
    assert np.allclose(got.tok["lse"][m], lse[m], rtol=0, atol=1e-12)
    assert np.all(got.tok["lse"][~m] == 0.0)
