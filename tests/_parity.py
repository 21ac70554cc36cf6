"""Comparison helpers for the HIP path against the fp64 oracle.

Tolerances (stated by the loss path's acceptance criteria, made concrete):
  * advantages, per-sequence weights, token counts: bit-exact (the GPU computes
    them in binary64 in the defining order and rounds once to float32);
  * float32 logits: loss relative error <= 1e-5, gradient
    max|dg| <= 1e-5 * max|g|;
  * bf16 logits (oracle fed the same bf16 values): loss relative error
    <= 1e-4, gradient |dg| <= 2^-7 |g| per element, with an absolute floor of
    2^-126 (below it bf16 has no relative precision).
Two refinements follow from the arithmetic, and every use is counted:
  * clip-ambiguous tokens: when the oracle's ratio lies within the float32
    log-prob error of a clip bound, either side is a correct result, so the
    row's gradient may match the clipped or the unclipped branch;
  * ill-conditioned rows: when G (d loss / d logp) cancels, e.g. A = 0 and
    d close to 0, float32 log-probs (absolute error about 1e-6 at |logp| ~ 12)
    cannot give G to 2^-7; such a row is compared at its propagated error
    bound instead.
"""

from __future__ import annotations

import math

import numpy as np
import torch

import oracle

# absolute error budget of a float32 log-prob computed over a long row
LOGP_ABS_ERR = 2.0 ** -19


def f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def assert_bits_equal(gpu, ref64, what):
    g = f32_bits(gpu)
    r = f32_bits(np.asarray(ref64, dtype=np.float64).astype(np.float32))
    bad = np.nonzero(g != r)[0]
    assert bad.size == 0, (f"{what}: {bad.size} values differ in bits, first at {bad[:5]}: "
                           f"gpu={np.asarray(gpu)[bad[:5]]} oracle={np.asarray(ref64)[bad[:5]]}")


def to_np(t):
    return t.detach().double().cpu().numpy() if t.dtype.is_floating_point else t.detach().cpu().numpy()


def cfg_from(wl, reduction=None):
    red = reduction or wl.reductions[0]
    return oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
                             reduction=red, alpha=wl.alpha if red == "length_alpha" else None)


def gpu_kwargs(wl, reduction=None):
    red = reduction or wl.reductions[0]
    kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=red,
              alpha=wl.alpha if red == "length_alpha" else None)
    kw.update(wl.groups_kwargs())
    return kw


def oracle_groups(wl):
    return wl.groups_kwargs()


def host_inputs(inp):
    """Host float64 / int views of a batch (bf16 values exactly as the GPU sees them)."""
    out = {}
    for k, v in inp.items():
        if v.dtype in (torch.bfloat16, torch.float32):
            out[k] = v.detach().float().cpu().numpy()
        else:
            out[k] = v.detach().cpu().numpy()
    return out


def ambiguous_rows(ref, cfg, mask):
    """Active slots whose oracle ratio is within float32 reach of a clip bound."""
    rho = ref.tok["rho"]
    band = rho * 4.0 * LOGP_ABS_ERR + 1e-7
    lo, hi = 1.0 - cfg.eps_low, 1.0 + cfg.eps_high
    A = ref.advantages[:, None]
    amb = ((np.abs(rho - hi) <= band) & (A > 0)) | ((np.abs(rho - lo) <= band) & (A < 0))
    return amb & mask


def g_rel_tolerance(ref, cfg, base):
    """Per-slot relative tolerance of G: max(base, propagated float32 error)."""
    A = ref.advantages[:, None]
    w = ref.seq_weight[:, None]
    rho = ref.tok["rho"]
    ed = np.exp(ref.tok["d"])
    G = ref.tok["G"]
    dG = np.abs(w) * (np.abs(A) * rho + 2.0 * cfg.beta * ed) * LOGP_ABS_ERR * 2.0
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(G != 0, dG / np.abs(G), np.inf)
    return np.maximum(base, rel), rel > base


def alt_G(ref, cfg):
    """G with the clip decision flipped (for ambiguous slots)."""
    A = ref.advantages[:, None]
    w = ref.seq_weight[:, None]
    rho = ref.tok["rho"]
    clipped = ref.tok["clipped"]
    dloss_alt = np.where(clipped, -A * rho, 0.0)
    return w * (dloss_alt + cfg.beta * ref.tok["dkl"])


def compare_scalars(res, ref, loss_rtol, what=""):
    loss = float(res.loss)
    kappa = (np.sum(ref.seq_weight * np.abs(ref.seq_policy)) + 1e-300) / max(abs(ref.loss), 1e-300)
    rel = abs(loss - ref.loss) / max(abs(ref.loss), 1e-300)
    assert rel <= loss_rtol, f"{what} loss gpu={loss!r} oracle={ref.loss!r} rel={rel:.3g} kappa={kappa:.3g}"
    # policy_loss and kl: relative to the weighted absolute sums they are made of
    scale_p = float(np.sum(ref.seq_weight * np.abs(ref.tok["loss"]).sum(axis=1))) + 1e-30
    scale_k = float(np.sum(ref.seq_weight * np.abs(ref.tok["kl"]).sum(axis=1))) + 1e-30
    assert abs(float(res.policy_loss) - ref.policy_loss) <= loss_rtol * scale_p, what
    assert abs(float(res.kl) - ref.kl) <= loss_rtol * scale_k, what
    # per-sequence totals: the relative bound plus the float32 log-prob error
    # propagated through each token (d l/d logp = -A rho, d k3/d d = e^d - 1)
    sp = to_np(res.seq_policy)
    sk = to_np(res.seq_kl)
    A = ref.advantages[:, None]
    prop_p = (np.abs(A) * ref.tok["rho"] * (ref.tok["dloss"] != 0)).sum(axis=1) * LOGP_ABS_ERR
    prop_k = (np.abs(np.expm1(ref.tok["d"]))).sum(axis=1) * 2 * LOGP_ABS_ERR
    tp = loss_rtol * np.abs(ref.tok["loss"]).sum(axis=1) + prop_p + 1e-30
    tk = loss_rtol * np.abs(ref.tok["kl"]).sum(axis=1) + prop_k + 1e-30
    ep = np.abs(sp - ref.seq_policy)
    ek = np.abs(sk - ref.seq_kl)
    assert np.all(ep <= tp), f"{what} seq_policy worst {np.max(ep / tp):.3g}x of bound"
    assert np.all(ek <= tk), f"{what} seq_kl worst {np.max(ek / tk):.3g}x of bound"
    return rel, kappa


def compare_exact_parts(res, ref, what=""):
    assert_bits_equal(to_np(res.advantages), ref.advantages, what + " advantages")
    assert_bits_equal(to_np(res.seq_weight), ref.seq_weight, what + " seq_weight")
    assert np.array_equal(to_np(res.seq_tokens), ref.seq_tokens), what + " seq_tokens"
    counts = to_np(res.counts)
    assert int(counts[0]) == ref.num_tokens, what + " N"
    return counts


def compare_logits_grad(grad_gpu, ref, cfg, mask, bf16, what=""):
    """grad_gpu: float64 numpy [B, T, V]; ref: oracle result with grad."""
    g = grad_gpu
    r = ref.grad
    amb = ambiguous_rows(ref, cfg, mask)
    stats = dict(ambiguous=int(amb.sum()), illcond=0, rows=int(mask.sum()))
    # masked rows: exactly zero
    assert np.all(g[~mask] == 0.0), what + " masked rows must be zero"
    if bf16:
        tol, ill = g_rel_tolerance(ref, cfg, 2.0 ** -7)
        stats["illcond"] = int((ill & mask).sum())
        floor = 2.0 ** -126
        err = np.abs(g - r)
        with np.errstate(invalid="ignore"):
            lim = np.where(np.abs(r) > 0, tol[..., None] * np.abs(r), 0.0) + floor
        ok = err <= lim
        bad_rows = ~ok.all(axis=-1) & mask
    else:
        gmax = float(np.max(np.abs(r))) if r.size else 0.0
        err = np.abs(g - r)
        ok = err <= 1e-5 * gmax + 1e-30
        bad_rows = ~ok.all(axis=-1) & mask
    # ambiguous rows may match the flipped branch instead
    for (i, t) in zip(*np.nonzero(bad_rows & amb)):
        G = ref.tok["G"][i, t]
        Ga = alt_G(ref, cfg)[i, t]
        if G != 0:
            alt = r[i, t] * (Ga / G)
        else:
            continue
        if bf16:
            ok_alt = np.all(np.abs(g[i, t] - alt) <= 2.0 ** -7 * np.abs(alt) + 2.0 ** -126)
        else:
            ok_alt = np.all(np.abs(g[i, t] - alt) <= 1e-5 * float(np.max(np.abs(r))) + 1e-30)
        if ok_alt:
            bad_rows[i, t] = False
    nbad = int(bad_rows.sum())
    if nbad:
        i, t = [int(v[0]) for v in np.nonzero(bad_rows)]
        e = np.abs(g[i, t] - r[i, t])
        k = int(np.argmax(e / (np.abs(r[i, t]) + 1e-300)))
        raise AssertionError(
            f"{what}: {nbad} gradient rows out of tolerance; first ({i},{t}) v={k}: "
            f"gpu={g[i, t, k]!r} oracle={r[i, t, k]!r} G={ref.tok['G'][i, t]!r} "
            f"rho={ref.tok['rho'][i, t]!r} A={ref.advantages[i]!r} d={ref.tok['d'][i, t]!r}")
    return stats
