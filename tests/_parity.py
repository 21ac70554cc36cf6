"""Comparison helpers for the HIP path against the fp64 oracle.

Tolerances (stated by the loss path's acceptance criteria, made concrete):
  * advantages, per-sequence weights, token counts: bit-exact (the GPU computes
    them in binary64 in the defining order and rounds once to float32);
  * float32 logits: loss relative error <= 1e-5, gradient
    max|dg| <= 1e-5 * max|g|;
  * bf16 logits (oracle fed the same bf16 values): loss relative error
    <= 1e-4, gradient |dg| <= 2^-7 |g| per element, with an absolute floor of
    2^-126 (below it bf16 has no relative precision);
  * f16 logits and gradient: the same loss bound as bf16 (16-bit storage),
    gradient |dg| <= 2^-10 |g| per element (round to nearest even in an
    11-bit significand, plus the float32 error of G), with an absolute floor
    of 2^-24 (the f16 subnormal spacing).
Three refinements follow from the arithmetic, and every use is counted:
  * branch-ambiguous tokens: when the oracle's log-prob or log-ratio lies
    within the float32 error of a branch point of the objective (a clip or
    dual-clip bound, a KL clamp), either side is a correct result, so the
    row's gradient may match any branch reached within that error;
  * ill-conditioned rows: when G (d loss / d logp) cancels, e.g. A = 0 and
    d close to 0, float32 log-probs (absolute error about 1e-6 at |logp| ~ 12)
    cannot give G to 2^-7; such a row is compared at its propagated error
    bound instead;
  * objectives whose value is linear in the log-prob itself (REINFORCE:
    -A logp; CISPO: -A sg(clip(rho)) logp) carry the float32 log-prob error
    (about 2^-19 absolute) into every token's loss at full size, so their
    summed loss is compared at rtol |loss| plus that propagated error.  For
    every other objective, the default clipped surrogate with k3 included,
    the relative bound is enforced outright.
Branch points and error bounds come from the oracle evaluated at perturbed
inputs, so they hold for every objective variant.
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


def cfg_from(wl, reduction=None, **objective):
    red = reduction or wl.reductions[0]
    return oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
                             reduction=red, alpha=wl.alpha if red == "length_alpha" else None,
                             **objective)


def gpu_kwargs(wl, reduction=None, **objective):
    red = reduction or wl.reductions[0]
    kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=red,
              alpha=wl.alpha if red == "length_alpha" else None)
    kw.update(wl.groups_kwargs())
    kw.update(objective)
    return kw


def oracle_groups(wl):
    return wl.groups_kwargs()


def host_inputs(inp):
    """Host float64 / int views of a batch (16-bit values exactly as the GPU sees them)."""
    out = {}
    for k, v in inp.items():
        if v.dtype in (torch.bfloat16, torch.float16, torch.float32):
            out[k] = v.detach().float().cpu().numpy()
        else:
            out[k] = v.detach().cpu().numpy()
    return out


# ---------------------------------------------------------------------------
# Perturbation of the oracle's per-token inputs.  The GPU evaluates the
# objective at a log-prob and a log-ratio d that carry float32 errors; the
# oracle evaluated at logp +- e (d held fixed) and at d +- e (logp held fixed)
# gives, for any objective variant, (a) which tokens sit close enough to a
# branch point (clip bound, dual-clip bound, KL clamp) for either branch to be
# a correct result, (b) the first-order error bound of values and of G.
# ---------------------------------------------------------------------------

def _active(ref):
    # the oracle stores 0 at masked slots; an active slot's ratio is positive
    return ref.tok["rho"] > 0


def _terms_at(ref, cfg, dlogp=0.0, dd=0.0):
    t = ref.tok
    act = _active(ref)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        old = np.where(act, t["logp"] - np.log(np.where(act, t["rho"], 1.0)), 0.0)
        lp = t["logp"] + dlogp
        lref = t["logp"] + t["d"] + dlogp + dd
        keep = None if ref.seq_keep is None else np.broadcast_to(ref.seq_keep[:, None], lp.shape)
        adv = t["adv"] if "adv" in t else ref.advantages[:, None]
        out = oracle.token_terms(lp, old, lref, adv, cfg, t.get("gen"), keep)
    for k, v in out.items():
        out[k] = np.where(act, v, np.zeros_like(v))
    return out


def _G_of(ref, cfg, t):
    return ref.seq_weight[:, None] * (t["dloss"] + cfg.beta * t["dkl"])


def _branch(t):
    return np.stack([t["clipped"], t["dkl"] == 0, t["dloss"] == 0])


def branch_ambiguity(ref, cfg, mask, e_logp=4 * LOGP_ABS_ERR, e_d=4 * LOGP_ABS_ERR):
    """(clip-flag ambiguous [B, T], branch ambiguous [B, T], candidate G list)."""
    center = _terms_at(ref, cfg)
    bc = _branch(center)
    flag = np.zeros(mask.shape, dtype=bool)
    anyb = np.zeros(mask.shape, dtype=bool)
    cands = [_G_of(ref, cfg, center)]
    for a, b in ((e_logp, 0.0), (-e_logp, 0.0), (0.0, e_d), (0.0, -e_d)):
        t = _terms_at(ref, cfg, a, b)
        flag |= t["clipped"] != center["clipped"]
        anyb |= np.any(_branch(t) != bc, axis=0)
        cands.append(_G_of(ref, cfg, t))
    return flag & mask, anyb & mask, cands


def _propagated(ref, cfg, key_fn, e_logp, e_d):
    """First-order error of key_fn(terms) from logp +- e_logp and d +- e_d,
    leaving out perturbations that change the token's branch."""
    center = _terms_at(ref, cfg)
    c = key_fn(center)
    bc = _branch(center)
    tot = np.zeros_like(c)
    for pair in (((e_logp, 0.0), (-e_logp, 0.0)), ((0.0, e_d), (0.0, -e_d))):
        worst = np.zeros_like(c)
        for a, b in pair:
            t = _terms_at(ref, cfg, a, b)
            same = np.all(_branch(t) == bc, axis=0)
            with np.errstate(invalid="ignore"):
                worst = np.maximum(worst, np.where(same, np.abs(key_fn(t) - c), 0.0))
        tot = tot + worst
    return tot


def ambiguous_rows(ref, cfg, mask):
    """Active slots where either branch of the objective is a correct result."""
    return branch_ambiguity(ref, cfg, mask)[1]


def g_rel_tolerance(ref, cfg, base):
    """Per-slot relative tolerance of G: max(base, propagated float32 error)."""
    G = ref.tok["G"]
    dG = _propagated(ref, cfg, lambda t: _G_of(ref, cfg, t), 2 * LOGP_ABS_ERR, 4 * LOGP_ABS_ERR)
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(G != 0, dG / np.abs(G), np.inf)
    # rows with G = 0 are compared at the absolute floor, not counted here
    return np.maximum(base, rel), (rel > base) & (G != 0)


def value_bounds(ref, cfg, e_logp=LOGP_ABS_ERR, e_d=2 * LOGP_ABS_ERR):
    """Per-token propagated float32 error of the policy loss and KL values."""
    pl = _propagated(ref, cfg, lambda t: t["loss"], e_logp, e_d)
    kl = _propagated(ref, cfg, lambda t: t["kl"], e_logp, e_d)
    return pl, kl


# objectives whose per-token value is linear in logp itself, so the float32
# log-prob error enters the loss value undamped: only these may fall back to
# the propagated bound (the value of every other objective depends on logp
# through the ratio or d only)
VALUE_LINEAR_IN_LOGP = ("reinforce", "cispo")


def compare_scalars(res, ref, cfg, loss_rtol, what="", e_logp=LOGP_ABS_ERR,
                    e_d=2 * LOGP_ABS_ERR, allow_propagated=None):
    """Scalars and per-sequence totals.  The loss must meet loss_rtol
    relative to the oracle's loss.  Only when ``allow_propagated`` (default:
    the objective is one of VALUE_LINEAR_IN_LOGP) may a loss outside that
    bound pass at rtol |loss| plus the float32 log-prob error propagated
    through every token; the returned flag and the printed line say when it
    did.  Returns (rel, kappa, propagated)."""
    if allow_propagated is None:
        allow_propagated = cfg.pg_loss in VALUE_LINEAR_IN_LOGP
    loss = float(res.loss)
    kappa = (np.sum(ref.seq_weight * np.abs(ref.seq_policy)) + 1e-300) / max(abs(ref.loss), 1e-300)
    rel = abs(loss - ref.loss) / max(abs(ref.loss), 1e-300)
    pp, pk = value_bounds(ref, cfg, e_logp, e_d)
    prop_loss = float(np.sum(ref.seq_weight * (pp.sum(axis=1) + cfg.beta * pk.sum(axis=1))))
    propagated = rel > loss_rtol
    print(f"  [{what}] loss gpu={loss!r} oracle={ref.loss!r} rel={rel:.3g} (bar {loss_rtol:g}) "
          f"kappa={kappa:.3g} propagated-bound={prop_loss:.3g} "
          f"{'FALLBACK' if propagated else 'strict'}", flush=True)
    if propagated:
        assert allow_propagated, (
            f"{what} loss gpu={loss!r} oracle={ref.loss!r} rel={rel:.3g} > {loss_rtol:g} "
            f"(kappa={kappa:.3g}; objective {cfg.pg_loss}/{cfg.kl_estimator} has no fallback)")
        lim = loss_rtol * abs(ref.loss) + prop_loss
        assert abs(loss - ref.loss) <= lim, (
            f"{what} loss gpu={loss!r} oracle={ref.loss!r} rel={rel:.3g} kappa={kappa:.3g} "
            f"propagated bound {prop_loss:.3g}")
    # policy_loss and kl: relative to the weighted absolute sums they are made of
    scale_p = float(np.sum(ref.seq_weight * np.abs(ref.tok["loss"]).sum(axis=1))) + 1e-30
    scale_k = float(np.sum(ref.seq_weight * np.abs(ref.tok["kl"]).sum(axis=1))) + 1e-30
    wp = float(np.sum(ref.seq_weight * pp.sum(axis=1)))
    wk = float(np.sum(ref.seq_weight * pk.sum(axis=1)))
    assert abs(float(res.policy_loss) - ref.policy_loss) <= loss_rtol * scale_p + wp, what
    assert abs(float(res.kl) - ref.kl) <= loss_rtol * scale_k + wk, what
    # per-sequence totals: the relative bound plus the propagated error
    sp = to_np(res.seq_policy)
    sk = to_np(res.seq_kl)
    tp = loss_rtol * np.abs(ref.tok["loss"]).sum(axis=1) + pp.sum(axis=1) + 1e-30
    tk = loss_rtol * np.abs(ref.tok["kl"]).sum(axis=1) + pk.sum(axis=1) + 1e-30
    ep = np.abs(sp - ref.seq_policy)
    ek = np.abs(sk - ref.seq_kl)
    assert np.all(ep <= tp), f"{what} seq_policy worst {np.max(ep / tp):.3g}x of bound"
    assert np.all(ek <= tk), f"{what} seq_kl worst {np.max(ek / tk):.3g}x of bound"
    return rel, kappa, propagated


def compare_token_values(res, ref, cfg, mask, rtol, e_logp=LOGP_ABS_ERR, e_d=2 * LOGP_ABS_ERR):
    """Per-token loss and KL outputs: rtol plus the propagated error; 0 at
    masked slots."""
    pp, pk = value_bounds(ref, cfg, e_logp, e_d)
    for name, bound in (("loss", pp), ("kl", pk)):
        g = to_np(getattr(res, "tok_" + name))
        r = ref.tok[name]
        assert np.all(g[~mask] == 0.0), f"tok_{name} at masked slots"
        lim = rtol * np.abs(r) + 2.0 * bound + 1e-30
        bad = (np.abs(g - r) > lim) & mask
        assert not bad.any(), (f"tok_{name}: {int(bad.sum())} values out of bound, first at "
                               f"{np.argwhere(bad)[0]}: gpu={g[bad][0]!r} oracle={r[bad][0]!r}")


def compare_token_grad(g, ref, cfg, mask, bar=1e-5, what=""):
    """d loss / d logp of the log-prob token path against the oracle at
    bar * max|G|.  The inputs are float32 log-probs, so the one place where
    two results are correct is a token whose float32 ratio sits at a clip
    bound (within 4e-7 relative): there the value must match the oracle's G
    or the other branch's (clipped: the KL part alone; unclipped: -A rho
    plus it), never be skipped.  Masked tokens must be exactly 0.  Returns
    (ambiguous tokens, how many took the other branch)."""
    g = np.asarray(g, dtype=np.float64)
    G = ref.grad
    lim = bar * float(np.max(np.abs(G)))
    rho = ref.tok["rho"]
    lo, hi = 1.0 - cfg.eps_low, 1.0 + cfg.eps_high
    amb = ((np.abs(rho - hi) <= 4e-7 * rho) | (np.abs(rho - lo) <= 4e-7 * rho)) & mask
    t = _terms_at(ref, cfg)
    adv = ref.tok["adv"] if "adv" in ref.tok else ref.advantages[:, None]
    other = np.where(t["clipped"], -adv * t["rho"], 0.0)
    G_other = ref.seq_weight[:, None] * (other + cfg.beta * t["dkl"])
    near = np.abs(g - G) <= lim
    near_other = amb & (np.abs(g - G_other) <= lim)
    bad = mask & ~(near | near_other)
    assert not bad.any(), (f"{what} {int(bad.sum())} dlogp values out of tolerance (bar {bar:g} "
                           f"x max|G| = {lim:.3g})")
    assert np.all(g[~mask] == 0.0), what
    n_amb, n_other = int(amb.sum()), int((near_other & ~near).sum())
    print(f"  [{what}] dlogp: {n_amb} tokens at a clip bound, {n_other} took the other branch",
          flush=True)
    return n_amb, n_other


def compare_exact_parts(res, ref, what=""):
    assert_bits_equal(to_np(res.advantages), ref.advantages, what + " advantages")
    assert_bits_equal(to_np(res.seq_weight), ref.seq_weight, what + " seq_weight")
    assert np.array_equal(to_np(res.seq_tokens), ref.seq_tokens), what + " seq_tokens"
    counts = to_np(res.counts)
    assert int(counts[0]) == ref.num_tokens, what + " N"
    return counts


# per-element bar of 16-bit gradients: (relative bound, absolute floor)
GRAD16_BAR = {"bf16": (2.0 ** -7, 2.0 ** -126), "f16": (2.0 ** -10, 2.0 ** -24)}


def compare_logits_grad(grad_gpu, ref, cfg, mask, gdt, what="", policy=None, ids=None,
                        branches=None):
    """grad_gpu: float64 numpy [B, T, V]; ref: oracle result with grad.
    gdt: the gradient's storage, "f32", "bf16" or "f16" (True means "bf16",
    False "f32").
    policy, ids: host policy logits and action ids, needed only to rebuild a
    row whose oracle G is exactly zero when the GPU took the other branch.
    branches: precomputed (flag-ambiguous, branch-ambiguous, candidate G
    list, relative G tolerance, ill-conditioned) for the sequence-level
    losses (seq_branches); None derives them per token."""
    if gdt is True or gdt is False:
        gdt = "bf16" if gdt else "f32"
    bf16 = gdt != "f32"                         # a 16-bit per-element bar
    base, floor = GRAD16_BAR.get(gdt, (None, None))
    g = grad_gpu
    r = ref.grad
    if branches is None:
        flag_amb, amb, cands = branch_ambiguity(ref, cfg, mask)
    else:
        flag_amb, amb, cands = branches[:3]
    stats = dict(ambiguous=int(flag_amb.sum()), branch_ambiguous=int(amb.sum()), illcond=0,
                 rows=int(mask.sum()))
    # masked rows: exactly zero
    assert np.all(g[~mask] == 0.0), what + " masked rows must be zero"
    gmax = float(np.max(np.abs(r))) if r.size else 0.0

    def row_ok(gi, ri, tol_rel):
        if bf16:
            with np.errstate(invalid="ignore"):
                lim = np.where(np.abs(ri) > 0, tol_rel * np.abs(ri), 0.0) + floor
            return np.abs(gi - ri) <= lim
        return np.abs(gi - ri) <= 1e-5 * gmax + 1e-30

    if bf16:
        tol, ill = g_rel_tolerance(ref, cfg, base) if branches is None else branches[3:5]
        stats["illcond"] = int((ill & mask).sum())
        ok = row_ok(g, r, tol[..., None])
    else:
        tol = np.full(mask.shape, 1e-5)
        ok = row_ok(g, r, None)
    bad_rows = ~ok.all(axis=-1) & mask
    # rows at a branch point may match any candidate branch instead
    for (i, t) in zip(*np.nonzero(bad_rows & amb)):
        G = ref.tok["G"][i, t]
        for C in cands[1:]:
            Gc = C[i, t]
            if G != 0:
                alt = r[i, t] * (Gc / G)
            elif policy is not None and ids is not None:
                x = policy[i, t].astype(np.float64)
                p = np.exp(x - x.max())
                p /= p.sum()
                onehot = np.zeros_like(p)
                onehot[int(ids[i, t])] = 1.0
                alt = Gc * (onehot - p)
            else:
                continue
            if np.all(row_ok(g[i, t], alt, base)):
                bad_rows[i, t] = False
                break
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


def token_branches(ref, cfg, mask, base):
    """The branch tuple of seq_branches for a token-level objective:
    (flag-ambiguous, branch-ambiguous, candidate G list, relative G
    tolerance, ill-conditioned), all [B, T]."""
    flag, amb, cands = branch_ambiguity(ref, cfg, mask)
    tol, ill = g_rel_tolerance(ref, cfg, base)
    return flag, amb, cands, tol, ill


def check_grad_row(g, x, a, key, branches, gdt, what=""):
    """One 16-bit gradient row ``g`` (float64 [V]) against the oracle's row
    G (onehot(a) - softmax(x)) for logits ``x`` and taken id ``a``, with G
    the oracle's value at slot ``key`` = (i, t) of ``branches`` (token_branches
    or seq_branches).  At a branch point a row that matches any candidate
    G passes (at the plain 16-bit bar)."""
    base, floor = GRAD16_BAR[gdt]
    _, amb, cands, tol, _ = branches
    i, t = key
    xr = np.asarray(x, dtype=np.float64)[None]
    lse = oracle.row_logsumexp(xr)
    ids = np.array([int(a)])
    worst = None
    for k, C in enumerate(cands):
        if k > 0 and not amb[i, t]:
            break
        r = oracle.softmax_grad_rows(xr, ids, lse, np.array([C[i, t]]))[0]
        rel = tol[i, t] if k == 0 else base
        with np.errstate(invalid="ignore"):
            lim = np.where(np.abs(r) > 0, rel * np.abs(r), 0.0) + floor
        err = np.abs(g - r)
        if np.all(err <= lim):
            return
        if worst is None:
            v = int(np.argmax(err / lim))
            worst = (float(err[v] / lim[v]), v, float(g[v]), float(r[v]), float(C[i, t]))
    raise AssertionError(f"{what} gradient row {key}: worst element {worst[1]} at {worst[0]:.3g}x "
                         f"of its bound (gpu {worst[2]!r}, oracle {worst[3]!r}, G {worst[4]!r})")


def sample_rows(B, T, mask, rng, n=24):
    """Flat slot indices to check one by one: the first and last slot, one
    active slot per sequence, the last slot of every ragged sequence (a
    masked one) and ``n`` uniform draws."""
    rows = {0, B * T - 1}
    for i in range(B):
        act = np.nonzero(mask[i])[0]
        if act.size:
            rows.add(i * T + int(act[rng.integers(0, act.size)]))
        if act.size < T:
            rows.add(i * T + T - 1)
    rows |= set(int(v) for v in rng.integers(0, B * T, n))
    return sorted(rows)


def assert_grad_rows_sum_to_zero(grad2d, chunk=2048):
    """Every gradient row is G (onehot - softmax), so it sums to G (1 - sum p)
    = 0 up to the storage rounding of its elements."""
    n = grad2d.shape[0]
    for s in range(0, n, chunk):
        blk = grad2d[s:s + chunk].double()
        rs = blk.sum(dim=1)
        ra = blk.abs().sum(dim=1)
        assert bool(torch.all(rs.abs() <= 2.0 ** -7 * ra + 1e-30)), f"row sums, rows {s}..{s + chunk}"


# ---------------------------------------------------------------------------
# Sequence-level losses (GSPO, REAL).  Their policy part depends on s_i, the
# mean log-ratio of a sequence, which the GPU forms from float32 log-probs:
# its error is at most the log-prob error.  As for the token-level helpers,
# the oracle evaluated at s +- e (and at d +- e for the KL part) gives the
# candidate G of a sequence at a branch point (a GSPO sequence at its clip
# bound) and the propagated error of G and of the values elsewhere.
# ---------------------------------------------------------------------------

SEQ_ABS_ERR = 2 * LOGP_ABS_ERR


def _active_index(mask):
    ii, tt = np.nonzero(mask)
    return ii, tt


def _token_is_weights(cfg, h, mask):
    """Off-policy weight of every slot (1 without generating log-probs; 0 at
    masked slots)."""
    if h.get("gen_logps") is None:
        return mask.astype(np.float64)
    om = oracle.is_weights(h["old_logps"], h["gen_logps"], cfg)
    return np.where(mask, om, 0.0)


def _seq_policy_part(ref, cfg, s, h, mask, groups):
    """Per sequence (gpol coefficient, policy value l_i or group losses) at
    log-ratios s, via the oracle's own sequence functions."""
    B = mask.shape[0]
    A = ref.advantages
    L = ref.seq_tokens
    w = ref.seq_weight
    if cfg.pg_loss == "gspo":
        _, l_seq, dl_ds, clipped = oracle.gspo_terms(s, A, cfg)
        om_mean = _token_is_weights(cfg, h, mask).sum(axis=1) / np.maximum(L, 1)
        return dict(coef=w * om_mean * dl_ds, value=l_seq, branch=clipped, om_mean=om_mean)
    off = oracle.group_offsets(B, groups.get("samples_per_prompt"), groups.get("group_boundaries"))
    gl, dpol, pol = oracle.real_terms(s, A, L, off, cfg.real_tau)
    return dict(coef=dpol / np.maximum(L, 1), value=gl, policy_loss=pol,
                branch=np.zeros(B, dtype=bool), dpol=dpol)


def _seq_G(ref, cfg, part, dkl):
    return part["coef"][:, None] + ref.seq_weight[:, None] * (cfg.beta * dkl)


def seq_branches(ref, cfg, mask, h, groups, base, e_s=SEQ_ABS_ERR, e_d=4 * LOGP_ABS_ERR):
    """(flag-ambiguous, branch-ambiguous [B, T], candidate G list, relative G
    tolerance [B, T], ill-conditioned [B, T]) for a sequence-level loss."""
    s = ref.seq_logratio
    center = _seq_policy_part(ref, cfg, s, h, mask, groups)
    dkl0 = ref.tok["dkl"]
    G0 = _seq_G(ref, cfg, center, dkl0)
    cands = [G0]
    flag = np.zeros(mask.shape, dtype=bool)
    anyb = np.zeros(mask.shape, dtype=bool)
    dG = np.zeros(mask.shape)
    for ds in (e_s, -e_s):
        part = _seq_policy_part(ref, cfg, s + ds, h, mask, groups)
        Gp = _seq_G(ref, cfg, part, dkl0)
        cands.append(Gp)
        chg = (part["branch"] != center["branch"])[:, None] & mask
        flag |= chg
        anyb |= chg
        dG = np.maximum(dG, np.where(chg, 0.0, np.abs(Gp - G0)))
    dGd = np.zeros(mask.shape)
    for dd in (e_d, -e_d):
        _, dkl = oracle.kl_terms(ref.tok["d"] + dd, cfg)
        dkl = np.where(mask, dkl, 0.0)
        Gp = _seq_G(ref, cfg, center, dkl)
        cands.append(Gp)
        chg = ((dkl == 0) != (dkl0 == 0)) & mask
        anyb |= chg
        dGd = np.maximum(dGd, np.where(chg, 0.0, np.abs(Gp - G0)))
    with np.errstate(divide="ignore", invalid="ignore"):
        rel = np.where(G0 != 0, (dG + dGd) / np.abs(G0), np.inf)
    return flag & mask, anyb & mask, cands, np.maximum(base, rel), (rel > base) & (G0 != 0) & mask


def compare_seq_outputs(res, ref, cfg, mask, h, groups, rtol, what=""):
    """Scalars, per-sequence and per-token values of a sequence-level loss.
    Returns the number of sequences at a clip bound (either branch correct)."""
    B = mask.shape[0]
    s = ref.seq_logratio
    gs = to_np(res.seq_logratio)
    lim_s = SEQ_ABS_ERR + 2.0 ** -23 * np.abs(s)
    assert np.all(np.abs(gs - s) <= lim_s), (
        f"{what} seq_logratio worst {np.max(np.abs(gs - s) / lim_s):.3g}x of bound")
    center = _seq_policy_part(ref, cfg, s, h, mask, groups)
    _, pk = value_bounds(ref, cfg)
    kl_prop = float(np.sum(ref.seq_weight * pk.sum(axis=1)))
    ambiguous_seq = np.zeros(B, dtype=bool)
    if cfg.pg_loss == "gspo":
        # error of l_i from s +- e (a sequence at its clip bound may take either branch)
        dval = np.zeros(B)
        for ds in (SEQ_ABS_ERR, -SEQ_ABS_ERR):
            part = _seq_policy_part(ref, cfg, s + ds, h, mask, groups)
            ambiguous_seq |= part["branch"] != center["branch"]
            dval = np.maximum(dval, np.abs(part["value"] - center["value"]))
        dval = dval + rtol * np.abs(center["value"])
        om = _token_is_weights(cfg, h, mask)
        tok_bound = om * dval[:, None] + rtol * np.abs(ref.tok["loss"]) + 1e-30
        tl = to_np(res.tok_loss)
        bad = (np.abs(tl - ref.tok["loss"]) > tok_bound) & mask
        assert not bad.any(), f"{what} tok_loss: {int(bad.sum())} values out of bound"
        assert np.all(tl[~mask] == 0.0), f"{what} tok_loss at masked slots"
        seq_bound = tok_bound.sum(axis=1)
        sp = to_np(res.seq_policy)
        assert np.all(np.abs(sp - ref.seq_policy) <= seq_bound), f"{what} seq_policy"
        pol_prop = float(np.sum(ref.seq_weight * seq_bound))
        pol_scale = float(np.sum(ref.seq_weight * np.abs(ref.seq_policy)))
    else:
        pol_prop = float(np.sum(np.abs(center["dpol"]))) * SEQ_ABS_ERR
        pol_scale = float(np.sum(np.abs(center["value"]))) / max(len(center["value"]), 1)
        assert np.all(to_np(res.seq_policy) == 0.0), f"{what} REAL seq_policy must be 0"
        assert np.all(to_np(res.tok_loss) == 0.0), f"{what} REAL token losses must be 0"
    loss = float(res.loss)
    lim = rtol * abs(ref.loss) + pol_prop + cfg.beta * kl_prop + 1e-30
    assert abs(loss - ref.loss) <= lim, (
        f"{what} loss gpu={loss!r} oracle={ref.loss!r} bound {lim:.3g}")
    assert abs(float(res.policy_loss) - ref.policy_loss) <= rtol * pol_scale + pol_prop + 1e-30, (
        f"{what} policy_loss gpu={float(res.policy_loss)!r} oracle={ref.policy_loss!r}")
    scale_k = float(np.sum(ref.seq_weight * np.abs(ref.tok["kl"]).sum(axis=1))) + 1e-30
    assert abs(float(res.kl) - ref.kl) <= rtol * scale_k + kl_prop, f"{what} kl"
    tk = rtol * np.abs(ref.tok["kl"]).sum(axis=1) + pk.sum(axis=1) + 1e-30
    assert np.all(np.abs(to_np(res.seq_kl) - ref.seq_kl) <= tk), f"{what} seq_kl"
    return int(ambiguous_seq.sum())
