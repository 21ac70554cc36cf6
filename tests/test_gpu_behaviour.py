"""Behaviour of the HIP path that parity alone does not show: bitwise
reproducibility, masked-slot immunity, in-place gradients, the ref == policy
identity, device-detected data faults, and the split forward/backward used by
autograd."""

import math

import numpy as np
import pytest
import torch

import oracle
from _parity import cfg_from, compare_logits_grad, compare_scalars, gpu_kwargs, host_inputs, to_np
from rl_post_loss_amd._abi import GRPO_ABI_VERSION
from workloads import WORKLOADS, LogitsWorkload, make_logits_inputs, poison_masked

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _wl(V=5000, dtype="bf16", T=8, sizes=(4, 4), **kw):
    base = dict(name=f"beh_V{V}", group_sizes=sizes, T=T, V=V, dtype=dtype, logit_std=2.0,
                ref_noise_std=math.sqrt(0.1), old_noise_std=math.sqrt(0.05), reward_p=0.5,
                len_range=(1, T))
    base.update(kw)
    return LogitsWorkload(**base)


def _inputs(wl, seed=0):
    cpu = make_logits_inputs(wl, device="cpu", seed=seed)
    return cpu, {k: v.to(DEV) for k, v in cpu.items()}


def _call(rpl, inp, wl, **extra):
    kw = gpu_kwargs(wl)
    kw.update(extra)
    res = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                inp["rewards"], inp["mask"], per_token=True, **kw)
    torch.cuda.synchronize()
    return res


def _same(a, b):
    return torch.equal(a.view(torch.uint8) if a.dtype != torch.bool else a,
                       b.view(torch.uint8) if b.dtype != torch.bool else b)


def _bits(t):
    return t.contiguous().view(torch.uint8)


@pytest.mark.parametrize("V,dtype", [(151936, "bf16"), (32, "f32"), (5000, "bf16")])
def test_bitwise_reproducible(gpu_lib, V, dtype):
    wl = _wl(V, dtype, T=16 if V > 10000 else 64)
    announce(f"determinism V={V} {dtype}")
    _, inp = _inputs(wl, seed=11)
    first = _call(gpu_lib, inp, wl)
    for k in range(10):
        again = _call(gpu_lib, inp, wl)
        assert torch.equal(_bits(first.scalars), _bits(again.scalars)), k
        assert torch.equal(_bits(first.seq_policy), _bits(again.seq_policy)), k
        assert torch.equal(_bits(first.seq_kl), _bits(again.seq_kl)), k
        assert torch.equal(_bits(first.grad), _bits(again.grad)), k


def test_masked_nan_inf_garbage_ids_do_not_leak(gpu_lib):
    wl = _wl(3001, "bf16", T=12)
    announce("masked poison")
    cpu, inp = _inputs(wl, seed=12)
    clean = _call(gpu_lib, inp, wl)
    bad = poison_masked(inp, V=wl.V)
    dirty = _call(gpu_lib, bad, wl)
    assert torch.equal(_bits(clean.scalars), _bits(dirty.scalars))
    assert torch.equal(_bits(clean.grad), _bits(dirty.grad))
    assert int(dirty.status[0]) == 0


@pytest.mark.parametrize("V", [8192, 40000, 60000, 151936])
def test_in_place_gradient_matches_out_of_place(gpu_lib, V):
    """The gradient written over the policy logits equals the out-of-place
    one bit for bit: resident rows at 256 and 512 threads, and streaming
    rows whose first chunks pass 2 takes from LDS rather than from the
    (by then partly overwritten) logits."""
    wl = _wl(V, "bf16", T=8 if V < 100000 else 4)
    announce(f"in place V={V}")
    _, inp = _inputs(wl, seed=13)
    out = _call(gpu_lib, inp, wl)
    pol = inp["policy"].clone()
    res = gpu_lib.grpo_loss_fwd_bwd(pol, inp["ref"], inp["action_ids"], inp["old_logps"],
                                    inp["rewards"], inp["mask"], grad_out=pol, **gpu_kwargs(wl))
    torch.cuda.synchronize()
    assert res.grad.data_ptr() == pol.data_ptr()
    assert torch.equal(_bits(out.scalars), _bits(res.scalars))
    assert torch.equal(_bits(out.grad), _bits(pol))


def test_identity_ref_is_policy_and_old_is_logp(gpu_lib):
    """ref_logits is policy_logits and old_logps equals the kernel's own
    log-probs: rho = 1 and k3 = 0 exactly, so the loss is -sum_i w_i L_i A_i."""
    wl = _wl(20000, "bf16", T=10)
    announce("identity")
    _, inp = _inputs(wl, seed=14)
    first = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["policy"], inp["action_ids"],
                                      inp["old_logps"], inp["rewards"], inp["mask"],
                                      per_token=True, **gpu_kwargs(wl))
    torch.cuda.synchronize()
    old = first.tok_logp.clone()
    for eps in (0.1, 0.2, 0.45):
        kw = gpu_kwargs(wl)
        kw.update(eps_low=eps, eps_high=eps)
        res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["policy"], inp["action_ids"], old,
                                        inp["rewards"], inp["mask"], per_token=True, **kw)
        torch.cuda.synchronize()
        assert float(res.kl) == 0.0
        assert torch.all(res.tok_kl == 0.0)
        assert int(res.counts[1]) == 0
        A = to_np(res.advantages)
        w = to_np(res.seq_weight).astype(np.float64)
        L = to_np(res.seq_tokens).astype(np.float64)
        # per token the loss is -A exactly (rho == 1), so the sequence total is -L*A
        assert np.array_equal(to_np(res.seq_policy), (-L * A).astype(np.float32).astype(np.float64))
        h_old = first.tok_logp
        assert torch.equal(res.tok_logp, h_old)
        expect = -np.sum(w.astype(np.float32).astype(np.float64) * L * A)
        assert abs(float(res.loss) - expect) <= 1e-6 * max(1.0, abs(expect))


def test_bad_action_id_flags_and_zeroes_row(gpu_lib):
    wl = _wl(1000, "f32", T=4, len_range=None)
    announce("bad action id")
    _, inp = _inputs(wl, seed=15)
    ids = inp["action_ids"].clone()
    ids[1, 2] = wl.V          # out of range at an active slot
    ids[3, 0] = -3
    res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], ids, inp["old_logps"],
                                    inp["rewards"], inp["mask"], per_token=True, **gpu_kwargs(wl))
    torch.cuda.synchronize()
    assert int(res.status[0]) & gpu_lib.GRPO_FAULT_BAD_ACTION
    assert torch.all(res.grad[1, 2] == 0) and torch.all(res.grad[3, 0] == 0)
    assert float(res.tok_loss[1, 2]) == 0.0 and float(res.tok_kl[3, 0]) == 0.0
    assert math.isfinite(float(res.loss))
    # the next clean call reports no fault (status is per call)
    clean = _call(gpu_lib, inp, wl)
    assert int(clean.status[0]) == 0


def test_no_active_tokens(gpu_lib):
    wl = _wl(700, "bf16", T=5)
    announce("no active tokens")
    _, inp = _inputs(wl, seed=16)
    mask = torch.zeros_like(inp["mask"])
    for red in ("token_mean", "sequence_mean", "length_alpha", "per_sequence_then_mean"):
        res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"],
                                        inp["old_logps"], inp["rewards"], mask,
                                        **dict(gpu_kwargs(wl), reduction=red, alpha=0.5))
        torch.cuda.synchronize()
        assert int(res.status[0]) & gpu_lib.GRPO_FAULT_NO_TOKENS
        assert float(res.loss) == 0.0 and float(res.kl) == 0.0
        assert torch.all(res.grad == 0)
        assert int(res.counts[0]) == 0


@pytest.mark.parametrize("V", [6000, 12000, 20000])
def test_autograd_split_forward_backward(gpu_lib, V):
    """grpo_loss() runs the forward pass, keeps per-row weights, and the
    backward pass writes the gradient scaled by the upstream gradient.
    12 KB rows: the fused kernel and both split kernels give a row 256
    threads, so the split path carries the fused call's bits.  24 KB and
    40 KB rows: the fused kernel holds a row at 512 threads (and the
    gradient-only kernel runs 1024 on 40 KB rows), so the log-sum-exp trees
    differ and both paths are held to the oracle instead."""
    wl = _wl(V, "bf16", T=6)
    bitwise = V * 2 <= 16384
    announce(f"autograd split V={V} ({'bitwise against the fused call' if bitwise else 'oracle'})")
    cpu, inp = _inputs(wl, seed=17)
    fused = _call(gpu_lib, inp, wl)
    pol = inp["policy"].clone().requires_grad_(True)
    loss, pl, kl = gpu_lib.grpo_loss(pol, inp["ref"], inp["action_ids"], inp["old_logps"],
                                     inp["rewards"], inp["mask"], **gpu_kwargs(wl))
    if bitwise:
        assert torch.equal(_bits(loss.detach().reshape(1)), _bits(fused.scalars[:1]))
    # policy_loss and kl are detached reporting values
    assert loss.requires_grad and not pl.requires_grad and not kl.requires_grad
    with pytest.raises(RuntimeError):
        kl.backward()
    loss.backward()
    torch.cuda.synchronize()
    h = host_inputs(cpu)
    cfg = cfg_from(wl)

    def oracle_ref(scale):
        return oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"],
                                        h["mask"], h["rewards"], groups=wl.groups_kwargs(),
                                        cfg=cfg, grad_scale=scale)

    if bitwise:
        assert torch.equal(_bits(pol.grad), _bits(fused.grad))
    else:
        ref = oracle_ref(1.0)
        rel = abs(float(loss.detach()) - ref.loss) / abs(ref.loss)
        print(f"  split loss rel {rel:.3g} against the oracle (bar 1e-4)", flush=True)
        assert rel <= 1e-4
        compare_logits_grad(to_np(pol.grad), ref, cfg, h["mask"], "bf16", "split backward")
    pol.grad = None
    loss2, _, _ = gpu_lib.grpo_loss(pol, inp["ref"], inp["action_ids"], inp["old_logps"],
                                    inp["rewards"], inp["mask"], **gpu_kwargs(wl))
    (2.0 * loss2).backward()
    torch.cuda.synchronize()
    if bitwise:
        scale = torch.tensor([2.0], device=DEV)
        fused2 = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"],
                                           inp["old_logps"], inp["rewards"], inp["mask"],
                                           grad_scale=scale, **gpu_kwargs(wl))
        torch.cuda.synchronize()
        assert torch.equal(_bits(pol.grad), _bits(fused2.grad))
    else:
        compare_logits_grad(to_np(pol.grad), oracle_ref(2.0), cfg, h["mask"], "bf16",
                            "split backward, upstream 2")


@pytest.mark.parametrize("V,dtype,ld,gdtype", [
    (32768, "bf16", None, None),            # 64 KB rows: the row kernel (the flat map's limit)
    (32776, "bf16", None, None),            # one chunk more: the flat gradient map
    (40000, "bf16", None, None),            # 80 KB rows
    (40003, "bf16", 40008, None),           # padded 16-byte rows: the flat map's scalar tail
    (20000, "f32", None, None),             # float32 rows of 80 KB
    (40000, "bf16", None, torch.float32),   # bf16 logits, float32 gradient
    (40000, "f16", None, None),             # IEEE half logits and gradient
])
def test_split_backward_long_rows(gpu_lib, V, dtype, ld, gdtype):
    """The gradient-only pass on rows above 64 KB (the flat map over 16-byte
    chunks, a block per 4 KB of a row) after a forward-only pass on the same
    workspace, with an upstream gradient of 1 and 2, against the oracle; the
    gradient buffer's row padding stays untouched."""
    wl = _wl(V, dtype, T=6)
    announce(f"split backward long rows V={V} {dtype} ld={ld} grad={gdtype}")
    cpu, inp = _inputs(wl, seed=23)
    B, T = wl.B, wl.T
    pol, ref = inp["policy"], inp["ref"]
    gdt = pol.dtype if gdtype is None else gdtype
    if ld is not None:
        pbuf = torch.full((B, T, ld), float("nan"), dtype=pol.dtype, device=DEV)
        rbuf = torch.full((B, T, ld), float("inf"), dtype=pol.dtype, device=DEV)
        pbuf[..., :V] = pol
        rbuf[..., :V] = ref
        pol, ref = pbuf[..., :V], rbuf[..., :V]
    gbuf = torch.full((B, T, ld or V), 7.0, dtype=gdt, device=DEV)
    h = host_inputs(cpu)
    cfg = cfg_from(wl)
    for scale in (1.0, 2.0):
        ws = gpu_lib.workspace(B, T, 0, DEV, dedicated=True)
        res = gpu_lib.grpo_loss_fwd_bwd(pol, ref, inp["action_ids"], inp["old_logps"],
                                        inp["rewards"], inp["mask"], grad_out=False, _ws=ws,
                                        **gpu_kwargs(wl))
        gs = torch.tensor([scale], dtype=torch.float32, device=DEV)
        gpu_lib.grpo_loss_bwd(pol, inp["action_ids"], inp["mask"], ws, grad_out=gbuf[..., :V],
                              grad_scale=gs)
        torch.cuda.synchronize()
        if ld is not None:
            assert torch.all(gbuf[..., V:] == 7.0), "padding of the gradient must stay untouched"
        ref64 = oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"],
                                         h["mask"], h["rewards"], groups=wl.groups_kwargs(),
                                         cfg=cfg, grad_scale=scale)
        compare_scalars(res, ref64, cfg, 1e-4 if dtype != "f32" else 1e-5, f"forward V={V}")
        gname = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}[gdt]
        compare_logits_grad(to_np(gbuf[..., :V]), ref64, cfg, h["mask"], gname, f"backward x{scale}")


def test_confident_token_gradient_relative_accuracy(gpu_lib):
    """p_a close to 1: 1 - p_a is formed without cancellation, so g_a keeps
    its relative accuracy."""
    V = 4096
    wl = _wl(V, "f32", T=2, len_range=None, beta=0.0)
    announce("confident tokens")
    cpu, inp = _inputs(wl, seed=18)
    ids = inp["action_ids"]
    pol = inp["policy"].clone()
    # the taken token dominates: 1 - p_a is about 4e-7
    pol.scatter_(2, ids[..., None], 25.0)
    res = gpu_lib.grpo_loss_fwd_bwd(pol, inp["ref"], ids, inp["old_logps"], inp["rewards"],
                                    inp["mask"], per_token=True, **gpu_kwargs(wl))
    torch.cuda.synchronize()
    h = host_inputs(dict(cpu, policy=pol.cpu()))
    ref = oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"],
                                   h["mask"], h["rewards"], groups=wl.groups_kwargs(),
                                   cfg=cfg_from(wl))
    g = to_np(res.grad)
    r = ref.grad
    idx = np.take_along_axis(r, h["action_ids"][..., None], -1)[..., 0]
    gi = np.take_along_axis(g, h["action_ids"][..., None], -1)[..., 0]
    nz = idx != 0
    rel = np.abs(gi - idx)[nz] / np.abs(idx[nz])
    assert np.all(rel < 1e-4), rel.max()
    lp = to_np(res.tok_logp)
    assert np.all(np.abs(lp - ref.tok["logp"]) <= 1e-6 * np.abs(ref.tok["logp"]) + 1e-12)


@pytest.mark.parametrize("reduction", ["token_mean", "sequence_mean", "length_alpha",
                                       "fixed_constant", "per_sequence_then_mean"])
def test_token_loss_fault_bits(gpu_lib, reduction):
    """The log-prob entry point's fault bits, on both of its launch
    structures (token mean and the mean over live sequences, whose weights
    need a batch count: counts, token and scalar kernels; the others: the
    token kernel forms its own counts and reports faults per sequence): no
    active token gives NO_TOKENS with zero loss and gradient; a non-finite
    per-token value at an active slot gives NONFINITE; the next clean call
    on the same workspace reports no fault (status is per call)."""
    from workloads import TOKEN_WORKLOADS, make_token_inputs
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    announce(f"token loss fault bits {reduction}")
    inp = make_token_inputs(wl, device=DEV, seed=21, B=32, T=256)
    kw = dict(eps_low=0.2, eps_high=0.2, beta=0.04, samples_per_prompt=16, reduction=reduction,
              alpha=0.5 if reduction == "length_alpha" else None)
    if reduction == "fixed_constant":
        kw["norm_constant"] = 500.0

    def call(mask, old):
        res = gpu_lib.grpo_token_loss(inp["logp"], old, inp["ref_logp"], inp["rewards"], mask, **kw)
        torch.cuda.synchronize()
        return res

    none = call(torch.zeros_like(inp["mask"]), inp["old_logps"])
    assert int(none.status[0]) & gpu_lib.GRPO_FAULT_NO_TOKENS
    assert float(none.loss) == 0.0 and float(none.kl) == 0.0 and int(none.counts[0]) == 0
    assert torch.all(none.grad == 0)

    # an old log-prob of -inf at an active slot makes the ratio infinite
    old = inp["old_logps"].clone()
    act = torch.nonzero(inp["mask"][3])
    old[3, int(act[0])] = float("-inf")
    bad = call(inp["mask"], old)
    assert int(bad.status[0]) & gpu_lib.GRPO_FAULT_NONFINITE
    assert not int(bad.status[0]) & gpu_lib.GRPO_FAULT_NO_TOKENS

    clean = call(inp["mask"], inp["old_logps"])
    assert int(clean.status[0]) == 0
    assert int(clean.counts[0]) == int(inp["mask"].sum())


@pytest.mark.parametrize("V,dtype", [(5000, "bf16"), (1000, "f32"), (4097, "f16")])
def test_autograd_precompute_grad(gpu_lib, V, dtype):
    """grpo_loss(..., precompute_grad=True): the forward call writes the fused
    kernel's gradient and the backward multiplies it by the upstream
    gradient in place (grpo_scale_grad).  Upstream 1 leaves the fused
    gradient untouched (bitwise); other upstream values give exactly the
    float32 product rounded once to the storage, as torch's own multiply
    and conversion do; the split autograd path agrees within the storage's
    rounding."""
    wl = _wl(V, dtype, T=6)
    announce(f"autograd precompute_grad V={V} {dtype}")
    _, inp = _inputs(wl, seed=23)
    fused = _call(gpu_lib, inp, wl)
    for upstream in (1.0, 0.5, 0.37):
        pol = inp["policy"].clone().requires_grad_(True)
        loss, _, _ = gpu_lib.grpo_loss(pol, inp["ref"], inp["action_ids"], inp["old_logps"],
                                       inp["rewards"], inp["mask"], precompute_grad=True,
                                       **gpu_kwargs(wl))
        loss.backward(torch.tensor(upstream, device=DEV))
        torch.cuda.synchronize()
        assert float(loss.detach()) == float(fused.loss)
        want = fused.grad if upstream == 1.0 else (fused.grad.float() * upstream).to(fused.grad.dtype)
        assert torch.equal(_bits(pol.grad), _bits(want)), upstream
    # the split path (forward pass, then a backward stream with the scale inside G)
    pol = inp["policy"].clone().requires_grad_(True)
    loss, _, _ = gpu_lib.grpo_loss(pol, inp["ref"], inp["action_ids"], inp["old_logps"],
                                   inp["rewards"], inp["mask"], **gpu_kwargs(wl))
    loss.backward(torch.tensor(0.37, device=DEV))
    torch.cuda.synchronize()
    # Both gradients are rounded to the storage once (the fused one before
    # the scale, the split one after it), each within unit roundoff u of its
    # value, so they differ by at most 2u/(1-u) relative to ref, plus the
    # float32 arithmetic of the two orders (2^-20).  Below the smallest normal
    # the spacing is fixed: each rounding is off by at most half of it.
    u, tiny = {"bf16": (2.0 ** -8, 2.0 ** -133), "f16": (2.0 ** -11, 2.0 ** -24),
               "f32": (0.0, 2.0 ** -149)}[dtype]
    rel = 2 * u / (1 - u) + 2.0 ** -20
    ref = fused.grad.double() * 0.37
    err = (pol.grad.double() - ref).abs()
    excess = (err - tiny) / ref.abs().clamp_min(1e-300)
    assert bool(torch.all(err <= rel * ref.abs() + tiny)), (float(err.max()), float(excess.max()), rel)


@pytest.mark.parametrize("reduction", ["token_mean", "sequence_mean"])
def test_autograd_logp_loss(gpu_lib, reduction):
    """grpo_logp_loss: the same loss as grpo_token_loss, and logp.grad is
    that call's d loss / d logp (upstream 1, bitwise) or its float32 product
    with the upstream gradient (0.5, 0.37, exactly as torch multiplies)."""
    from workloads import TOKEN_WORKLOADS, make_token_inputs
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    announce(f"autograd logp loss {reduction}")
    inp = make_token_inputs(wl, device=DEV, seed=29, B=32, T=258)
    kw = dict(eps_low=0.2, eps_high=0.28, beta=0.04, samples_per_prompt=8, reduction=reduction)
    direct = gpu_lib.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                                     inp["mask"], **kw)
    torch.cuda.synchronize()
    for upstream in (1.0, 0.5, 0.37):
        lp = inp["logp"].clone().requires_grad_(True)
        loss, pol, kl = gpu_lib.grpo_logp_loss(lp, inp["old_logps"], inp["ref_logp"], inp["rewards"],
                                               inp["mask"], **kw)
        assert loss.requires_grad and not pol.requires_grad and not kl.requires_grad
        loss.backward(torch.tensor(upstream, device=DEV))
        torch.cuda.synchronize()
        assert float(loss.detach()) == float(direct.loss)
        assert float(pol.detach()) == float(direct.policy_loss)
        assert float(kl.detach()) == float(direct.kl)
        want = direct.grad if upstream == 1.0 else direct.grad * upstream
        assert torch.equal(_bits(lp.grad), _bits(want)), upstream


def test_logp_loss_chain_against_oracle(gpu_lib):
    """d loss / d logits through torch's log-softmax and gather into
    grpo_logp_loss (the token kernel's gradient, chained by torch's
    backward) against the oracle's fused gradient, at the float32 bar of the
    logits path: an end-to-end check of the token path that shares no kernel
    with the vocabulary kernel."""
    wl = _wl(V=1000, dtype="f32", T=12, sizes=(4, 4, 4), len_range=(1, 12))
    announce("logp loss chain vs oracle V=1000 f32")
    cpu, inp = _inputs(wl, seed=31)
    logits = inp["policy"].clone().requires_grad_(True)
    ids = inp["action_ids"][..., None]
    logp = torch.log_softmax(logits, dim=-1).gather(-1, ids).squeeze(-1)
    with torch.no_grad():
        ref_logp = torch.log_softmax(inp["ref"], dim=-1).gather(-1, ids).squeeze(-1).contiguous()
    loss, _, _ = gpu_lib.grpo_logp_loss(logp.contiguous(), inp["old_logps"], ref_logp, inp["rewards"],
                                        inp["mask"], **gpu_kwargs(wl))
    loss.backward()
    # the same call without autograd, for its per-sequence totals
    direct = gpu_lib.grpo_token_loss(logp.detach().contiguous(), inp["old_logps"], ref_logp,
                                     inp["rewards"], inp["mask"], **gpu_kwargs(wl))
    torch.cuda.synchronize()
    assert float(loss.detach()) == float(direct.loss)
    h = host_inputs(cpu)
    ref = oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"], h["action_ids"], h["old_logps"], h["mask"],
                                   h["rewards"], groups=wl.groups_kwargs(), cfg=cfg_from(wl))
    # the log-probs this path receives are torch's float32 log-softmax, not
    # exact values: their float32 error (not the kernel's) enters the loss,
    # whose condition number here is about 360, so the loss is held to the
    # relative bar plus that input error propagated through every token
    compare_scalars(direct, ref, cfg_from(wl), 1e-5, "logp chain", allow_propagated=True)
    compare_logits_grad(to_np(logits.grad), ref, cfg_from(wl), h["mask"], "f32", "logp chain")


def test_result_provenance(gpu_lib):
    """GRPOResult.provenance records the call; its fingerprint is the same
    for the same settings on other data and sizes, and differs when a setting
    that changes the numbers differs."""
    wl = _wl(1000, "f32", T=4)
    announce("provenance")
    _, inp = _inputs(wl, seed=41)
    a = _call(gpu_lib, inp, wl).provenance
    assert a["entry"] == "grpo_loss_fwd_bwd" and a["abi_version"] == GRPO_ABI_VERSION
    assert a["sizes"] == dict(B=wl.B, T=4, V=1000) and a["dtypes"]["logits"] == "torch.float32"
    assert a["groups"]["samples_per_prompt"] == 4 and a["device"]
    _, inp2 = _inputs(_wl(1000, "f32", T=9), seed=42)
    assert _call(gpu_lib, inp2, _wl(1000, "f32", T=9)).provenance["fingerprint"] == a["fingerprint"]
    other = _call(gpu_lib, inp, wl, eps_high=0.3).provenance
    assert other["fingerprint"] != a["fingerprint"] and other["config"]["eps_high"] == 0.3
    lp = torch.log_softmax(inp["policy"], -1).gather(-1, inp["action_ids"][..., None])[..., 0]
    t = gpu_lib.grpo_token_loss(lp.contiguous(), inp["old_logps"], lp.contiguous(), inp["rewards"],
                                inp["mask"], **gpu_kwargs(wl))
    torch.cuda.synchronize()
    assert t.provenance["entry"] == "grpo_token_loss" and t.provenance["inputs"]["grad"]


def test_scale_grad_layouts(gpu_lib):
    """grpo_scale_grad on a padded row stride (scalar path) and on aligned
    rows (vector path) in every storage: the rows scale exactly as torch's
    float32 multiply and conversion do, the padding is never touched, and a
    scale of 1 leaves every bit as it was."""
    announce("scale_grad layouts")
    g = torch.Generator(device=DEV).manual_seed(3)
    s = torch.tensor([0.73], dtype=torch.float32, device=DEV)
    one = torch.ones(1, dtype=torch.float32, device=DEV)
    for dt in (torch.float32, torch.bfloat16, torch.float16):
        for V, ld in ((1000, 1000), (1001, 1008), (4096, 4100)):
            buf = torch.randn((37, ld), generator=g, device=DEV).to(dt)
            view = buf[:, :V]
            before = buf.clone()
            gpu_lib.grpo_scale_grad(view, one)
            torch.cuda.synchronize()
            assert torch.equal(_bits(buf), _bits(before))
            gpu_lib.grpo_scale_grad(view, s)
            torch.cuda.synchronize()
            assert torch.equal(_bits(view.contiguous()),
                               _bits((before[:, :V].float() * 0.73).to(dt)))
            assert torch.equal(_bits(buf[:, V:].contiguous()), _bits(before[:, V:].contiguous()))
    # every finite 16-bit pattern (both zeros, subnormals, the largest values),
    # through the scalar path (7-element rows) and the vector path (8)
    pat = torch.arange(-(1 << 15), 1 << 15, dtype=torch.int32).to(torch.int16)
    for dt in (torch.bfloat16, torch.float16):
        x = pat.view(dt).to(DEV)
        x = x[torch.isfinite(x)]
        for V in (7, 8):
            n = (x.numel() // V) * V
            rows = x[:n].reshape(-1, V).contiguous()
            for scale in (0.5, 0.73, 1.75):
                got = rows.clone()
                gpu_lib.grpo_scale_grad(got, torch.tensor([scale], dtype=torch.float32, device=DEV))
                torch.cuda.synchronize()
                assert torch.equal(_bits(got), _bits((rows.float() * scale).to(dt))), (dt, V, scale)


@pytest.mark.parametrize("general", [False, True])
def test_kl_estimator_accuracy(gpu_lib, general):
    """The k3 estimator e^d - 1 - d and its derivative e^d - 1 as the kernels
    evaluate them, against binary64, over d in [-40, 40] (dense near 0).
    With logp = old (ratio 1), equal rewards (A = 0), beta = 1 and a fixed
    normaliser of 1, the token's KL output is k3(d) and its gradient is
    -(e^d - 1) with no other rounding.  For |d| < 1 (the series) both are
    within 4 ulp; beyond, within 4 ulp of the hardware exponential's error
    e^d (|d| + 1) 2^-24.  general: the objective's general code path (an
    input clamp no value reaches)."""
    announce(f"KL estimator accuracy general={general}")
    B, T = 16, 4096
    rng = np.random.default_rng(5)
    tiny = np.logspace(-8, 0, 6000)
    d_want = np.concatenate([tiny, -tiny, np.linspace(-1.5, 1.5, 20000), rng.uniform(-40, 40, 20000),
                             [0.0, 1.0, -1.0, 0.9999999, -0.9999999]])
    d_want = np.resize(d_want, B * T).reshape(B, T)
    logp = np.full((B, T), -1.25, dtype=np.float32)
    ref = (logp.astype(np.float64) + d_want).astype(np.float32)
    d = (ref - logp).astype(np.float64)                 # the float32 difference the kernel forms
    kw = dict(samples_per_prompt=8, beta=1.0, reduction="fixed_constant", norm_constant=1.0,
              per_token=True)
    if general:
        kw["kl_input_clamp"] = 1000.0
    lp = torch.from_numpy(logp).to(DEV)
    res = gpu_lib.grpo_token_loss(lp, lp.clone(), torch.from_numpy(ref).to(DEV),
                                  torch.ones(B, device=DEV), torch.ones((B, T), dtype=torch.bool, device=DEV),
                                  **kw)
    torch.cuda.synchronize()
    k3 = to_np(res.tok_kl)
    em1 = -to_np(res.grad)
    em1_x = np.expm1(d)
    k3_x = np.where(np.abs(d) < 1e-3, d * d * (0.5 + d / 6 + d * d / 24 + d ** 3 / 120), em1_x - d)
    u = 2.0 ** -24
    small = np.abs(d) < 1.0
    assert np.all(np.abs(k3 - k3_x)[small] <= 4 * u * k3_x[small]), float(np.max(np.abs(k3 - k3_x)[small] / k3_x[small]))
    assert np.all(np.abs(em1 - em1_x)[small] <= 4 * u * np.abs(em1_x)[small])
    big = ~small
    lim = 4 * u * (np.exp(d) * (np.abs(d) + 1) + np.abs(em1_x) + np.abs(k3_x))
    assert np.all(np.abs(k3 - k3_x)[big] <= lim[big])
    assert np.all(np.abs(em1 - em1_x)[big] <= lim[big])
    assert np.all(k3[d == 0] == 0) and np.all(em1[d == 0] == 0)
    assert np.all(k3 >= 0)


def test_two_streams_at_once(gpu_lib):
    """Calls on two streams with no synchronisation between them each get
    their own workspace (the binding keys it by stream), so both results
    equal the single-stream ones bit for bit: the fused logits call and the
    log-prob token loss."""
    wl = _wl(6000, "bf16", T=32, sizes=(4, 4, 4, 4))
    announce("two streams")
    _, a = _inputs(wl, seed=51)
    _, b = _inputs(wl, seed=52)
    ref_a, ref_b = _call(gpu_lib, a, wl), _call(gpu_lib, b, wl)
    lp = {k: torch.log_softmax(v["policy"].float(), -1).gather(-1, v["action_ids"][..., None])[..., 0]
          .contiguous() for k, v in (("a", a), ("b", b))}
    tok = {k: gpu_lib.grpo_token_loss(lp[k], v["old_logps"], lp[k], v["rewards"], v["mask"],
                                      **gpu_kwargs(wl)) for k, v in (("a", a), ("b", b))}
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    out = {"a": [], "b": []}
    for _ in range(4):
        for key, inp, s in (("a", a, s1), ("b", b, s2)):
            with torch.cuda.stream(s):
                r = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"],
                                              inp["old_logps"], inp["rewards"], inp["mask"],
                                              **gpu_kwargs(wl))
                t = gpu_lib.grpo_token_loss(lp[key], inp["old_logps"], lp[key], inp["rewards"],
                                            inp["mask"], **gpu_kwargs(wl))
                out[key].append((r, t))
    torch.cuda.synchronize()
    for key, ref, rt in (("a", ref_a, tok["a"]), ("b", ref_b, tok["b"])):
        for r, t in out[key]:
            assert torch.equal(_bits(r.scalars), _bits(ref.scalars)), key
            assert torch.equal(_bits(r.grad), _bits(ref.grad)), key
            assert torch.equal(_bits(t.scalars), _bits(rt.scalars)), key
            assert torch.equal(_bits(t.grad), _bits(rt.grad)), key
