"""Parity of the advantage estimators on the HIP path, through the C ABI,
against the fp64 oracle: REINFORCE++ returns and REINFORCE++-baseline token
advantages with the global masked normalization (Relax REINFORCE++ page),
GDPO multi-reward advantages and the advantage clamp (dockyard_rl, Advantage
estimation), and both loss entry points fed token advantages.

Bar for the estimators: both sides compute in binary64 and round once to
float32, but sums over slots run in different (fixed) orders, so a value
may land one float32 ulp away when its binary64 value sits next to a
rounding boundary: |gpu - oracle_f32| <= 1 ulp, with the bit-exact count
reported.  Group advantages with a clamp keep the sequential order of the
definition and are bit-exact."""

import math

import numpy as np
import pytest
import torch

import oracle
from _parity import (assert_bits_equal, cfg_from, compare_exact_parts, compare_logits_grad,
                     compare_scalars, compare_token_values, gpu_kwargs, host_inputs, to_np)
from workloads import TOKEN_WORKLOADS, LogitsWorkload, make_logits_inputs, make_token_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _within_ulp(gpu, ref64, what):
    r32 = np.asarray(ref64, dtype=np.float64).astype(np.float32)
    g = np.asarray(gpu, dtype=np.float32)
    ulp = np.spacing(np.abs(r32)).astype(np.float64)
    err = np.abs(g.astype(np.float64) - r32.astype(np.float64))
    bad = err > ulp
    assert not bad.any(), (f"{what}: {int(bad.sum())} values beyond 1 ulp, first at "
                           f"{np.argwhere(bad)[0]}: gpu={g[bad][0]!r} oracle={r32[bad][0]!r}")
    return int(np.sum(g.view(np.uint32) == r32.view(np.uint32))), g.size


def _token_case(B, T, seed, holes=True):
    g = torch.Generator().manual_seed(seed)
    lens = torch.randint(1, T + 1, (B,), generator=g)
    mask = torch.arange(T)[None, :] < lens[:, None]
    if holes:
        mask &= torch.rand((B, T), generator=g) > 0.15
        mask[:, 0] = True
    old = -torch.rand((B, T), generator=g) * 5.0
    ref = old + torch.randn((B, T), generator=g) * 0.3
    R = (torch.rand(B, generator=g) < 0.5).float() + 0.25 * torch.randn(B, generator=g)
    return mask, old, ref, R


TOKEN_CASES = [
    dict(estimator="reinforce_pp", kl_coef=0.01, gamma=1.0, normalize=True),
    dict(estimator="reinforce_pp", kl_coef=0.05, gamma=0.95, normalize=True),
    dict(estimator="reinforce_pp", kl_coef=0.05, gamma=0.9, normalize=False),
    dict(estimator="reinforce_pp", kl_coef=0.0, gamma=1.0, normalize=True, no_logps=True),
    dict(estimator="reinforce_pp_baseline", normalize=True, spp=4),
    dict(estimator="reinforce_pp_baseline", normalize=False, spp=4),
    dict(estimator="reinforce_pp_baseline", normalize=True, csr=[0, 2, 6, 8, 16]),
    dict(estimator="reinforce_pp_baseline", normalize=True, spp=4, adv_clip=(-1.0, 1.5)),
    dict(estimator="reinforce_pp", kl_coef=0.02, gamma=1.0, normalize=True, spp=4,
         adv_clip=(-0.8, 0.8)),
]


def _case_id(kw):
    return "-".join(f"{k}={v}" for k, v in kw.items())


@pytest.mark.parametrize("kw", TOKEN_CASES, ids=_case_id)
@pytest.mark.parametrize("T", [203, 4096, 5000, 5008])
def test_token_advantages(gpu_lib, kw, T):
    rpl = gpu_lib
    kw = dict(kw)
    B = 16
    mask, old, ref, R = _token_case(B, T, seed=T)
    no_logps = kw.pop("no_logps", False)
    spp = kw.pop("spp", None)
    csr = kw.pop("csr", None)
    adv_clip = kw.pop("adv_clip", None)
    announce(f"token advantages T={T} {kw} spp={spp} csr={csr} clip={adv_clip}")
    d = dict(mask=mask.to(DEV), old=old.to(DEV), ref=ref.to(DEV), R=R.to(DEV))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    A = rpl.grpo_token_advantages(kw["estimator"], d["R"], d["mask"],
                                  old_logps=None if no_logps else d["old"],
                                  ref_logps=None if no_logps else d["ref"],
                                  samples_per_prompt=spp, group_boundaries=csr,
                                  kl_coef=kw.get("kl_coef", 0.0), gamma=kw.get("gamma", 1.0),
                                  normalize=kw["normalize"], adv_clip=adv_clip, status=st)
    torch.cuda.synchronize()
    groups = None
    if spp is not None or csr is not None or adv_clip is not None:
        groups = dict(samples_per_prompt=spp) if spp is not None else dict(
            group_boundaries=csr if csr is not None else [0, B])
        if adv_clip is not None:
            groups.update(adv_clip_low=adv_clip[0], adv_clip_high=adv_clip[1])
    m = mask.numpy()
    want = oracle.token_advantages(kw["estimator"], R.numpy(), None if no_logps else old.numpy(),
                                   None if no_logps else ref.numpy(), m, groups=groups,
                                   kl_coef=kw.get("kl_coef", 0.0), gamma=kw.get("gamma", 1.0),
                                   normalize=kw["normalize"])
    got = A.cpu().numpy()
    assert np.all(got[~m] == 0.0)
    exact, n = _within_ulp(got, want, "token advantages")
    assert int(st[0]) == 0
    if adv_clip is not None:
        assert np.any(want[m] <= adv_clip[0]) or np.any(want[m] >= adv_clip[1])
    print(f"  bit-exact {exact}/{n}", flush=True)


def test_token_advantages_empty_mask(gpu_lib):
    rpl = gpu_lib
    B, T = 8, 64
    mask = torch.zeros((B, T), dtype=torch.bool, device=DEV)
    R = torch.ones(B, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    announce("token advantages empty mask")
    A = rpl.grpo_token_advantages("reinforce_pp_baseline", R, mask, samples_per_prompt=4,
                                  normalize=True, status=st)
    torch.cuda.synchronize()
    assert torch.all(A == 0) and int(st[0]) & rpl.GRPO_FAULT_NO_TOKENS


@pytest.mark.parametrize("T", [777, 776])   # single slots, quads of four slots
def test_token_advantages_bitwise_repeat_and_masked_garbage(gpu_lib, T):
    rpl = gpu_lib
    B = 12
    mask, old, ref, R = _token_case(B, T, seed=3)
    d = dict(mask=mask.to(DEV), old=old.to(DEV), ref=ref.to(DEV), R=R.to(DEV))
    announce(f"token advantages repeat / garbage T={T}")
    kw = dict(old_logps=d["old"], ref_logps=d["ref"], kl_coef=0.03, gamma=0.97)
    a = rpl.grpo_token_advantages("reinforce_pp", d["R"], d["mask"], **kw)
    b = rpl.grpo_token_advantages("reinforce_pp", d["R"], d["mask"], **kw)
    old2, ref2 = d["old"].clone(), d["ref"].clone()
    old2[~d["mask"]] = float("nan")
    ref2[~d["mask"]] = float("inf")
    c = rpl.grpo_token_advantages("reinforce_pp", d["R"], d["mask"], old_logps=old2, ref_logps=ref2,
                                  kl_coef=0.03, gamma=0.97)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    assert torch.equal(a.view(torch.int32), c.view(torch.int32))


@pytest.mark.parametrize("normalize", [True, False])
def test_token_advantages_unaligned_rows(gpu_lib, normalize):
    """T % 4 == 0 but log-prob and mask rows that start off a 16-byte (and
    4-byte) boundary: the returns kernel takes single slots instead of quads
    and still matches the oracle."""
    rpl = gpu_lib
    B, T = 16, 4096
    mask, old, ref, R = _token_case(B, T, seed=11)
    announce(f"token advantages unaligned rows normalize={normalize}")

    def shifted(x, k):
        buf = torch.empty(x.numel() + k, dtype=x.dtype, device=DEV)
        v = buf[k:].view(x.shape)
        v.copy_(x.to(DEV))
        return v

    o, r, mk = shifted(old, 1), shifted(ref, 3), shifted(mask, 1)
    assert o.data_ptr() % 16 and r.data_ptr() % 16 and mk.data_ptr() % 4
    A = rpl.grpo_token_advantages("reinforce_pp", R.to(DEV), mk, old_logps=o, ref_logps=r,
                                  kl_coef=0.02, gamma=1.0, normalize=normalize)
    torch.cuda.synchronize()
    want = oracle.token_advantages("reinforce_pp", R.numpy(), old.numpy(), ref.numpy(), mask.numpy(),
                                   kl_coef=0.02, gamma=1.0, normalize=normalize)
    got = A.cpu().numpy()
    assert np.all(got[~mask.numpy()] == 0.0)
    exact, n = _within_ulp(got, want, "token advantages, unaligned rows")
    print(f"  bit-exact {exact}/{n}", flush=True)


GDPO_CASES = [
    dict(C=2, spp=4),
    dict(C=3, spp=8, scale_by_std=False),
    dict(C=2, csr=[0, 2, 6, 12, 16]),
    dict(C=3, spp=4, adv_clip=(-1.2, 1.2)),
]


@pytest.mark.parametrize("kw", GDPO_CASES, ids=_case_id)
def test_gdpo_advantages(gpu_lib, kw):
    rpl = gpu_lib
    B = 16 if "csr" in kw else 64
    g = torch.Generator().manual_seed(B + kw["C"])
    comps = torch.stack([(torch.rand(B, generator=g) < 0.5).float(),
                         torch.randn(B, generator=g),
                         2.0 * torch.rand(B, generator=g)][: kw["C"]]).contiguous()
    gk = dict(samples_per_prompt=kw.get("spp"), group_boundaries=kw.get("csr"),
              scale_by_std=kw.get("scale_by_std", True), adv_clip=kw.get("adv_clip"))
    announce(f"GDPO {kw}")
    A = rpl.grpo_gdpo_advantages(comps.to(DEV), **gk)
    torch.cuda.synchronize()
    og = {k: v for k, v in dict(samples_per_prompt=kw.get("spp"), group_boundaries=kw.get("csr"),
                                leave_one_out=True, scale_by_std=kw.get("scale_by_std", True)).items()
          if v is not None}
    if "adv_clip" in kw:
        og.update(adv_clip_low=kw["adv_clip"][0], adv_clip_high=kw["adv_clip"][1])
    want = oracle.gdpo_advantages(comps.numpy(), groups=og)
    exact, n = _within_ulp(A.cpu().numpy(), want, "GDPO")
    print(f"  bit-exact {exact}/{n}", flush=True)


@pytest.mark.parametrize("estimator", ["reinforce_pp", "reinforce_pp_baseline"])
def test_token_advantages_fullsize(gpu_lib, estimator):
    """The benchmarked configuration, compared whole: B = 1024 in groups of
    16, T = 4096, ragged lengths, normalized (REINFORCE++: k1 shaping 0.01,
    gamma 1).  Then the same call captured in a HIP graph and replayed,
    with eager calls on other inputs in between: every replay bit-identical
    to the eager result."""
    rpl = gpu_lib
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    announce(f"token advantages full size {estimator}: generating")
    a = make_token_inputs(wl, device=DEV, seed=0)
    b = make_token_inputs(wl, device=DEV, seed=1)
    if estimator == "reinforce_pp":
        kw = dict(kl_coef=0.01, gamma=1.0, normalize=True)
        extra = lambda c: dict(old_logps=c["old_logps"], ref_logps=c["ref_logp"])  # noqa: E731
        groups = None
    else:
        kw = dict(samples_per_prompt=wl.group_size, normalize=True)
        extra = lambda c: {}  # noqa: E731
        groups = dict(samples_per_prompt=wl.group_size)
    got = rpl.grpo_token_advantages(estimator, a["rewards"], a["mask"], **extra(a), **kw)
    torch.cuda.synchronize()
    announce(f"token advantages full size {estimator}: oracle")
    h = {k: v.cpu().numpy() for k, v in a.items()}
    want = oracle.token_advantages(estimator, h["rewards"], h["old_logps"], h["ref_logp"],
                                   h["mask"], groups=groups, kl_coef=kw.get("kl_coef", 0.0),
                                   gamma=kw.get("gamma", 1.0), normalize=True)
    g = got.cpu().numpy()
    assert np.all(g[~h["mask"]] == 0.0)
    exact, n = _within_ulp(g, want, f"full size {estimator}")
    print(f"  bit-exact {exact}/{n}", flush=True)

    announce(f"token advantages full size {estimator}: graph replays")
    static = {k: v.clone() for k, v in a.items()}
    box = {}

    def call():
        box["A"] = rpl.grpo_token_advantages(estimator, static["rewards"], static["mask"],
                                             **extra(static), **kw)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        call()
    eager_b = rpl.grpo_token_advantages(estimator, b["rewards"], b["mask"], **extra(b), **kw)
    torch.cuda.synchronize()
    for rep in range(4):
        src, ref = (a, got) if rep % 2 == 0 else (b, eager_b)
        for k in static:
            static[k].copy_(src[k])
        graph.replay()
        junk = rpl.grpo_token_advantages(estimator, b["rewards"], a["mask"], **extra(b), **kw)
        torch.cuda.synchronize()
        assert torch.equal(box["A"].view(torch.int32), ref.view(torch.int32)), rep
        del junk


def test_group_advantage_clamp_bit_exact(gpu_lib):
    rpl = gpu_lib
    B = 4096
    g = torch.Generator().manual_seed(5)
    r = torch.randn(B, generator=g)
    announce("group advantages with clamp")
    for kw in (dict(samples_per_prompt=8), dict(samples_per_prompt=4, leave_one_out=True)):
        A = rpl.grpo_advantages(r.to(DEV), adv_clip=(-0.9, 1.1), **kw)
        torch.cuda.synchronize()
        want = oracle.grpo_advantages(r.numpy(), groups=dict(kw, adv_clip_low=-0.9,
                                                             adv_clip_high=1.1))
        assert_bits_equal(A.cpu().numpy(), want, "clamped advantages")
        assert np.any(want == -0.9) and np.any(want == 1.1)


def _wl(V, dtype, T=16, sizes=(4, 4, 4, 4)):
    return LogitsWorkload(name=f"tokadv_V{V}_{dtype}", group_sizes=sizes, T=T, V=V, dtype=dtype,
                          logit_std=2.0, ref_noise_std=math.sqrt(0.1), old_noise_std=0.5,
                          reward_p=0.5, len_range=(1, T), beta=0.05)


@pytest.mark.parametrize("estimator", ["reinforce_pp", "reinforce_pp_baseline"])
@pytest.mark.parametrize("V,dtype", [(1000, "f32"), (4097, "bf16"), (151936, "bf16")])
def test_loss_with_token_advantages(gpu_lib, estimator, V, dtype):
    """The recipes end to end: the oracle's token advantages (rounded to
    float32) feed both the GPU loss and the oracle loss; the GPU estimator's
    own advantages then give the same loss within the loss bar."""
    rpl = gpu_lib
    wl = _wl(V, dtype, T=6 if V > 100000 else 16, sizes=(4, 4) if V > 100000 else (4, 4, 4, 4))
    announce(f"loss with token advantages {estimator} V={V} {dtype}")
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=V)
    h = host_inputs(inp_cpu)
    y = h["ref"]
    ids = h["action_ids"]
    lse = np.log(np.sum(np.exp(y - y.max(-1, keepdims=True)), -1)) + y.max(-1)
    ref_lp = (np.take_along_axis(y, ids[..., None], -1)[..., 0] - lse).astype(np.float32)
    if estimator == "reinforce_pp":
        A = oracle.token_advantages(estimator, h["rewards"], h["old_logps"], ref_lp, h["mask"],
                                    kl_coef=0.01, gamma=1.0)
        cfg = oracle.LossConfig(eps_low=0.2, eps_high=0.2, beta=0.0, reduction="sequence_mean")
        kw = dict(beta=0.0, reduction="sequence_mean")
        ref_logits = None
    else:
        A = oracle.token_advantages(estimator, h["rewards"], None, None, h["mask"],
                                    groups=dict(samples_per_prompt=4))
        cfg = oracle.LossConfig(eps_low=0.2, eps_high=0.2, beta=0.01, kl_estimator="k2",
                                reduction="sequence_mean")
        kw = dict(beta=0.01, kl_estimator="k2", reduction="sequence_mean")
        ref_logits = inp_cpu["ref"].to(DEV)
    A32 = A.astype(np.float32)
    ref = oracle.grpo_loss_fwd_bwd(h["policy"], None if ref_logits is None else h["ref"], ids,
                                   h["old_logps"], h["mask"], None, groups=None, cfg=cfg,
                                   advantages=A32.astype(np.float64))
    d = {k: v.to(DEV) for k, v in inp_cpu.items()}
    res = rpl.grpo_loss_fwd_bwd(d["policy"], ref_logits, d["action_ids"], d["old_logps"], None,
                                d["mask"], token_advantages=torch.from_numpy(A32).to(DEV),
                                per_token=True, **kw)
    torch.cuda.synchronize()
    rtol = 1e-5 if dtype == "f32" else 1e-4
    assert_bits_equal(to_np(res.seq_weight), ref.seq_weight, "seq_weight")
    compare_scalars(res, ref, cfg, rtol, estimator)
    compare_token_values(res, ref, cfg, h["mask"], rtol)
    compare_logits_grad(to_np(res.grad), ref, cfg, h["mask"], dtype, estimator,
                        policy=h["policy"], ids=ids)
    # the GPU estimator's advantages in the same call
    if estimator == "reinforce_pp":
        Ag = rpl.grpo_token_advantages(estimator, d["rewards"], d["mask"], old_logps=d["old_logps"],
                                       ref_logps=torch.from_numpy(ref_lp).to(DEV), kl_coef=0.01)
    else:
        Ag = rpl.grpo_token_advantages(estimator, d["rewards"], d["mask"], samples_per_prompt=4)
    res2 = rpl.grpo_loss_fwd_bwd(d["policy"], ref_logits, d["action_ids"], d["old_logps"], None,
                                 d["mask"], token_advantages=Ag, **kw)
    torch.cuda.synchronize()
    assert abs(float(res2.loss) - ref.loss) <= rtol * abs(ref.loss) + 1e-6 * rtol


@pytest.mark.parametrize("T", [256, 203])
def test_token_loss_with_token_advantages(gpu_lib, T):
    """Log-prob entry point (vector and scalar paths) with per-token advantages."""
    rpl = gpu_lib
    B = 24
    mask, old, ref, R = _token_case(B, T, seed=11, holes=False)
    g = torch.Generator().manual_seed(12)
    logp = old + 0.3 * torch.randn((B, T), generator=g)
    A = oracle.token_advantages("reinforce_pp_baseline", R.numpy(), None, None, mask.numpy(),
                                groups=dict(samples_per_prompt=4)).astype(np.float32)
    announce(f"token loss with token advantages T={T}")
    res = rpl.grpo_token_loss(logp.to(DEV), old.to(DEV), ref.to(DEV), None, mask.to(DEV),
                              token_advantages=torch.from_numpy(A).to(DEV), beta=0.01,
                              kl_estimator="k2", reduction="sequence_mean", per_token=True)
    torch.cuda.synchronize()
    cfg = oracle.LossConfig(beta=0.01, kl_estimator="k2", reduction="sequence_mean")
    want = oracle.grpo_token_loss(logp.numpy(), old.numpy(), ref.numpy(), mask.numpy(), None,
                                  groups=None, cfg=cfg, advantages=A.astype(np.float64))
    compare_scalars(res, want, cfg, 1e-5, "token loss")
    g_ = to_np(res.grad)
    assert np.all(np.abs(g_ - want.grad) <= 1e-5 * np.max(np.abs(want.grad)) + 1e-30)
