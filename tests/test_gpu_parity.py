"""Parity of the HIP path (through the C ABI) against the fp64 oracle.

Sizes here let the oracle finish in seconds while still spanning several
vector chunks per thread, ragged masks, vector tails and the scalar path.
Full-size workloads are covered by tests/test_gpu_fullsize.py.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from _parity import (assert_bits_equal, cfg_from, compare_exact_parts, compare_logits_grad,
                     compare_scalars, compare_token_grad, gpu_kwargs, host_inputs, to_np)
from workloads import (TOKEN_WORKLOADS, WORKLOADS, LogitsWorkload, make_logits_inputs,
                       make_token_inputs, poison_masked)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def run_logits(rpl, inp, wl, reduction=None, **extra):
    kw = gpu_kwargs(wl, reduction)
    kw.update(extra)
    res = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                inp["rewards"], inp["mask"], per_token=True, **kw)
    torch.cuda.synchronize()
    return res


def oracle_logits(h, wl, reduction=None, with_ref=True):
    return oracle.grpo_loss_fwd_bwd(h["policy"], h["ref"] if with_ref else None, h["action_ids"],
                                    h["old_logps"], h["mask"], h["rewards"],
                                    groups=wl.groups_kwargs(), cfg=cfg_from(wl, reduction))


def check_logits_case(rpl, wl, seed=0, reduction=None, empty=()):
    """``empty``: sequences whose whole mask row is cleared first."""
    announce(f"logits parity {wl.name} reduction={reduction or wl.reductions[0]} seed={seed}"
             + (f" empty={list(empty)}" if empty else ""))
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=seed)
    for i in empty:
        inp_cpu["mask"][i] = False
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    res = run_logits(rpl, inp, wl, reduction)
    h = host_inputs(inp_cpu)
    ref = oracle_logits(h, wl, reduction)
    cfg = cfg_from(wl, reduction)
    compare_exact_parts(res, ref, wl.name)
    half = wl.dtype != "f32"
    compare_scalars(res, ref, cfg, 1e-4 if half else 1e-5, wl.name)
    stats = compare_logits_grad(to_np(res.grad), ref, cfg, h["mask"], wl.dtype, wl.name)
    clipped = int(to_np(res.counts)[1])
    assert abs(clipped - ref.clipped) <= stats["ambiguous"], (clipped, ref.clipped, stats)
    st = int(to_np(res.status)[0])
    assert st == 0, f"status bits {st}"
    print(f"  stats {stats} clipped gpu={clipped} oracle={ref.clipped}", flush=True)
    return res, ref


def test_tiny_logits_workload(gpu_lib):
    check_logits_case(gpu_lib, WORKLOADS["tiny_logits"])


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tiny_logits_more_seeds(gpu_lib, seed):
    check_logits_case(gpu_lib, WORKLOADS["tiny_logits"], seed=seed)


def test_v32000_recipe_reduced(gpu_lib):
    check_logits_case(gpu_lib, WORKLOADS["logits_v32000"].scaled(T=32, prompts=2))


def test_v151936_recipe_reduced(gpu_lib):
    check_logits_case(gpu_lib, WORKLOADS["logits_v151936"].scaled(T=12, prompts=1))


@pytest.mark.parametrize("reduction", ["token_mean", "sequence_mean", "length_alpha"])
def test_csr_v128256_recipe_reduced(gpu_lib, reduction):
    check_logits_case(gpu_lib, WORKLOADS["logits_csr_v128256"].scaled(T=8, prompts=3),
                      reduction=reduction)


def _custom(V, dtype="bf16", T=6, sizes=(4, 4), **kw):
    base = dict(name=f"custom_V{V}_{dtype}", group_sizes=sizes, T=T, V=V, dtype=dtype,
                logit_std=2.0, ref_noise_std=math.sqrt(0.1), old_noise_std=math.sqrt(0.05),
                reward_p=0.5, len_range=(1, T))
    base.update(kw)
    return LogitsWorkload(**base)


@pytest.mark.parametrize("V,dtype", [
    (1, "f32"), (2, "bf16"), (7, "f32"), (64, "bf16"), (1000, "bf16"), (1000, "f32"),
    (2048, "f32"), (4097, "bf16"), (8200, "bf16"), (40000, "f32"), (70001, "bf16"),
])
def test_vocab_sizes_and_paths(gpu_lib, V, dtype):
    """Wave-per-row, block-per-row, vector and scalar paths, ragged tails."""
    check_logits_case(gpu_lib, _custom(V, dtype))


@pytest.mark.parametrize("V,dtype", [
    (2048, "bf16"), (2056, "bf16"),        # 4 KB rows: wave per row, then a resident block
    (8192, "bf16"), (8200, "bf16"),        # 16 KB: resident at 256 threads (4 chunks), then 512
    (32768, "bf16"), (32776, "bf16"),      # 64 KB: 512 threads x 8 chunks, then 12
    (49152, "bf16"), (49160, "bf16"),      # 96 KB: 512 threads x 12 chunks, then 16
    (65536, "bf16"), (65544, "bf16"),      # 128 KB: the largest resident row, then streaming
    (4096, "f32"), (4100, "f32"),          # the same limits for float32 rows
    (16384, "f32"), (16388, "f32"),
    (24576, "f32"), (24580, "f32"),
    (32768, "f32"), (32772, "f32"),
])
def test_kernel_variant_boundaries(gpu_lib, V, dtype):
    """Row sizes exactly at each kernel variant's limit and one chunk past
    it, so that both sides of every switch in the row-kernel choice run."""
    check_logits_case(gpu_lib, _custom(V, dtype, T=4, sizes=(4, 4)), seed=9)


@pytest.mark.parametrize("V,dtype", [(40000, "bf16"), (20001 * 4 // 4, "f32")])
def test_many_rows_per_block(gpu_lib, V, dtype):
    """More rows than compute units, ragged masks: each persistent block walks
    several rows and skips (zero-fills) the masked ones between them."""
    wl = _custom(V, dtype, T=64, sizes=(8, 8), len_range=(1, 64))
    check_logits_case(gpu_lib, wl, seed=21)


@pytest.mark.parametrize("V", [1000, 4097, 40000, 151936])
def test_f16_logits_and_gradient(gpu_lib, V):
    """IEEE half logits and gradient on every row-kernel path: wave per row,
    block per row with a scalar tail, resident, streaming."""
    T = 6 if V > 100000 else 16
    check_logits_case(gpu_lib, _custom(V, "f16", T=T), seed=3)


def test_f16_logits_f32_gradient(gpu_lib):
    wl = _custom(5000, "f16", T=8)
    announce("f16 logits -> f32 grad")
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=12)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                    inp["rewards"], inp["mask"], grad_dtype=torch.float32,
                                    **gpu_kwargs(wl))
    torch.cuda.synchronize()
    assert res.grad.dtype == torch.float32
    h = host_inputs(inp_cpu)
    r = oracle_logits(h, wl)
    compare_scalars(res, r, cfg_from(wl), 1e-4)
    compare_logits_grad(to_np(res.grad), r, cfg_from(wl), h["mask"], "f32")


@pytest.mark.parametrize("V,ld", [
    (4097, 4104),     # the vector path with a scalar tail
    (40000, 40008),   # 80 KB rows held at 512 threads x 12 chunks, padded 16-byte stride
    (60000, 60064),   # 120 KB rows held at 512 threads x 16 chunks
])
def test_padded_row_stride_vector_tail(gpu_lib, V, ld):
    """Rows padded to a 16-byte multiple: the row stride differs from V in
    the policy, reference and gradient, and the padding stays untouched."""
    rpl = gpu_lib
    wl = _custom(V, "bf16", T=5)
    announce(f"padded stride V={V} ld={ld}")
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=5)
    B, T, V = wl.B, wl.T, wl.V
    pol = torch.full((B, T, ld), float("nan"), dtype=torch.bfloat16)
    ref = torch.full((B, T, ld), float("inf"), dtype=torch.bfloat16)
    pol[..., :V] = inp_cpu["policy"]
    ref[..., :V] = inp_cpu["ref"]
    polg, refg = pol.to(DEV)[..., :V], ref.to(DEV)[..., :V]
    other = {k: v.to(DEV) for k, v in inp_cpu.items() if k not in ("policy", "ref")}
    gbuf = torch.full((B, T, ld), 7.0, dtype=torch.bfloat16, device=DEV)
    res = gpu_lib.grpo_loss_fwd_bwd(polg, refg, other["action_ids"], other["old_logps"],
                                    other["rewards"], other["mask"], grad_out=gbuf[..., :V],
                                    **gpu_kwargs(wl))
    torch.cuda.synchronize()
    assert torch.all(gbuf[..., V:] == 7.0), "padding of the gradient must stay untouched"
    h = host_inputs(inp_cpu)
    r = oracle_logits(h, wl)
    compare_exact_parts(res, r)
    compare_scalars(res, r, cfg_from(wl), 1e-4)
    compare_logits_grad(to_np(gbuf[..., :V]), r, cfg_from(wl), h["mask"], True)


def test_int32_ids_and_f32_grad_from_bf16(gpu_lib):
    wl = _custom(3000, "bf16", T=4)
    announce("int32 ids, bf16 logits -> f32 grad")
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=9)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    ids32 = inp["action_ids"].to(torch.int32)
    res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], ids32, inp["old_logps"],
                                    inp["rewards"], inp["mask"], grad_dtype=torch.float32,
                                    **gpu_kwargs(wl))
    torch.cuda.synchronize()
    assert res.grad.dtype == torch.float32
    h = host_inputs(inp_cpu)
    r = oracle_logits(h, wl)
    compare_scalars(res, r, cfg_from(wl), 1e-4)
    # float32 output: the tighter float32 criterion applies
    compare_logits_grad(to_np(res.grad), r, cfg_from(wl), h["mask"], False)


def test_no_reference_beta_zero(gpu_lib):
    wl = _custom(513, "f32", T=4, beta=0.0)
    announce("beta=0 without reference logits")
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=4)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    res = gpu_lib.grpo_loss_fwd_bwd(inp["policy"], None, inp["action_ids"], inp["old_logps"],
                                    inp["rewards"], inp["mask"], **gpu_kwargs(wl))
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    r = oracle_logits(h, wl, with_ref=False)
    compare_scalars(res, r, cfg_from(wl), 1e-5)
    assert float(res.kl) == 0.0
    compare_logits_grad(to_np(res.grad), r, cfg_from(wl), h["mask"], False)


# ---------------------------------------------------------------------------
# advantages and weights: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["bernoulli", "normal", "tiny_std"])
@pytest.mark.parametrize("loo", [False, True])
@pytest.mark.parametrize("scale", [True, False])
def test_advantages_bit_exact(gpu_lib, kind, loo, scale):
    announce(f"advantages {kind} loo={loo} scale={scale}")
    rng = np.random.default_rng(zlib.crc32(f"{kind}{loo}{scale}".encode()))
    sizes = [2, 3, 4, 5, 8, 16, 7, 64, 2, 31]
    off = [0] + list(np.cumsum(sizes))
    B = off[-1]
    if kind == "bernoulli":
        r = rng.integers(0, 2, B).astype(np.float32)
    elif kind == "normal":
        r = rng.normal(0.3, 1.7, B).astype(np.float32)
    else:
        r = (1.0 + rng.normal(0, 1e-7, B)).astype(np.float32)
    rt = torch.tensor(r, device=DEV)
    a = gpu_lib.grpo_advantages(rt, group_boundaries=off, leave_one_out=loo, scale_by_std=scale)
    torch.cuda.synchronize()
    ref = oracle.grpo_advantages(r, groups=dict(group_boundaries=off, leave_one_out=loo,
                                                scale_by_std=scale))
    assert_bits_equal(to_np(a), ref, "advantages")
    # uniform groups
    B2 = 8 * 16
    r2 = rng.normal(0, 1, B2).astype(np.float32)
    a2 = gpu_lib.grpo_advantages(torch.tensor(r2, device=DEV), samples_per_prompt=8,
                                 leave_one_out=loo, scale_by_std=scale)
    torch.cuda.synchronize()
    ref2 = oracle.grpo_advantages(r2, groups=dict(samples_per_prompt=8, leave_one_out=loo,
                                                  scale_by_std=scale))
    assert_bits_equal(to_np(a2), ref2, "advantages uniform")


def test_many_group_sqrt_and_division_bit_exact(gpu_lib):
    """Thousands of groups with random real rewards: every binary64 sqrt and
    division on the device must round exactly like numpy's."""
    announce("advantages 4096 groups")
    rng = np.random.default_rng(77)
    sizes = rng.integers(2, 20, 4096)
    off = [0] + list(np.cumsum(sizes))
    r = (rng.standard_normal(off[-1]) * rng.uniform(1e-3, 1e3)).astype(np.float32)
    a = gpu_lib.grpo_advantages(torch.tensor(r, device=DEV), group_boundaries=off)
    torch.cuda.synchronize()
    ref = oracle.grpo_advantages(r, groups=dict(group_boundaries=off))
    assert_bits_equal(to_np(a), ref, "advantages")


@pytest.mark.parametrize("reduction,alpha", [("token_mean", None), ("sequence_mean", None),
                                             ("length_alpha", 0.5), ("length_alpha", 0.0),
                                             ("length_alpha", 1.0)])
def test_weights_bit_exact(gpu_lib, reduction, alpha):
    announce(f"weights {reduction} alpha={alpha}")
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    inp_cpu = make_token_inputs(wl, device="cpu", seed=3, B=64, T=300)
    inp_cpu["mask"][5] = False  # an empty sequence
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    res = gpu_lib.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                                  inp["mask"], samples_per_prompt=16, reduction=reduction,
                                  alpha=alpha)
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    ref = oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"], h["rewards"],
                                 groups=dict(samples_per_prompt=16),
                                 cfg=oracle.LossConfig(reduction=reduction, alpha=alpha))
    compare_exact_parts(res, ref)


def test_weights_general_alpha_within_one_ulp(gpu_lib):
    announce("weights alpha=0.3")
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    inp_cpu = make_token_inputs(wl, device="cpu", seed=4, B=32, T=500)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    res = gpu_lib.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                                  inp["mask"], samples_per_prompt=16, reduction="length_alpha",
                                  alpha=0.3)
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    ref = oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"], h["rewards"],
                                 groups=dict(samples_per_prompt=16),
                                 cfg=oracle.LossConfig(reduction="length_alpha", alpha=0.3))
    g = to_np(res.seq_weight).astype(np.float32).view(np.int32).astype(np.int64)
    r = ref.seq_weight.astype(np.float32).view(np.int32).astype(np.int64)
    assert np.max(np.abs(g - r)) <= 1


# ---------------------------------------------------------------------------
# logprob-level token loss
# ---------------------------------------------------------------------------

def check_token_case(rpl, wl, B, T, seed=0, reduction=None):
    announce(f"token loss {wl.name} B={B} T={T} seed={seed}")
    inp_cpu = make_token_inputs(wl, device="cpu", seed=seed, B=B, T=T)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    red = reduction or wl.reduction
    res = rpl.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                              inp["mask"], eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
                              samples_per_prompt=wl.group_size, reduction=red, per_token=True)
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    cfg = oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=red)
    ref = oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"], h["rewards"],
                                 groups=dict(samples_per_prompt=wl.group_size), cfg=cfg)
    compare_exact_parts(res, ref)
    compare_scalars(res, ref, cfg, 1e-5)
    compare_token_grad(to_np(res.grad), ref, cfg, h["mask"].astype(bool), 1e-5, wl.name)
    return res, ref


def test_token_loss_small_full(gpu_lib):
    check_token_case(gpu_lib, TOKEN_WORKLOADS["token_loss_full"], B=64, T=257)


def test_token_loss_small_ragged(gpu_lib):
    check_token_case(gpu_lib, TOKEN_WORKLOADS["token_loss_ragged"], B=64, T=1000)


@pytest.mark.parametrize("T", [65536, 65537])
@pytest.mark.parametrize("name", ["token_loss_full", "token_loss_ragged"])
def test_token_loss_long_sequences(gpu_lib, name, T):
    """Sequences 16 times the benchmark's length: each block walks 16 rounds
    of its loads (vector path) or 257 strided steps (scalar path, odd T)
    before the sequence's reductions."""
    check_token_case(gpu_lib, TOKEN_WORKLOADS[name], B=16, T=T, seed=13)


@pytest.mark.parametrize("reduction", ["token_mean", "length_alpha"])
def test_token_loss_other_reductions(gpu_lib, reduction):
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    if reduction == "length_alpha":
        import dataclasses
        announce("token loss alpha")
        inp_cpu = make_token_inputs(wl, device="cpu", seed=8, B=32, T=128)
        inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
        res = gpu_lib.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"],
                                      inp["rewards"], inp["mask"], samples_per_prompt=16,
                                      reduction="length_alpha", alpha=0.5)
        torch.cuda.synchronize()
        h = host_inputs(inp_cpu)
        ref = oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"],
                                     h["rewards"], groups=dict(samples_per_prompt=16),
                                     cfg=oracle.LossConfig(reduction="length_alpha", alpha=0.5))
        compare_exact_parts(res, ref)
        compare_scalars(res, ref, oracle.LossConfig(reduction="length_alpha", alpha=0.5), 1e-5)
    else:
        check_token_case(gpu_lib, wl, B=32, T=130, reduction=reduction)


def test_token_loss_unaligned_scalar_path(gpu_lib):
    """T not a multiple of 4: the scalar path of the token kernel."""
    check_token_case(gpu_lib, TOKEN_WORKLOADS["token_loss_ragged"], B=32, T=131)


# ---------------------------------------------------------------------------
# the mean over live sequences ("GRPO Loss", Normalizer semantics,
# per_sequence_then_mean) and the page's reduction names
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("V,dtype", [(1000, "f32"), (8200, "bf16"), (40000, "bf16"),
                                     (70001, "bf16"), (151936, "bf16")])
def test_per_sequence_then_mean_logits(gpu_lib, V, dtype):
    """Fused logits call on each row-kernel path with two empty sequences:
    the weights bit-exact (1 / (B_live L_i), 0 for the empty ones), the
    scalars and every gradient row against the oracle."""
    check_logits_case(gpu_lib, _custom(V, dtype, T=6 if V < 100000 else 3, sizes=(4, 4)), seed=31,
                      reduction="per_sequence_then_mean", empty=(1, 5))


@pytest.mark.parametrize("T", [300, 301])
def test_per_sequence_then_mean_token_loss(gpu_lib, T):
    """Log-prob token loss (vector and scalar paths) with three empty
    sequences: the live count comes from the prep kernel's counts."""
    from _parity import compare_token_grad
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    announce(f"token loss per_sequence_then_mean T={T}")
    inp_cpu = make_token_inputs(wl, device="cpu", seed=5, B=64, T=T)
    inp_cpu["mask"][[3, 17, 40]] = False
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    res = gpu_lib.grpo_token_loss(inp["logp"], inp["old_logps"], inp["ref_logp"], inp["rewards"],
                                  inp["mask"], eps_low=wl.eps_low, eps_high=wl.eps_high,
                                  beta=wl.beta, samples_per_prompt=wl.group_size,
                                  reduction="per_sequence_then_mean", per_token=True)
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    cfg = oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
                            reduction="per_sequence_then_mean")
    ref = oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"], h["rewards"],
                                 groups=dict(samples_per_prompt=wl.group_size), cfg=cfg)
    w = to_np(res.seq_weight)
    assert np.all(w[[3, 17, 40]] == 0.0)
    compare_exact_parts(res, ref)
    compare_scalars(res, ref, cfg, 1e-5)
    compare_token_grad(to_np(res.grad), ref, cfg, h["mask"].astype(bool), 1e-5, "live mean")


def test_per_sequence_then_mean_autograd_split(gpu_lib):
    """grpo_loss (forward pass, then the gradient-only pass) under the live
    mean with empty sequences, against the oracle."""
    wl = _custom(40000, "bf16", T=6, sizes=(4, 4))
    red = "per_sequence_then_mean"
    announce("autograd split per_sequence_then_mean")
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=33)
    inp_cpu["mask"][[2, 6]] = False
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    pol = inp["policy"].clone().requires_grad_(True)
    loss, _, _ = gpu_lib.grpo_loss(pol, inp["ref"], inp["action_ids"], inp["old_logps"],
                                   inp["rewards"], inp["mask"], **gpu_kwargs(wl, red))
    loss.backward()
    torch.cuda.synchronize()
    h = host_inputs(inp_cpu)
    ref = oracle_logits(h, wl, red)
    cfg = cfg_from(wl, red)
    assert abs(float(loss.detach()) - ref.loss) <= 1e-4 * abs(ref.loss)
    compare_logits_grad(to_np(pol.grad), ref, cfg, h["mask"], "bf16", "live mean split")


def test_reduction_names_of_the_loss_page(gpu_lib):
    """'global_active_tokens' is the token mean under another name: the
    same bits; 'per_sequence_then_mean' equals the sequence mean when no
    sequence is empty."""
    wl = _custom(3000, "bf16", T=6, sizes=(4, 4))
    announce("reduction names")
    inp_cpu = make_logits_inputs(wl, device="cpu", seed=35)
    inp = {k: v.to(DEV) for k, v in inp_cpu.items()}
    assert bool(inp["mask"].any(dim=1).all())
    a = run_logits(gpu_lib, inp, wl, "token_mean")
    b = run_logits(gpu_lib, inp, wl, "global_active_tokens")
    assert torch.equal(a.scalars.view(torch.int32), b.scalars.view(torch.int32))
    assert torch.equal(a.grad.view(torch.int16), b.grad.view(torch.int16))
    c = run_logits(gpu_lib, inp, wl, "sequence_mean")
    d = run_logits(gpu_lib, inp, wl, "per_sequence_then_mean")
    assert torch.equal(c.scalars.view(torch.int32), d.scalars.view(torch.int32))
    assert torch.equal(c.grad.view(torch.int16), d.grad.view(torch.int16))
