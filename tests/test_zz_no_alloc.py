"""The entry point without a workspace argument (grpo_loss_fwd_bwd_noalloc,
for callers that cannot allocate) against grpo_loss_fwd_bwd with a caller's
workspace: every output bit-identical, on two calls in a row whose second is
smaller (the scratch array keeps the first call's contents), and sizes
beyond the scratch array refused."""

import pytest
import torch

from rl_post_loss_amd import GrpoError, _abi
from workloads import WORKLOADS, make_logits_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def announce(msg):
    print(f"[gpu-case] {msg}", flush=True)


def _kw(wl, reduction=None):
    red = reduction or wl.reductions[0]
    kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=red,
              alpha=wl.alpha if red == "length_alpha" else None)
    kw.update(wl.groups_kwargs())
    return kw


def _bits(t):
    return t.view({4: torch.int32, 2: torch.int16, 8: torch.int64}[t.element_size()])


def _same(a, b, what):
    for name in ("scalars", "advantages", "seq_policy", "seq_kl", "seq_weight", "seq_tokens",
                 "counts", "status", "tok_logp", "tok_loss", "tok_kl", "grad"):
        x, y = getattr(a, name), getattr(b, name)
        assert torch.equal(_bits(x), _bits(y)), f"{what}: {name} differs"


def _check(rpl, wl, reduction=None, seed=0):
    what = f"{wl.name} {reduction or wl.reductions[0]}"
    announce(f"no-alloc vs workspace call: {what} B={wl.B} T={wl.T} V={wl.V}")
    inp = make_logits_inputs(wl, device=DEV, seed=seed)
    args = (inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"], inp["rewards"],
            inp["mask"])
    want = rpl.grpo_loss_fwd_bwd(*args, per_token=True, **_kw(wl, reduction))
    got = rpl.grpo_loss_fwd_bwd_noalloc(*args, per_token=True, **_kw(wl, reduction))
    torch.cuda.synchronize()
    assert got.provenance["entry"] == "grpo_loss_fwd_bwd_noalloc"
    _same(got, want, what)
    return got


def test_noalloc_matches_workspace_entry_two_calls(gpu_lib):
    """A full-size call (B = 64, T = 1024, V = 32,000 bf16, ragged: 1.9 MB of
    workspace) and then a smaller one (B = 8, T = 16, V = 32 f32)."""
    _check(gpu_lib, WORKLOADS["logits_v32000"])
    _check(gpu_lib, WORKLOADS["tiny_logits"])


def test_noalloc_csr_groups_and_reductions(gpu_lib):
    """CSR groups (the offsets copied into the scratch array), four
    reductions in a row, each smaller than the one before."""
    wl = WORKLOADS["logits_csr_v128256"]
    for red, T in (("token_mean", 24), ("sequence_mean", 12), ("length_alpha", 5),
                   ("per_sequence_then_mean", 3)):
        _check(gpu_lib, wl.scaled(T=T, prompts=4 if T > 12 else 3), reduction=red, seed=T)


def test_noalloc_refuses_sizes_beyond_the_scratch(gpu_lib):
    lib = gpu_lib.load_library()
    B, T = 1024, 4096
    assert lib.grpo_workspace_bytes(B, T, 0) > _abi.NOALLOC_SCRATCH_BYTES
    announce("no-alloc refusal B=1024 T=4096 V=1")
    x = torch.zeros((B, T, 1), dtype=torch.float32, device=DEV)
    ids = torch.zeros((B, T), dtype=torch.int64, device=DEV)
    old = torch.zeros((B, T), dtype=torch.float32, device=DEV)
    r = torch.zeros(B, dtype=torch.float32, device=DEV)
    with pytest.raises(GrpoError) as e:
        gpu_lib.grpo_loss_fwd_bwd_noalloc(x, x, ids, old, r, None, samples_per_prompt=16)
    assert e.value.code == 6
