"""Host-side checks of the C ABI that run without a GPU: the library loads,
exports every function include/grpo.h declares, sizes its workspace, and
rejects invalid arguments before launching anything."""

import ctypes as C
import os
import re
import subprocess

import pytest
import torch

import rl_post_loss_amd as rpl
from rl_post_loss_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grpo.h")

# Argument-validation tests pass fake device addresses; they must never be able
# to reach a kernel launch on a machine with a GPU, so they run on CPU hosts only.
cpu_only = pytest.mark.skipif(torch.cuda.is_available(), reason="host-validation tests use fake pointers")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"GRPO_API\s+[\w\s\*]*?\b(grpo_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("grpo_advantages", "grpo_token_loss", "grpo_loss_fwd_bwd", "grpo_loss_bwd",
                 "grpo_token_advantages", "grpo_gdpo_advantages",
                 "grpo_workspace_bytes", "grpo_workspace_init", "grpo_status_str",
                 "grpo_abi_version", "grpo_set_timing_events"):
        assert name in fns
    assert set(fns) == set(_abi.SIGNATURES), "binding and header disagree"


def test_library_loads_and_exports_every_symbol():
    lib = rpl.load_library()
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.grpo_abi_version() == _abi.GRPO_ABI_VERSION


def test_status_strings():
    lib = rpl.load_library()
    for code in range(0, 9):
        assert lib.grpo_status_str(code)
    assert lib.grpo_status_str(99) == b"unknown status"


def test_workspace_bytes():
    lib = rpl.load_library()
    a = lib.grpo_workspace_bytes(32, 2048, 0)
    b = lib.grpo_workspace_bytes(32, 2048, 12)
    assert a > 32 * 2048 * 24 and a % 256 == 0 and b >= a
    assert lib.grpo_workspace_bytes(0, 10, 0) == 0
    assert lib.grpo_workspace_bytes(10, -1, 0) == 0
    assert lib.grpo_workspace_bytes(1 << 40, 1 << 40, 0) == 0


def _groups(spp=4, bounds=None, loo=0, scale=1, eps=1e-6):
    g = _abi.GrpoGroups()
    g.samples_per_prompt = spp
    keep = None
    if bounds is not None:
        keep = (C.c_int64 * len(bounds))(*bounds)
        g.group_boundaries = C.cast(keep, C.POINTER(C.c_int64))
        g.num_groups = len(bounds) - 1
    g.leave_one_out, g.scale_by_std, g.std_eps = loo, scale, eps
    return g, keep


def _cfg(lo=0.2, hi=0.2, beta=0.04, red=0, alpha=0.0, **extra):
    c = _abi.GrpoCfg()
    c.eps_low, c.eps_high, c.beta, c.reduction, c.alpha = lo, hi, beta, red, alpha
    c.sapo_tau_pos = c.sapo_tau_neg = 1.0
    for k, v in extra.items():
        setattr(c, k, v)
    return c


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors have the C compiler's sizes and field offsets."""
    structs = {"grpo_groups": _abi.GrpoGroups, "grpo_cfg": _abi.GrpoCfg,
               "grpo_outputs": _abi.GrpoOutputs}
    lines = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append(f'printf("{name} %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{name}.{f} %zu\\n", offsetof({name}, {f}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-o", str(exe), str(src)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], check=True, capture_output=True,
                                                        text=True).stdout.splitlines())
    for name, cls in structs.items():
        assert int(out[name]) == C.sizeof(cls), name
        for f, _ in cls._fields_:
            assert int(out[f"{name}.{f}"]) == getattr(cls, f).offset, f"{name}.{f}"


FAKE = 0x10000000          # never dereferenced: every call below fails validation first
FAKE_WS = 0x20000000


def _fwd(lib, B=8, T=4, V=32, g=None, cfg=None, ref=FAKE, grad=FAKE + 0x4000000, ws=FAKE_WS,
         ws_bytes=1 << 30, ld=None, gld=None, dtype=0, gdtype=0, ids_dtype=0, scalars=FAKE,
         gen=None, rewards=FAKE, tadv=None, no_groups=False):
    if g is None:
        g, _ = _groups()
    cfg = cfg or _cfg()
    o = _abi.GrpoOutputs()
    o.scalars = scalars
    return lib.grpo_loss_fwd_bwd(FAKE, ref, dtype, ld or V, FAKE, ids_dtype, FAKE, gen, None,
                                 rewards, tadv, B, T, V, None if no_groups else C.byref(g),
                                 C.byref(cfg), grad, gdtype, gld or V, None,
                                 C.byref(o), ws, ws_bytes, None)


@cpu_only
def test_fwd_bwd_argument_validation():
    lib = rpl.load_library()
    E = {v: k for k, v in _abi.STATUS_NAMES.items()}
    assert _fwd(lib, scalars=None) == E["GRPO_ERR_NULL"]
    assert _fwd(lib, B=0) == E["GRPO_ERR_SHAPE"]
    assert _fwd(lib, V=0) == E["GRPO_ERR_SHAPE"]
    assert _fwd(lib, ld=16) == E["GRPO_ERR_SHAPE"]          # row stride < V
    assert _fwd(lib, gld=16) == E["GRPO_ERR_SHAPE"]
    # a block per row: B*T above 2^31 - 1 rows is refused, not truncated
    assert _fwd(lib, B=1 << 16, T=1 << 15, V=1) == E["GRPO_ERR_SHAPE"]
    assert lib.grpo_loss_bwd(FAKE, 0, 1, FAKE, 0, None, 1 << 16, 1 << 15, 1, FAKE + 0x4000000, 0, 1,
                             None, FAKE_WS, 1 << 30, None) == E["GRPO_ERR_SHAPE"]
    assert _fwd(lib, dtype=7) == E["GRPO_ERR_DTYPE"]
    assert _fwd(lib, gdtype=9) == E["GRPO_ERR_DTYPE"]
    assert _fwd(lib, ids_dtype=3) == E["GRPO_ERR_DTYPE"]
    assert _fwd(lib, dtype=1, gdtype=2) == E["GRPO_ERR_DTYPE"]      # bf16 logits -> f16 grad
    assert _fwd(lib, dtype=0, gdtype=2) == E["GRPO_ERR_DTYPE"]      # f32 logits -> f16 grad
    assert _fwd(lib, dtype=2, gdtype=1) == E["GRPO_ERR_DTYPE"]      # f16 logits -> bf16 grad
    # groups: neither, both, B % spp, bad CSR, singleton
    g, _ = _groups(spp=0)
    assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"]
    g, keep = _groups(spp=4, bounds=[0, 4, 8])
    assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"]
    g, _ = _groups(spp=3)
    assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"]
    for bad in ([0, 4, 7], [1, 4, 8], [0, 5, 4, 8], [0, 1, 8], [0, 8, 8]):
        g, keep = _groups(spp=0, bounds=bad)
        assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"], bad
    g, _ = _groups(spp=1)
    assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"]
    g, _ = _groups(eps=0.0)
    assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"]
    g, _ = _groups()
    g.clip_advantages, g.adv_clip_low, g.adv_clip_high = 1, 1.0, -1.0    # low > high
    assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"]
    g.clip_advantages, g.adv_clip_low, g.adv_clip_high = 1, -float("inf"), 1.0
    assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"]
    g.clip_advantages = 2
    assert _fwd(lib, g=g) == E["GRPO_ERR_GROUPS"]
    # advantage source: exactly one of rewards (with groups) or token advantages
    assert _fwd(lib, rewards=None) == E["GRPO_ERR_NULL"]
    assert _fwd(lib, tadv=FAKE) == E["GRPO_ERR_CONFIG"]                       # and rewards
    assert _fwd(lib, tadv=FAKE, rewards=None) == E["GRPO_ERR_CONFIG"]         # and groups
    assert _fwd(lib, tadv=FAKE, rewards=None, no_groups=True,
                cfg=_cfg(pg_loss=5, red=1)) == E["GRPO_ERR_CONFIG"]          # sequence-level
    # config
    assert _fwd(lib, cfg=_cfg(lo=1.0)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(lo=-0.1)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(hi=-0.1)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(beta=-1.0)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(beta=float("nan"))) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(beta=0.1), ref=None) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(red=5)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(red=2, alpha=1.5)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(red=3)) == E["GRPO_ERR_CONFIG"]             # no norm_constant
    assert _fwd(lib, cfg=_cfg(red=3, norm_constant=float("inf"))) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(pg_loss=7)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(pg_loss=-1)) == E["GRPO_ERR_CONFIG"]
    # sequence-level losses: GSPO excludes the token mean and the dual clip;
    # REAL needs the token mean, a positive temperature and no gen_logps
    assert _fwd(lib, cfg=_cfg(pg_loss=5)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(pg_loss=5, red=1, dual_clip_c=3.0)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(pg_loss=6, red=1, real_tau=0.5)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(pg_loss=6, real_tau=0.0)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(pg_loss=6, real_tau=float("inf"))) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(pg_loss=6, real_tau=0.5), gen=FAKE) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(kl_estimator=3)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(dual_clip_c=1.0)) == E["GRPO_ERR_CONFIG"]    # needs c > 1
    assert _fwd(lib, cfg=_cfg(dual_clip_c=3.0, pg_loss=1)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(pg_loss=2, sapo_tau_neg=0.0)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(kl_input_clamp=-1.0)) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(kl_output_clamp=float("nan"))) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(tis_type=1, tis_ratio_max=2.0)) == E["GRPO_ERR_CONFIG"]  # no gen
    assert _fwd(lib, cfg=_cfg(tis_type=4, tis_ratio_max=2.0), gen=FAKE) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(tis_type=3, tis_ratio_max=2.0)) == E["GRPO_ERR_CONFIG"]   # no gen
    assert _fwd(lib, cfg=_cfg(tis_type=3, tis_ratio_min=0.5, tis_ratio_max=2.0, pg_loss=5, red=1),
                gen=FAKE) == E["GRPO_ERR_CONFIG"]                   # not with sequence ratios
    assert _fwd(lib, cfg=_cfg(tis_type=2, tis_ratio_max=0.0), gen=FAKE) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(tis_type=2, tis_ratio_min=3.0, tis_ratio_max=2.0),
                gen=FAKE) == E["GRPO_ERR_CONFIG"]
    assert _fwd(lib, cfg=_cfg(tis_type=1, tis_ratio_min=-1.0, tis_ratio_max=2.0),
                gen=FAKE) == E["GRPO_ERR_CONFIG"]
    # aliasing: in place with another dtype or stride, partial overlap
    assert _fwd(lib, grad=FAKE, gdtype=1) == E["GRPO_ERR_ALIAS"]
    assert _fwd(lib, grad=FAKE + 64) == E["GRPO_ERR_ALIAS"]
    assert _fwd(lib, grad=FAKE + 64, ref=FAKE + 0x4000000 + 64) == E["GRPO_ERR_ALIAS"]
    # workspace: null, misaligned, too small
    assert _fwd(lib, ws=None) == E["GRPO_ERR_WORKSPACE"]
    assert _fwd(lib, ws=FAKE_WS + 8) == E["GRPO_ERR_WORKSPACE"]
    assert _fwd(lib, ws_bytes=100) == E["GRPO_ERR_WORKSPACE"]


@cpu_only
def test_token_loss_and_advantages_validation():
    lib = rpl.load_library()
    E = {v: k for k, v in _abi.STATUS_NAMES.items()}
    g, _ = _groups()
    cfg = _cfg()
    o = _abi.GrpoOutputs()
    o.scalars = FAKE
    call = lambda **k: lib.grpo_token_loss(
        k.get("logp", FAKE), FAKE, k.get("ref", FAKE), k.get("gen"), None, FAKE, None, k.get("B", 8),
        k.get("T", 4),
        C.byref(k.get("g", g)), C.byref(k.get("cfg", cfg)), FAKE, None, C.byref(o),
        k.get("ws", FAKE_WS), k.get("wsb", 1 << 30), None)
    assert call(logp=None) == E["GRPO_ERR_NULL"]
    assert call(T=0) == E["GRPO_ERR_SHAPE"]
    assert call(B=6) == E["GRPO_ERR_GROUPS"]
    assert call(ref=None) == E["GRPO_ERR_CONFIG"]           # beta > 0 needs ref
    assert call(cfg=_cfg(tis_type=2, tis_ratio_min=0.5, tis_ratio_max=2.0)) == E["GRPO_ERR_CONFIG"]
    assert call(wsb=10) == E["GRPO_ERR_WORKSPACE"]
    assert lib.grpo_advantages(FAKE, 8, C.byref(_groups(spp=3)[0]), FAKE, FAKE_WS, 1 << 20,
                               None) == E["GRPO_ERR_GROUPS"]
    assert lib.grpo_advantages(None, 8, C.byref(g), FAKE, FAKE_WS, 1 << 20, None) == E["GRPO_ERR_NULL"]
    assert lib.grpo_loss_bwd(FAKE, 0, 32, FAKE, 0, None, 8, 4, 32, None, 0, 32, None, FAKE_WS,
                             1 << 30, None) == E["GRPO_ERR_NULL"]
    assert lib.grpo_loss_bwd(FAKE, 0, 32, FAKE, 0, None, 8, 4, 32, FAKE + 4, 0, 32, None, FAKE_WS,
                             1 << 30, None) == E["GRPO_ERR_ALIAS"]
    # token advantages
    tok = lambda est=0, r=FAKE, old=FAKE, ref=FAKE, g=None, kl=0.1, gamma=1.0, norm=1, out=FAKE, \
        wsb=1 << 30: lib.grpo_token_advantages(est, r, old, ref, None, 8, 4,
                                               None if g is None else C.byref(g), kl, gamma, norm,
                                               out, None, FAKE_WS, wsb, None)
    assert tok(r=None) == E["GRPO_ERR_NULL"]
    assert tok(out=None) == E["GRPO_ERR_NULL"]
    assert tok(est=2) == E["GRPO_ERR_CONFIG"]
    assert tok(kl=-1.0) == E["GRPO_ERR_CONFIG"]
    assert tok(gamma=0.0) == E["GRPO_ERR_CONFIG"]
    assert tok(gamma=1.5) == E["GRPO_ERR_CONFIG"]
    assert tok(norm=2) == E["GRPO_ERR_CONFIG"]
    assert tok(ref=None) == E["GRPO_ERR_NULL"]                     # KL shaping needs ref
    # the output pass launches a block per 256 slots at most: 2^31 such blocks are refused
    assert lib.grpo_token_advantages(0, FAKE, FAKE, FAKE, None, 1 << 20, 1 << 19, None, 0.1, 1.0,
                                     1, FAKE, None, FAKE_WS, 1 << 30, None) == E["GRPO_ERR_SHAPE"]
    assert tok(est=1) == E["GRPO_ERR_NULL"]                        # baseline needs groups
    gb, _ = _groups(scale=1)
    assert tok(est=1, g=gb) == E["GRPO_ERR_GROUPS"]                # inclusive mean, no std
    gb, _ = _groups(spp=3, scale=0)
    assert tok(est=1, g=gb) == E["GRPO_ERR_GROUPS"]
    assert tok(wsb=10) == E["GRPO_ERR_WORKSPACE"]
    # GDPO
    gd = lambda r=FAKE, c=2, g=g, out=FAKE: lib.grpo_gdpo_advantages(r, c, 8, C.byref(g), out,
                                                                     FAKE_WS, 1 << 20, None)
    assert gd(r=None) == E["GRPO_ERR_NULL"]
    assert gd(c=1) == E["GRPO_ERR_CONFIG"]
    assert gd(g=_groups(spp=3)[0]) == E["GRPO_ERR_GROUPS"]


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        _abi.load_library(str(tmp_path / "missing.so"))


@cpu_only
def test_scale_grad_argument_validation():
    lib = rpl.load_library()
    E = {v: k for k, v in _abi.STATUS_NAMES.items()}
    scale = C.c_void_p(FAKE)
    assert lib.grpo_scale_grad(None, 1, 4, 8, 8, scale, None) == E["GRPO_ERR_NULL"]
    assert lib.grpo_scale_grad(FAKE, 1, 4, 8, 8, None, None) == E["GRPO_ERR_NULL"]
    assert lib.grpo_scale_grad(FAKE, 5, 4, 8, 8, scale, None) == E["GRPO_ERR_DTYPE"]
    assert lib.grpo_scale_grad(FAKE, 1, 0, 8, 8, scale, None) == E["GRPO_ERR_SHAPE"]
    assert lib.grpo_scale_grad(FAKE, 1, 4, 0, 8, scale, None) == E["GRPO_ERR_SHAPE"]
    assert lib.grpo_scale_grad(FAKE, 1, 4, 8, 7, scale, None) == E["GRPO_ERR_SHAPE"]   # stride < V
    assert lib.grpo_scale_grad(FAKE, 1, 1 << 40, 1 << 30, 1 << 30, scale, None) == E["GRPO_ERR_SHAPE"]


def test_provenance_fingerprint(monkeypatch):
    """The fingerprint of a result's provenance follows the settings that fix
    the numbers (entry point, storage types, objective, groups) and nothing
    else: not the sizes, the optional-input flags or the device."""
    import torch
    from rl_post_loss_amd import loss as L
    monkeypatch.setattr(torch.cuda, "get_device_name", lambda d=None: "gpu")

    def fp(entry="grpo_loss_fwd_bwd", eps=0.2, red="token_mean", spp=8, bounds=None, B=16,
           logits="torch.bfloat16", inputs=None):
        cfg = L._make_cfg(eps, None, None, 0.04, red, None, **L.OBJECTIVE_DEFAULTS)
        g, _, _ = L._make_groups(B, spp, bounds, False, True, 1e-6)
        d = L._provenance(entry, dict(B=B, T=4, V=32), dict(logits=logits), cfg, g, bounds,
                          inputs or {}, "cuda:0")
        assert d["config"]["eps_low"] == eps and d["groups"]["group_boundaries"] == (
            None if bounds is None else list(bounds))
        return d["fingerprint"]

    base = fp()
    assert fp(B=32, inputs=dict(mask=True)) == base
    for other in (fp(entry="grpo_token_loss"), fp(eps=0.25), fp(red="sequence_mean"), fp(spp=4),
                  fp(logits="torch.float32"), fp(spp=None, bounds=[0, 8, 16])):
        assert other != base
    assert fp(spp=None, bounds=[0, 8, 16]) != fp(spp=None, bounds=[0, 4, 16])


def test_autograd_wrappers_reject_conflicting_arguments():
    """The autograd entry points take the gradient's scale from the backward
    pass and return scalars only, so the keywords that would contradict that
    are rejected before any work is done."""
    import torch
    import rl_post_loss_amd as rpl
    x = torch.zeros((2, 3))
    for kw in (dict(want_grad=False), dict(grad_scale=x), dict(out=None), dict(per_token=True)):
        with pytest.raises(ValueError):
            rpl.grpo_logp_loss(x, x, x, None, None, **kw)
    with pytest.raises(ValueError):
        rpl.grpo_loss(x, x, x, x, x, None, precompute_grad=True, grad_scale=x)
    with pytest.raises(ValueError):
        rpl.grpo_loss(x, x, x, x, x, None, precompute_grad=True, grad_out=x)


def _fwd_noalloc(lib, B=8, T=4, V=32, g=None, cfg=None, scalars=FAKE, grad=FAKE + 0x4000000,
                 ld=None):
    if g is None:
        g, _ = _groups()
    cfg = cfg or _cfg()
    o = _abi.GrpoOutputs()
    o.scalars = scalars
    return lib.grpo_loss_fwd_bwd_noalloc(FAKE, FAKE, 0, ld or V, FAKE, 0, FAKE, None, None, FAKE,
                                         None, B, T, V, C.byref(g), C.byref(cfg), grad, 0, V,
                                         None, C.byref(o), None)


@cpu_only
def test_noalloc_argument_validation():
    """The entry point without a workspace validates every argument as
    grpo_loss_fwd_bwd does and refuses sizes whose workspace exceeds the
    library's scratch array, all before touching a device."""
    lib = rpl.load_library()
    E = {v: k for k, v in _abi.STATUS_NAMES.items()}
    assert _fwd_noalloc(lib, scalars=None) == E["GRPO_ERR_NULL"]
    assert _fwd_noalloc(lib, B=0) == E["GRPO_ERR_SHAPE"]
    assert _fwd_noalloc(lib, ld=16) == E["GRPO_ERR_SHAPE"]
    assert _fwd_noalloc(lib, cfg=_cfg(lo=1.0)) == E["GRPO_ERR_CONFIG"]
    g, _ = _groups(spp=3)
    assert _fwd_noalloc(lib, g=g) == E["GRPO_ERR_GROUPS"]
    # the largest T whose workspace fits, and one past it
    B = 8
    fits = max(t for t in (1 << k for k in range(10, 24))
               if lib.grpo_workspace_bytes(B, t, 0) <= _abi.NOALLOC_SCRATCH_BYTES)
    assert lib.grpo_workspace_bytes(B, 2 * fits, 0) > _abi.NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(lib, B=B, T=2 * fits, V=1) == E["GRPO_ERR_WORKSPACE"]
    assert _fwd_noalloc(lib, B=1024, T=4096, V=1) == E["GRPO_ERR_WORKSPACE"]
    # the stated capacity: about 280,000 slots
    assert 200_000 <= B * fits * 2 and lib.grpo_workspace_bytes(1, 280_000, 0) <= 8 << 20
