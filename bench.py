"""Benchmark of the GRPO loss hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME|all] [--objective NAME]

One step is one pass of the whole path over one batch of synthetic inputs
already resident in HBM: advantages and weights, the fused vocabulary pass
with the analytic gradient, the fixed-order reductions
(grpo_loss_fwd_bwd); for the log-prob workloads one grpo_token_loss call.

The default (``--workload all``) prints ONE JSON line whose headline is the
Qwen-size vocabulary (B = 32 as 4 prompts x 8 samples, T = 2048,
V = 151,936, bf16 logits, full mask, token mean) and whose ``configs`` holds
one record per other workload: the tiny f32 batch, the 4,194,304-token loss
(full and ragged masks), the V = 32,000 batch and the CSR V = 128,256 batch
under the token mean, the sequence mean and length^0.5.  Every record has
tokens/s, a ``roofline`` block for its dominant kernel (algorithmic bytes
over that kernel's own HIP-event-timed duration, against 8 TB/s HBM, plus
HBM traffic from committed rocprofv3 counter summaries when they match the
current sources) and a ``cpu_baseline``: the fp64 oracle, as it stands, on
a bounded sample of the same batch over the host's cores (worker processes
started before the GPU is touched).

--workload NAME runs one workload alone (one line); --objective selects
another objective on a logits workload.  The sequence-level objectives
(gspo, real) run a forward row pass, the per-sequence phase and a gradient
pass; the timed kernel then spans all three.

Auxiliary modes (for the HBM-traffic counters, see profiles/):
  --calibrate-only       run only a plain elementwise kernel over 2 GiB that
                         reads and writes known bytes (counter scale)
  --summarize-pmc F W CF CW --kernel K
                         write profiles/<K>_<workload>_pmc.json from four
                         rocprofv3 --pmc csv runs: FETCH_SIZE and WRITE_SIZE of
                         the bench, then of the calibration run
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "tokens/s for fused GRPO fwd+bwd from [B,T,V] logits; % of MI355X peak HBM GB/s"
# The sources each kernel family is built from (its own files and the shared
# headers, the C ABI and its launch code): a profile summary records their
# hash, and its HBM traffic is reported only while that hash still matches.
_SHARED_SOURCES = ["include/grpo.h", "rl_post_loss_amd/csrc/grpo_device.hpp",
                   "rl_post_loss_amd/csrc/grpo_internal.hpp", "rl_post_loss_amd/csrc/grpo_api.hip"]
_LOGITS_SOURCES = ["rl_post_loss_amd/csrc/grpo_rows.hip", "rl_post_loss_amd/csrc/grpo_rows_resident.hip",
                   "rl_post_loss_amd/csrc/grpo_rowcore.hpp", "rl_post_loss_amd/csrc/grpo_objective.hpp",
                   "rl_post_loss_amd/csrc/grpo_seq.hip"]
_TOKEN_SOURCES = ["rl_post_loss_amd/csrc/grpo_reduce.hip", "rl_post_loss_amd/csrc/grpo_objective.hpp",
                  "rl_post_loss_amd/csrc/grpo_groupadv.hpp", "rl_post_loss_amd/csrc/grpo_prep.hip"]
_ESTIMATOR_SOURCES = ["rl_post_loss_amd/csrc/grpo_adv.hip", "rl_post_loss_amd/csrc/grpo_groupadv.hpp"]
FAMILY_SOURCES = {"grpo_rows_kernel": _LOGITS_SOURCES, "grpo_rows_resident_kernel": _LOGITS_SOURCES,
                  "grpo_seq_path": _LOGITS_SOURCES, "grpo_token_kernel": _TOKEN_SOURCES,
                  "grpo_tokadv_kernels": _ESTIMATOR_SOURCES}
KERNEL_SOURCES = sorted(set(_SHARED_SOURCES + _LOGITS_SOURCES + _TOKEN_SOURCES + _ESTIMATOR_SOURCES))
CALIB_BYTES = 1 << 31   # 2 GiB copy for counter calibration
MAX_WORKERS = 16        # host processes for the oracle (the machine's CPU share per GPU)

# objective presets: (keyword overrides, needs generating log-probs)
OBJECTIVES = {
    "default": ({}, False),
    "cispo": (dict(pg_loss="cispo"), False),
    "gspo": (dict(pg_loss="gspo", reduction="sequence_mean"), False),
    "real": (dict(pg_loss="real", reduction="token_mean"), False),
    "seq_mask": (dict(tis_type="seq_mask", tis_ratio_min=0.8, tis_ratio_max=1.25), True),
}


def kernel_source_hash(kernel=None):
    """Hash of the sources ``kernel``'s family is built from (every kernel
    source when ``kernel`` is None or not a known family)."""
    rels = _SHARED_SOURCES + FAMILY_SOURCES[kernel] if kernel in FAMILY_SOURCES else KERNEL_SOURCES
    h = hashlib.sha256()
    for rel in rels:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# Byte models (algorithmic bytes per launch of the dominant kernel)
# ---------------------------------------------------------------------------

def byte_model(wl, active, rows):
    """The stated model of the fused logits call: every active row reads the
    policy row twice and the reference row once and writes the gradient row
    once; a masked row only writes its zero gradient; plus the per-slot side
    inputs (int64 action id, float32 old log-prob, mask byte)."""
    bx = 4 if wl.dtype == "f32" else 2
    bg = bx
    V = wl.V
    return active * V * (3 * bx + bg) + (rows - active) * V * bg + rows * (8 + 4 + 1)


HELD_CHUNKS = 8 * 1024   # 16-byte policy chunks per row the fused streaming kernel keeps in LDS


def min_bytes(wl, active, rows, resident):
    """The bytes the chosen row kernel must move at least: the resident kernel
    reads each active policy row once (policy + reference + gradient); the
    streaming kernel reads it twice except the first HELD_CHUNKS 16-byte
    chunks of the row, which it keeps in LDS between its passes."""
    bx = 4 if wl.dtype == "f32" else 2
    V = wl.V
    if not resident:
        # only the 1024-thread kernel (rows above 64 KB) holds chunks
        held = min(V * bx // 16, HELD_CHUNKS) * 16 if V * bx > 65536 else 0
        return byte_model(wl, active, rows) - active * held
    return active * V * (2 * bx + bx) + (rows - active) * V * bx + rows * (8 + 4 + 1)


def token_bytes(active, rows):
    """Log-prob token loss: an active token reads logp, old and ref (f32) and
    the mask byte and writes dlogp (17 B); a masked one reads its mask byte
    and writes a zero (5 B)."""
    return active * 17 + (rows - active) * 5


# ---------------------------------------------------------------------------
# CPU baseline: the fp64 oracle as it stands, on a bounded sample of the same
# batch, spread over worker processes (started before the GPU is touched).
# ---------------------------------------------------------------------------

def host_workers():
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))


def under_profiler():
    """True when a profiler's library is preloaded into this process (it may
    have initialised the GPU before main, so no worker process is started)."""
    if any(k.startswith("ROCPROF") for k in os.environ):
        return True
    return "rocprof" in os.environ.get("LD_PRELOAD", "")


def start_pool(workers):
    """Worker processes for the oracle, spawned before this process touches
    the GPU (the children never do).  Returns once every worker has finished
    its imports: a worker still starting up competes with the timed steps
    for the host cores (measured: 1.90 ms per V = 32,000 step against 1.51)."""
    import multiprocessing
    ctx = multiprocessing.get_context("spawn")
    ready = ctx.Barrier(workers + 1)
    pool = ctx.Pool(workers, initializer=_worker_init, initargs=(ready,))
    ready.wait(timeout=600)
    return pool


def _worker_init(ready):
    import numpy  # noqa: F401
    import oracle  # noqa: F401
    ready.wait(timeout=600)


def _cfg_of(d):
    import oracle
    return oracle.LossConfig(**d)


def _rows_job(job):
    """Worker: the oracle's forward and gradient over one chunk of active rows
    (policy and reference rows read from the shared float32 sample files)."""
    import numpy as np
    import oracle
    xpath, ypath, shape, s, e, ids, old, adv, w, cfg = job
    x = np.load(xpath, mmap_mode="r")[s:e]
    y = np.load(ypath, mmap_mode="r")[s:e]
    oracle.logits_rows(x, y, ids, old, adv, w, _cfg_of(cfg))
    return e - s


def _token_job(job):
    """Worker: the oracle's log-prob token loss over whole groups."""
    import oracle
    h, spp, cfg = job
    oracle.grpo_token_loss(h["logp"], h["old_logps"], h["ref_logp"], h["mask"], h["rewards"],
                           groups=dict(samples_per_prompt=spp), cfg=_cfg_of(cfg))
    return h["mask"].size


def _cfg_dict(wl, reduction, obj):
    d = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=reduction,
             alpha=wl.alpha if reduction == "length_alpha" else None)
    d.update(obj)
    return d


def _timed_passes(pool, jobs, target_s):
    """Runs the jobs over the pool, again and again, until target_s of wall
    time have passed; returns (units done, seconds)."""
    done = 0
    t0 = time.perf_counter()
    while True:
        done += sum(pool.map(_run_job, jobs, chunksize=1))
        el = time.perf_counter() - t0
        if el >= target_s:
            return done, el


def _adv_job(job):
    """Worker: the oracle's token-level advantage estimator over whole groups
    (normalised over the job's sequences: the same work per slot as the
    batch-wide normalization)."""
    import oracle
    h, est, kw = job
    oracle.token_advantages(est, h["rewards"], h.get("old_logps"), h.get("ref_logp"), h["mask"],
                            **kw)
    return h["mask"].size


def _run_job(job):
    kind, payload = job
    if kind == "rows":
        return _rows_job(payload)
    return _adv_job(payload) if kind == "adv" else _token_job(payload)


def cpu_baseline_logits(pool, workers, wl, inp, reduction, obj, target_s, sample_rows):
    """The oracle over the first ``sample_rows`` slots of this batch (its active
    rows: masked rows are never read), chunks of 16 rows spread over the
    worker processes, repeated until target_s of wall time.  Rows reach the
    workers through float32 files written before timing starts."""
    import numpy as np
    import torch

    import oracle
    B, T, V = wl.B, wl.T, wl.V
    h_mask = inp["mask"].cpu().numpy().astype(bool)
    h_rew = inp["rewards"].cpu().numpy()
    groups = wl.groups_kwargs()
    off = oracle.group_offsets(B, groups.get("samples_per_prompt"), groups.get("group_boundaries"))
    A = oracle.group_advantages(h_rew, off, groups.get("leave_one_out", False),
                                groups.get("scale_by_std", True))
    cfg = _cfg_dict(wl, reduction, obj)
    _, _, w = oracle.sequence_weights(h_mask, reduction, cfg["alpha"])
    n = min(B * T, sample_rows)
    sel = np.nonzero(h_mask.reshape(-1)[:n])[0]
    ids = inp["action_ids"].reshape(-1).cpu().numpy()[sel]
    old = inp["old_logps"].reshape(-1).cpu().numpy()[sel]
    seq = sel // T
    tmp = _sample_dir()
    try:
        xpath = os.path.join(tmp, "x.npy")
        ypath = os.path.join(tmp, "y.npy")
        idx = torch.from_numpy(sel.astype(np.int64)).to(inp["policy"].device)
        for path, t in ((xpath, inp["policy"]), (ypath, inp["ref"])):
            rows = t.reshape(B * T, V).index_select(0, idx).float().cpu().numpy()
            np.save(path, rows)
            del rows
        jobs = []
        for s in range(0, len(sel), 16):
            e = min(len(sel), s + 16)
            jobs.append(("rows", (xpath, ypath, (len(sel), V), s, e, ids[s:e], old[s:e], A[seq[s:e]],
                                  w[seq[s:e]], cfg)))
        rows_done, el = _timed_passes(pool, jobs, target_s)
    finally:
        _rmtree(tmp)
    passes = rows_done / max(len(sel), 1)
    slots = passes * n
    return dict(value=slots / el, unit="tokens/s", cores=workers, kind="oracle",
                sample=f"slots 0..{n - 1} of {B * T} ({len(sel)} active rows; masked rows are never "
                       f"read) of the same batch, {passes:.2f} passes, float64 numpy on {workers} worker "
                       f"processes, {el:.1f} s wall; GPU-to-host copies excluded")


def cpu_baseline_tokens(pool, workers, wl, inp, target_s, groups_per_job=1):
    """The oracle's log-prob token loss over whole groups of this batch, one
    job per group spread over the worker processes, repeated until target_s
    of wall time."""
    h = {k: v.cpu().numpy() for k, v in inp.items()}
    B, T = h["mask"].shape
    size = wl.group_size * groups_per_job
    cfg = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=wl.reduction)
    jobs = [("tok", ({k: v[s:s + size] for k, v in h.items()}, wl.group_size, cfg))
            for s in range(0, B, size)]
    slots, el = _timed_passes(pool, jobs, target_s)
    return dict(value=slots / el, unit="tokens/s", cores=workers, kind="oracle",
                sample=f"the whole batch in jobs of {size} sequences ({groups_per_job} group(s) each), "
                       f"{slots / (B * T):.2f} passes, float64 numpy on {workers} worker processes, "
                       f"{el:.1f} s wall")


def _sample_dir():
    """A scratch directory for the oracle's sample: /dev/shm when it has room,
    else the temporary directory."""
    import shutil
    for base in ("/dev/shm", tempfile.gettempdir()):
        try:
            if shutil.disk_usage(base).free > (24 << 30):
                return tempfile.mkdtemp(prefix="grpo_oracle_", dir=base)
        except OSError:
            pass
    return tempfile.mkdtemp(prefix="grpo_oracle_")


def _rmtree(path):
    import shutil
    shutil.rmtree(path, ignore_errors=True)


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """hipEvent_t pairs created through the HIP runtime (the kernel is launched
    by the library on torch's current stream; the library records these
    events right around that launch).  The events skip the system-scope fence
    (hipEventDisableSystemFence): they only time, and the fence's cache
    write-back and invalidate would add about 3 us to a 17 us kernel."""

    def __init__(self, n):
        import ctypes as C
        self.C = C
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = C.c_void_p(), C.c_void_p()
            f = HIP_EVENT_DISABLE_SYSTEM_FENCE
            assert (self.hip.hipEventCreateWithFlags(C.byref(a), f) == 0
                    and self.hip.hipEventCreateWithFlags(C.byref(b), f) == 0)
            self.pairs.append((a, b))

    def elapsed_ms(self, k):
        ms = self.C.c_float()
        a, b = self.pairs[k]
        rc = self.hip.hipEventElapsedTime(self.C.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


def timed_kernel(lib, steps, step):
    """Runs ``step(k)`` ``steps`` times with the library's timing hook set
    around the dominant kernel of each call; returns (host ms per step, list
    of kernel ms)."""
    import torch
    ev = HipEvents(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        lib.grpo_set_timing_events(ev.pairs[k][0], ev.pairs[k][1])
        step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.grpo_set_timing_events(None, None)
    kern = [ev.elapsed_ms(k) for k in range(steps)]
    ev.close()
    return (t1 - t0) * 1e3 / steps, kern


def _median(v):
    s = sorted(v)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def load_traffic(kernel, workload):
    """HBM traffic per launch (bytes) from the committed counter summary of
    ``kernel`` on ``workload``, if it was taken on the current sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return d.get("traffic_bytes_per_launch")


def roofline(kernel, workload, alg_bytes, kern_ms, extra=None):
    kavg = sum(kern_ms) / len(kern_ms)
    achieved = alg_bytes / (kavg * 1e-3) / 1e9
    traffic = load_traffic(kernel, workload)
    r = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
         "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, "kernel": kernel,
         "kernel_ms": kavg, "kernel_ms_median": _median(kern_ms), "algorithmic_bytes": alg_bytes,
         "physical_frac": None if traffic is None else traffic / (kavg * 1e-3) / 1e9 / PEAK_HBM_GBS}
    if extra:
        r.update(extra)
    return r


GRAPH_TIMING = ("GPU time per call: the calls captured in one HIP graph per replay (each input "
                "copy in turn), replays timed back to back; median of five measurements of four "
                "replays of 30 calls")


def _graph_times(step, ncopies, steps, per_graph=30):
    """(ms per call with `per_graph` calls captured in one HIP graph, ms per call
    with one graph per call).  The first is the GPU time of the path; the
    second adds one graph launch per call, which for calls of a few tens of
    microseconds the host's launch rate bounds rather than the GPU."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for j in range(ncopies):
            step(j)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    single = []
    for j in range(ncopies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step(j)
        single.append(g)
    multi = torch.cuda.CUDAGraph()
    with torch.cuda.graph(multi, stream=side):
        for k in range(per_graph):
            step(k % ncopies)
    torch.cuda.synchronize()
    reps = max(1, (steps + per_graph - 1) // per_graph)
    multi.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        multi.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / (reps * per_graph)
    for g in single:
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        single[k % ncopies].replay()
    torch.cuda.synchronize()
    ms_single = (time.perf_counter() - t0) * 1e3 / steps
    return ms, ms_single


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# Workload runners: each returns one record
# ---------------------------------------------------------------------------

def _row_kernel_name(wl, resident):
    return "grpo_rows_resident_kernel" if resident else "grpo_rows_kernel"


def _resident(wl):
    """Whether the fused call takes the resident-row kernel: rows above 4 KB
    and up to 128 KB, 16-byte aligned (the library's own choice, restated
    for labelling the record; the kernel trace names the kernel that ran)."""
    b = wl.V * (4 if wl.dtype == "f32" else 2)
    return 4096 < b <= 131072 and b % 16 == 0


def run_logits_record(args, wl, inp, reduction, objective="default", pool=None, workers=1,
                      cpu_seconds=None, sample_rows=None):
    import torch
    import rl_post_loss_amd as rpl
    from workloads import make_gen_logps

    lib = rpl.load_library()
    B, T, V = wl.B, wl.T, wl.V
    grad = torch.empty((B, T, V), dtype=inp["policy"].dtype, device=inp["policy"].device)
    kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=reduction,
              alpha=wl.alpha if reduction == "length_alpha" else None)
    kw.update(wl.groups_kwargs())
    obj, needs_gen = OBJECTIVES[objective]
    kw.update(obj)
    gen = make_gen_logps(inp["old_logps"], seed=args.seed) if needs_gen else None
    out = [None]

    def step(k=0):
        out[0] = rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"],
                                       inp["old_logps"], inp["rewards"], inp["mask"],
                                       grad_out=grad, gen_logps=gen, out=out[0], **kw)
        return out[0]

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    ref_scalars = out[0].scalars.clone()
    gview = grad.view(torch.int16 if grad.element_size() == 2 else torch.int32)
    ref_grad_sum = int(gview.sum(dtype=torch.int64))
    step_scalars = []

    def timed_step(k):
        step()
        step_scalars.append(out[0].scalars.clone())

    ms_per_step, kern = timed_kernel(lib, args.steps, timed_step)
    repro = (all(torch.equal(ref_scalars.view(torch.int32), sc.view(torch.int32)) for sc in step_scalars)
             and int(gview.sum(dtype=torch.int64)) == ref_grad_sum)
    active = int(inp["mask"].sum())
    rows = B * T
    resident = _resident(wl) and objective in ("default", "cispo", "seq_mask")
    kname = _row_kernel_name(wl, resident)
    key = wl.name if reduction == wl.reductions[0] else f"{wl.name}_{reduction}"
    alg = byte_model(wl, active, rows)
    mb = min_bytes(wl, active, rows, resident)
    kavg = sum(kern) / len(kern)
    rec = {
        "workload": f"{wl.name}: B={B} ({len(wl.group_sizes)} groups{', CSR' if wl.csr else ''}), "
                    f"T={T}, V={V}, {wl.dtype} logits and gradient, {reduction}, "
                    + ("full mask" if wl.len_range is None else "ragged lengths %d..%d" % wl.len_range)
                    + ("" if objective == "default" else f", objective {objective}"),
        "ms_per_step": ms_per_step,
        "tokens_per_s": rows / (ms_per_step * 1e-3),
        "active_tokens_per_s": active / (ms_per_step * 1e-3),
        "B": B, "T": T, "V": V, "storage": wl.dtype, "active_slots": active,
        "hbm_fraction_of_step": alg / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "bit_reproducible": bool(repro),
        "roofline": roofline(kname, key, alg, kern, {
            "byte_model": "policy row read twice, reference once, gradient written once per active "
                          "row; zero gradient per masked row; 13 B of side inputs per slot; "
                          "kernel_min_bytes: what the chosen kernel must move (the resident kernel "
                          "reads the policy row once, the streaming kernel keeps its first "
                          f"{HELD_CHUNKS} 16-byte chunks in LDS between its passes)",
            "kernel_min_bytes": mb,
            "kernel_min_frac": mb / (kavg * 1e-3) / 1e9 / PEAK_HBM_GBS}),
    }
    if objective != "default":
        rec["objective"] = obj
    if pool is not None and objective == "default":
        _log(f"oracle baseline {key}")
        rec["cpu_baseline"] = cpu_baseline_logits(pool, workers, wl, inp, reduction, obj,
                                                  cpu_seconds or args.cpu_seconds,
                                                  sample_rows or 4096)
    else:
        rec["cpu_baseline"] = None
    return rec


def run_autograd_record(args, wl, inp, precompute, upstream=1.0):
    """The autograd entry ("GRPO Loss", Entry Point: loss.backward() puts
    d loss / d logits into the policy's .grad): one step is grpo_loss(...)
    then loss.backward() on a leaf policy tensor whose .grad is cleared
    first, so autograd hands over the gradient without accumulating.
    precompute=False (default): forward-only kernel, then a gradient pass
    that streams the policy again; precompute=True: the fused kernel in the
    forward (its [B, T, V] gradient held until the backward), then an
    in-place scale by the upstream gradient (a no-op for 1)."""
    import torch
    import rl_post_loss_amd as rpl

    B, T, V = wl.B, wl.T, wl.V
    red = wl.reductions[0]
    kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=red,
              alpha=wl.alpha if red == "length_alpha" else None)
    kw.update(wl.groups_kwargs())
    pol = inp["policy"].detach().requires_grad_(True)

    def step():
        pol.grad = None
        loss, _, _ = rpl.grpo_loss(pol, inp["ref"], inp["action_ids"], inp["old_logps"],
                                   inp["rewards"], inp["mask"], precompute_grad=precompute, **kw)
        (loss if upstream == 1.0 else loss * upstream).backward()
        return loss

    for _ in range(max(1, args.warmup)):
        ref_loss = step().detach().clone()
    torch.cuda.synchronize()
    gview = pol.grad.view(torch.int16 if pol.grad.element_size() == 2 else torch.int32)
    ref_sum = int(gview.sum(dtype=torch.int64))
    losses = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        losses.append(step().detach())
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    gview = pol.grad.view(torch.int16 if pol.grad.element_size() == 2 else torch.int32)
    repro = (all(torch.equal(l.view(torch.int32), ref_loss.view(torch.int32)) for l in losses)
             and int(gview.sum(dtype=torch.int64)) == ref_sum)
    rows = B * T
    active = int(inp["mask"].sum())
    alg = byte_model(wl, active, rows)
    rec = {
        "workload": f"{wl.name} through grpo_loss(...).backward() "
                    + ("with precompute_grad=True (fused kernel in the forward, gradient held "
                       "until the backward)" if precompute else
                       "(forward-only pass, then a gradient pass that re-reads the policy)")
                    + ("" if upstream == 1.0 else f", upstream gradient {upstream}"),
        "ms_per_step": ms, "tokens_per_s": rows / (ms * 1e-3),
        "hbm_fraction_of_step": alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "algorithmic_bytes": alg, "bit_reproducible": bool(repro),
        "extra_memory_bytes_held": rows * V * pol.element_size() if precompute else 16 * rows,
        "timing": "host wall clock over the timed steps, synchronized at both ends",
    }
    pol.grad = None
    return rec


def run_token_record(args, wl, pool=None, workers=1, copies=None):
    """Logprob-level token loss (no vocabulary).  The 71 MB working set fits
    the memory-side cache, so the timed calls rotate over enough input copies
    (each call reads a different one) to keep it from being served there."""
    import torch
    import rl_post_loss_amd as rpl
    from workloads import make_token_inputs

    lib = rpl.load_library()
    dev = torch.device("cuda:0")
    ncop = copies or args.copies
    cps = [make_token_inputs(wl, device=dev, seed=args.seed + k) for k in range(ncop)]
    kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
              samples_per_prompt=wl.group_size, reduction=wl.reduction)
    results = [None] * ncop

    def step(k):
        j = k % ncop
        c = cps[j]
        results[j] = rpl.grpo_token_loss(c["logp"], c["old_logps"], c["ref_logp"], c["rewards"],
                                         c["mask"], out=results[j], **kw)

    for k in range(max(args.warmup, ncop)):
        step(k)
    torch.cuda.synchronize()
    ref_scalars = [r.scalars.clone() for r in results]
    ref_grads = [r.grad.clone() for r in results]
    ms_eager, kern = timed_kernel(lib, max(args.steps, 30), step)
    # calls this short vary from replay to replay: the median of five
    # measurements, each over four replays of a 30-call graph
    meas = [_graph_times(step, ncop, 120) for _ in range(5)]
    ms = _median([m[0] for m in meas])
    ms_graph_per_call = _median([m[1] for m in meas])
    torch.cuda.synchronize()
    repro = all(torch.equal(a.view(torch.int32), r.scalars.view(torch.int32)) and
                torch.equal(g.view(torch.int32), r.grad.view(torch.int32))
                for a, g, r in zip(ref_scalars, ref_grads, results))
    active = int(cps[0]["mask"].sum())
    rows = wl.B * wl.T
    alg = token_bytes(active, rows)
    rec = {
        "workload": f"{wl.name}: B={wl.B} ({wl.num_groups} groups of {wl.group_size}), T={wl.T}, "
                    f"f32 log-probs, {wl.reduction}, "
                    + ("full mask" if wl.len_range is None else "ragged lengths %d..%d" % wl.len_range)
                    + f"; input copies rotated: {ncop}",
        "ms_per_step": ms, "timing": GRAPH_TIMING,
        "tokens_per_s": rows / (ms * 1e-3), "active_tokens_per_s": active / (ms * 1e-3),
        "active_slots": active, "algorithmic_bytes": alg,
        "hbm_fraction_of_step": alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "ms_per_step_graph_per_call": ms_graph_per_call, "ms_per_step_eager_python": ms_eager,
        "bit_reproducible": bool(repro),
        "roofline": roofline("grpo_token_kernel", wl.name, alg, kern, {
            "byte_model": "17 B per active token (logp, old, ref f32 + mask in, dlogp out), 5 B per "
                          "masked token (mask in, zero out)",
            "timing": "the token kernel alone, HIP events around its launch in eager calls"}),
    }
    if pool is not None:
        _log(f"oracle baseline {wl.name}")
        rec["cpu_baseline"] = cpu_baseline_tokens(pool, workers, wl, cps[0], args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    del cps, results
    return rec


ADV_WORKLOADS = {"adv_reinforce_pp": "reinforce_pp", "adv_reinforce_pp_baseline": "reinforce_pp_baseline"}


def _adv_kwargs(est, wl):
    if est == "reinforce_pp":
        return dict(kl_coef=0.01, gamma=1.0, normalize=True)
    return dict(samples_per_prompt=wl.group_size, normalize=True)


def cpu_baseline_adv(pool, workers, wl, est, inp, target_s):
    """The oracle's estimator over the whole batch in jobs of one group each,
    repeated until target_s of wall time."""
    keys = ("rewards", "mask") + (("old_logps", "ref_logp") if est == "reinforce_pp" else ())
    h = {k: inp[k].cpu().numpy() for k in keys}
    B, T = h["mask"].shape
    size = wl.group_size
    kw = dict(_adv_kwargs(est, wl))
    spp = kw.pop("samples_per_prompt", None)
    if spp is not None:
        kw["groups"] = dict(samples_per_prompt=spp)
    jobs = [("adv", ({k: v[s:s + size] for k, v in h.items()}, est, kw)) for s in range(0, B, size)]
    slots, el = _timed_passes(pool, jobs, target_s)
    return dict(value=slots / el, unit="tokens/s", cores=workers, kind="oracle",
                sample=f"the whole batch in jobs of one group ({size} sequences) each, normalised over "
                       f"the job's sequences, {slots / (B * T):.2f} passes, float64 numpy on {workers} "
                       f"worker processes, {el:.1f} s wall")


def run_adv_record(args, name, pool=None, workers=1):
    """Token-level advantage estimator over the log-prob workload's shape
    (B = 1024 in groups of 16, T = 4096, ragged lengths): REINFORCE++
    returns (k1 shaping 0.01, gamma 1) or the inclusive group baseline, with
    the global masked normalization.  Input copies are rotated as for the
    token loss."""
    import torch
    import rl_post_loss_amd as rpl
    from workloads import TOKEN_WORKLOADS, make_token_inputs

    lib = rpl.load_library()
    dev = torch.device("cuda:0")
    est = ADV_WORKLOADS[name]
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    copies = [make_token_inputs(wl, device=dev, seed=args.seed + k) for k in range(args.copies)]
    kw = _adv_kwargs(est, wl)
    outs = [None] * len(copies)

    def step(k):
        j = k % len(copies)
        c = copies[j]
        extra = dict(old_logps=c["old_logps"], ref_logps=c["ref_logp"]) if est == "reinforce_pp" else {}
        outs[j] = rpl.grpo_token_advantages(est, c["rewards"], c["mask"], **extra, **kw)

    for k in range(max(args.warmup, len(copies))):
        step(k)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    _, kern = timed_kernel(lib, max(args.steps, 30), step)
    meas = [_graph_times(step, len(copies), 120) for _ in range(5)]
    ms = _median([m[0] for m in meas])
    ms_graph_per_call = _median([m[1] for m in meas])
    torch.cuda.synchronize()
    repro = all(torch.equal(a.view(torch.int32), o.view(torch.int32)) for a, o in zip(ref, outs))
    rows = wl.B * wl.T
    # minimum bytes: old, ref f32 and the mask read once (REINFORCE++), the output written once
    per_slot = (4 + 4 + 1 + 4) if est == "reinforce_pp" else (1 + 4)
    alg = rows * per_slot
    rec = {"workload": f"{name}: B={wl.B} (groups of {wl.group_size}), T={wl.T}, ragged lengths, "
                       f"{est}, normalized; input copies rotated: {args.copies}",
           "ms_per_step": ms, "timing": GRAPH_TIMING, "tokens_per_s": rows / (ms * 1e-3),
           "algorithmic_bytes": alg, "hbm_fraction_of_step": alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "ms_per_step_graph_per_call": ms_graph_per_call, "bit_reproducible": bool(repro),
           "roofline": roofline("grpo_tokadv_kernels", name, alg, kern, {
               "byte_model": f"{per_slot} B per slot: "
                             + ("old, ref f32 and the mask read, the advantage written"
                                if est == "reinforce_pp" else "the mask read, the advantage written"),
               "timing": "the estimator's kernels together, HIP events around them in eager calls"})}
    if pool is not None:
        _log(f"oracle baseline {name}")
        rec["cpu_baseline"] = cpu_baseline_adv(pool, workers, wl, est, copies[0], args.cpu_seconds)
    else:
        rec["cpu_baseline"] = None
    del copies, outs
    return rec


def run_pages_shapes(args):
    """The fused logits call at the shapes of the grpo.cpp README's CUDA table
    (1,024 token slots as B = 8 x T = 128 in groups of 4, f32 logits and
    gradient, V = 32,768 and 131,072), full and ragged masks, with and
    without reference logits.  Each call timed with events around it on the
    current stream (its launches and the gaps between them included); the
    median of ``steps`` calls."""
    import torch
    import rl_post_loss_amd as rpl
    from workloads import LogitsWorkload, make_logits_inputs

    rpl.load_library()
    dev = torch.device("cuda:0")
    recs = {}
    for V in (32768, 131072):
        for ragged in (False, True):
            wl = LogitsWorkload(name=f"pages_v{V}", group_sizes=(4, 4), T=128, V=V, dtype="f32",
                                logit_std=1.0, ref_noise_std=0.1 ** 0.5, old_noise_std=0.05 ** 0.5,
                                reward_p=0.5, len_range=(1, 128) if ragged else None)
            inp = make_logits_inputs(wl, device=dev, seed=args.seed)
            grad = torch.empty_like(inp["policy"])
            active = int(inp["mask"].sum())
            for with_ref in (False, True):
                kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, reduction="token_mean",
                          beta=wl.beta if with_ref else 0.0, **wl.groups_kwargs())
                ref = inp["ref"] if with_ref else None
                out = [None]

                def call():
                    out[0] = rpl.grpo_loss_fwd_bwd(inp["policy"], ref, inp["action_ids"],
                                                   inp["old_logps"], inp["rewards"], inp["mask"],
                                                   grad_out=grad, out=out[0], **kw)

                for _ in range(max(3, args.warmup)):
                    call()
                torch.cuda.synchronize()
                ms = []
                for _ in range(max(20, args.steps)):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    call()
                    b.record()
                    b.synchronize()
                    ms.append(a.elapsed_time(b))
                key = f"v{V}_{'ragged' if ragged else 'full'}_{'ref' if with_ref else 'noref'}"
                recs[key] = {"ms_per_call": _median(ms), "active_slots": active,
                             "V": V, "B": wl.B, "T": wl.T, "reference_logits": with_ref}
            del inp, grad
            torch.cuda.empty_cache()
    print(json.dumps({"metric": "ms per fused logits call at the grpo.cpp README table shapes "
                                "(1,024 token slots, f32)", "unit": "ms", "higher_is_better": False,
                      "timing": "events around each call on the current stream, median of the calls",
                      "data": "synthetic", "configs": recs}), flush=True)


def _line(rec, args, wl_key):
    """The bench line around one record."""
    return {
        "metric": ("tokens/s for the logprob-level GRPO token loss (forward + dlogp)"
                   if wl_key.startswith("token_loss") else
                   "tokens/s for the token-level advantage estimator (returns + global normalization)"
                   if wl_key in ADV_WORKLOADS else METRIC),
        "value": rec["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "f64" if wl_key in ADV_WORKLOADS else "f32", "data": "synthetic",
        "config": {k: v for k, v in rec.items() if k not in ("roofline", "cpu_baseline", "ms_per_step",
                                                              "tokens_per_s")},
        "roofline": rec["roofline"], "cpu_baseline": rec["cpu_baseline"],
    }


def run_single(args, pool, workers):
    import torch
    import rl_post_loss_amd as rpl
    from workloads import TOKEN_WORKLOADS, WORKLOADS, make_logits_inputs

    rpl.load_library()
    if args.workload in ADV_WORKLOADS:
        rec = run_adv_record(args, args.workload, pool, workers)
        print(json.dumps(_line(rec, args, args.workload)), flush=True)
        return
    if args.workload in TOKEN_WORKLOADS:
        rec = run_token_record(args, TOKEN_WORKLOADS[args.workload], pool, workers)
        print(json.dumps(_line(rec, args, args.workload)), flush=True)
        return
    name, _, red = args.workload.partition(":")
    wl = WORKLOADS[name]
    red = red or (OBJECTIVES[args.objective][0].get("reduction") or wl.reductions[0])
    _log(f"generating {wl.name}: B={wl.B} T={wl.T} V={wl.V} {wl.dtype}")
    inp = make_logits_inputs(wl, device=torch.device("cuda:0"), seed=args.seed)
    torch.cuda.synchronize()
    rec = run_logits_record(args, wl, inp, red, args.objective, pool, workers)
    print(json.dumps(_line(rec, args, name)), flush=True)


def memory_ceiling(gib=8):
    """The box's own streaming rates, for reading the fractions of 8 TB/s in
    context: torch's row sums over a bf16 tensor (read), its zero fill
    (write) and its copy (half read, half write), GIB GiB each way, median of
    5 after a warm-up, HIP events on the current stream."""
    import torch
    n = (gib << 30) // 2
    x = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    y = torch.empty_like(x)
    out = {}
    xr = x.view(-1, 4096)
    for name, fn, nbytes in (("read", lambda: xr.sum(dim=1, dtype=torch.float32), n * 2),
                             ("write", lambda: y.zero_(), n * 2),
                             ("copy", lambda: y.copy_(x), n * 4)):
        fn()
        ms = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ms.append(a.elapsed_time(b))
        t = _median(ms)
        out[f"{name}_GBps"] = nbytes / (t * 1e-3) / 1e9
        out[f"{name}_frac_of_peak"] = out[f"{name}_GBps"] / PEAK_HBM_GBS
    out["method"] = (f"torch row sums of 4,096 values (read), zero_ (write) and copy_ (read + "
                     f"write) over {gib} GiB of bf16, median of 5 timed with events; context for "
                     "the fractions of 8 TB/s, not a limit the kernels are held to")
    del x, y
    torch.cuda.empty_cache()
    return out


# sample of slots the CPU baseline takes from each logits workload (about
# 2-3 s of oracle work over 16 processes)
SAMPLE_ROWS = {"tiny_logits": 128, "logits_v32000": 16384, "logits_v151936": 2048,
               "logits_csr_v128256": 6144}


def run_all(args, pool, workers):
    """The headline (V = 151,936) and one record per other workload, in one line."""
    import torch
    import rl_post_loss_amd as rpl
    from workloads import TOKEN_WORKLOADS, WORKLOADS, make_logits_inputs

    rpl.load_library()
    dev = torch.device("cuda:0")
    subs = {}
    head = None
    for name in ("logits_v151936", "tiny_logits", "logits_v32000", "logits_csr_v128256"):
        wl = WORKLOADS[name]
        _log(f"generating {wl.name}: B={wl.B} T={wl.T} V={wl.V} {wl.dtype}")
        t0 = time.perf_counter()
        inp = make_logits_inputs(wl, device=dev, seed=args.seed)
        torch.cuda.synchronize()
        _log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
        for red in wl.reductions:
            key = name if red == wl.reductions[0] else f"{name}:{red}"
            _log(f"timing {key}")
            rec = run_logits_record(args, wl, inp, red, pool=pool, workers=workers,
                                    sample_rows=SAMPLE_ROWS[name])
            if name == "logits_v151936":
                head = rec
                for pre, up in ((False, 1.0), (True, 1.0), (False, 0.5), (True, 0.5)):
                    akey = ("autograd_precompute" if pre else "autograd_split") + \
                        ("" if up == 1.0 else "_upstream_0.5")
                    _log(f"timing {name} {akey}")
                    subs[f"{name}:{akey}"] = run_autograd_record(args, wl, inp, pre, up)
                    torch.cuda.empty_cache()
            else:
                subs[key] = rec
        del inp
        torch.cuda.empty_cache()
    for name in ("token_loss_full", "token_loss_ragged"):
        _log(f"timing {name}")
        subs[name] = run_token_record(args, TOKEN_WORKLOADS[name], pool, workers)
        torch.cuda.empty_cache()
    for name in ADV_WORKLOADS:
        _log(f"timing {name}")
        subs[name] = run_adv_record(args, name, pool, workers)
        torch.cuda.empty_cache()
    line = _line(head, args, "logits_v151936")
    line["configs"] = subs
    _log("timing the box's own streaming rates")
    line["memory_ceiling"] = memory_ceiling()
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Counter calibration and summaries
# ---------------------------------------------------------------------------

def calibrate_only():
    """One elementwise kernel over CALIB_BYTES of float32: reads CALIB_BYTES,
    writes CALIB_BYTES (torch.add with a scalar, out= a second buffer)."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_bytes_read": CALIB_BYTES, "calibration_bytes_written": CALIB_BYTES,
                      "check": float(dst[0])}))


# the dominant "kernel" of a record that launches several kernels per call
KERNEL_FAMILIES = {"grpo_tokadv_kernels": ("grpo_tokadv_kernel(", "grpo_tokadv_returns_kernel",
                                           "grpo_tokadv_norm_kernel")}


def _family(kernel):
    return KERNEL_FAMILIES.get(kernel, (kernel,))


def _csv_rows(d, suffix):
    import csv
    for path in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(path) as f:
            yield from csv.DictReader(f)


def _pmc_by_kernel(d, counter):
    """{kernel name: [per-dispatch counter value in dispatch order]} (a
    dispatch's csv rows summed)."""
    per = {}
    for row in _csv_rows(d, "counter_collection.csv"):
        if row.get("Counter_Name") != counter:
            continue
        key = (row.get("Kernel_Name", ""), int(row.get("Dispatch_Id")))
        per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in sorted(per.items(), key=lambda kv: kv[0][1]):
        out.setdefault(name, []).append(v)
    return out


def _matching(by_name, part):
    vals = []
    for name, v in by_name.items():
        if part in name:
            vals.extend(v)
    return vals


def _short(name):
    return name.split("(")[0].replace("void ", "").replace("grpo::", "")


def pmc_commands(workload, regex, dirs):
    wl_arg = workload.replace("_sequence_mean", ":sequence_mean").replace("_length_alpha", ":length_alpha")
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = dirs
    run = f"-- python3 bench.py --workload {wl_arg} --steps 3 --warmup 1 --no-cpu-baseline"
    return [f"rocprofv3 --pmc FETCH_SIZE --kernel-include-regex {regex} -f csv -d {fetch_dir} -o run {run}",
            f"rocprofv3 --pmc WRITE_SIZE --kernel-include-regex {regex} -f csv -d {write_dir} -o run {run}",
            "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex elementwise -f csv "
            f"-d {cal_fetch_dir} -o run -- python3 bench.py --calibrate-only",
            "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex elementwise -f csv "
            f"-d {cal_write_dir} -o run -- python3 bench.py --calibrate-only"]


def summarize_pmc(dirs, workload, kernel, out_dir, skip_first=1, regex=None):
    """Combine the four rocprofv3 --pmc runs into
    profiles/<kernel>_<workload>_pmc.json and .md.  The counters read over
    the calibration kernel, which moves a known number of bytes each way,
    give the scale from counter units to bytes.  The first ``skip_first``
    dispatches of each kernel (warm-up) are left out of its average.  A
    kernel family's traffic per call is the sum of its kernels' averages."""
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = dirs
    regex = regex or kernel
    res, per_kernel = {}, {}
    for counter, run_dir, cal_dir in (("FETCH_SIZE", fetch_dir, cal_fetch_dir),
                                      ("WRITE_SIZE", write_dir, cal_write_dir)):
        cal = _matching(_pmc_by_kernel(cal_dir, counter), "_add<float>")
        by_name = _pmc_by_kernel(run_dir, counter)
        if not cal or not by_name:
            raise SystemExit(f"missing {counter} values (calibration {len(cal)}, kernels {len(by_name)})")
        c = max(cal)
        scale = CALIB_BYTES / c
        total, present = 0.0, []
        for part in _family(kernel):
            rows = _matching(by_name, part)
            if not rows:
                continue   # a family member this estimator does not launch
            present.append(part)
            used = rows[skip_first:] if len(rows) > skip_first else rows
            total += sum(used) / len(used) * scale
        if not present:
            raise SystemExit(f"no {counter} dispatches of {kernel}")
        for name, rows in by_name.items():
            used = rows[skip_first:] if len(rows) > skip_first else rows
            d = dict(dispatches=len(rows), dispatches_averaged=len(used),
                     bytes_avg=sum(used) / len(used) * scale,
                     counter_median=_median(used), counter_min=min(used), counter_max=max(used))
            if len(rows) <= 16:
                d["counter_per_dispatch"] = rows
            per_kernel.setdefault(_short(name), {})[counter] = d
        res[counter] = dict(calibration_counter=c, calibration_bytes=CALIB_BYTES,
                            scale_bytes_per_unit=scale, kernel_bytes_avg=total)
    traffic = res["FETCH_SIZE"]["kernel_bytes_avg"] + res["WRITE_SIZE"]["kernel_bytes_avg"]
    cmds = pmc_commands(workload, regex, dirs) + [
        f"python bench.py --workload {workload} --kernel {kernel} --regex {regex} --summarize-pmc "
        f"{fetch_dir} {write_dir} {cal_fetch_dir} {cal_write_dir}"]
    summary = dict(kernel=kernel, members=[m for m in _family(kernel) if _matching(by_name, m)],
                   workload=workload,
                   kernel_source_hash=kernel_source_hash(kernel), counters=res, per_kernel=per_kernel,
                   traffic_bytes_per_launch=traffic, warmup_dispatches_skipped=skip_first,
                   commands=cmds)
    os.makedirs(out_dir, exist_ok=True)
    base = os.path.join(out_dir, f"{kernel}_{workload}_pmc")
    with open(base + ".json", "w") as f:
        json.dump(summary, f, indent=1)
    lines = [f"# {kernel} on {workload}: HBM traffic counters (FETCH_SIZE, WRITE_SIZE)", "",
             f"Kernel sources hash {summary['kernel_source_hash']} (bench.py reports `traffic` only "
             "while the sources match).  Each counter in a run of its own; the calibration kernel "
             f"(torch's float32 add, {CALIB_BYTES} B read and {CALIB_BYTES} B written) gives the "
             "bytes per counter unit.  The first dispatch of each kernel (warm-up) is left out.", "",
             "Commands (repository root, one MI355X):", ""] + ["    " + c for c in cmds] + [
             "", "| counter | calibration reading | bytes per unit |", "|---|---|---|"]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        r = res[counter]
        lines.append(f"| {counter} | {r['calibration_counter']:.1f} | {r['scale_bytes_per_unit']:.2f} |")
    lines += ["", "| kernel | dispatches | read (MB, avg) | written (MB, avg) |", "|---|---|---|---|"]
    for name, d in sorted(per_kernel.items()):
        f_, w_ = d.get("FETCH_SIZE", {}), d.get("WRITE_SIZE", {})
        lines.append(f"| {name} | {f_.get('dispatches', 0)} | "
                     f"{f_.get('bytes_avg', 0) / 1e6:.3f} | {w_.get('bytes_avg', 0) / 1e6:.3f} |")
    lines += ["", f"Traffic per launch of {kernel}"
              + (" (" + " + ".join(summary["members"]) + ")" if kernel in KERNEL_FAMILIES else "")
              + f": {traffic / 1e6:.3f} MB (read {res['FETCH_SIZE']['kernel_bytes_avg'] / 1e6:.3f}, "
              f"written {res['WRITE_SIZE']['kernel_bytes_avg'] / 1e6:.3f})."]
    with open(base + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(dict(kernel=kernel, workload=workload, traffic=traffic)), flush=True)


def summarize_counters(run_dirs, workload, name, out_dir, commands, skip_first=1):
    """profiles/<name>_<workload>_counters.md from rocprofv3 --pmc runs of
    SQ/GRBM counters: per libgrpo kernel, the median per dispatch of every
    counter (the first ``skip_first`` dispatches left out), and instructions
    per wave."""
    per = {}
    for d in run_dirs:
        for row in _csv_rows(d, "counter_collection.csv"):
            k = _short(row.get("Kernel_Name", ""))
            if "grpo" not in row.get("Kernel_Name", ""):
                continue
            did = int(row["Dispatch_Id"])
            c = row["Counter_Name"]
            per.setdefault(k, {}).setdefault(c, {})
            per[k][c][did] = per[k][c].get(did, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit("no libgrpo counter rows")
    lines = [f"# {name} on {workload}: wave and instruction counters", "",
             f"Kernel sources hash {kernel_source_hash(name)}.  Medians per dispatch over every "
             f"dispatch but the first {skip_first} (warm-up); each counter set in a run of its own.",
             "", "Commands (repository root, one MI355X):", ""] + ["    " + c for c in commands]
    for k in sorted(per):
        lines += ["", f"## {k}", "", "| counter | median per dispatch | dispatches |", "|---|---|---|"]
        med = {}
        for c in sorted(per[k]):
            vals = [v for _, v in sorted(per[k][c].items())]
            used = vals[skip_first:] if len(vals) > skip_first else vals
            med[c] = _median(used)
            lines.append(f"| {c} | {med[c]:.6g} | {len(used)} |")
        waves = med.get("SQ_WAVES")
        if waves:
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_VMEM_RD",
                      "SQ_INSTS_VMEM_WR"):
                if c in med:
                    lines.append(f"| {c} per wave | {med[c] / waves:.1f} | |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{name}_{workload}_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[-12:]), flush=True)


def summarize_trace(run_dir, workload, kernel, out_dir, command, skip_first):
    """profiles/<kernel>_<workload>_kernel_trace.md from a rocprofv3
    --kernel-trace --stats run: per libgrpo kernel, the dispatch count and
    the average, median, minimum and maximum duration over every dispatch
    but the first ``skip_first`` (warm-up), and the average over all."""
    per = {}
    for row in _csv_rows(run_dir, "kernel_trace.csv"):
        name = row.get("Kernel_Name", "")
        if "grpo" not in name:
            continue
        dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3  # us
        per.setdefault(name, []).append((int(row.get("Dispatch_Id", 0)), dur))
    if not per:
        raise SystemExit(f"no libgrpo dispatches under {run_dir}")
    lines = [f"# {kernel} on {workload}: kernel trace", "",
             f"Kernel sources hash {kernel_source_hash(kernel)}.  Durations in microseconds from the "
             f"trace's start and end timestamps; the first {skip_first} dispatches of each kernel "
             "(warm-up) are left out of the average, median, minimum and maximum.", "",
             "Command (repository root, one MI355X):", "", "    " + command, "",
             "| kernel | dispatches | avg us | median us | min us | max us | avg us, all dispatches |",
             "|---|---|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        d = [x for _, x in sorted(v)]
        used = d[skip_first:] if len(d) > skip_first else d
        lines.append(f"| {_short(name)} | {len(d)} | {sum(used) / len(used):.1f} | "
                     f"{_median(used):.1f} | {min(used):.1f} | {max(used):.1f} | "
                     f"{sum(d) / len(d):.1f} |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"{kernel}_{workload}_kernel_trace.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[-len(per):]), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all",
                    help="all | a logits workload (optionally name:reduction) | token_loss_full | "
                         "token_loss_ragged | adv_reinforce_pp | adv_reinforce_pp_baseline | "
                         "pages_shapes")
    ap.add_argument("--objective", default="default", choices=sorted(OBJECTIVES))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=2.5,
                    help="wall seconds of oracle work per workload over the worker processes")
    ap.add_argument("--copies", type=int, default=6, help="input copies rotated by the token-loss bench")
    ap.add_argument("--calibrate-only", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=4, default=None)
    ap.add_argument("--kernel", default="grpo_rows_kernel",
                    help="kernel (or family) named by --summarize-pmc / --summarize-trace")
    ap.add_argument("--regex", default=None, help="the --kernel-include-regex the counter runs used")
    ap.add_argument("--summarize-trace", nargs=1, default=None,
                    help="rocprofv3 --kernel-trace output directory to summarise")
    ap.add_argument("--trace-command", default="", help="the command that made --summarize-trace's run")
    ap.add_argument("--skip-first", type=int, default=1, help="warm-up dispatches left out")
    ap.add_argument("--summarize-counters", nargs="+", default=None,
                    help="rocprofv3 --pmc output directories of SQ/GRBM counter runs to summarise")
    ap.add_argument("--commands", nargs="*", default=[], help="the commands that made those runs")
    args = ap.parse_args()
    if args.calibrate_only:
        calibrate_only()
        return
    if args.summarize_pmc:
        key = args.workload.replace(":", "_")
        summarize_pmc(args.summarize_pmc, key, args.kernel, os.path.join(ROOT, "profiles"),
                      args.skip_first, args.regex)
        return
    if args.workload == "pages_shapes":
        run_pages_shapes(args)
        return
    if args.summarize_counters:
        key = args.workload.replace(":", "_")
        summarize_counters(args.summarize_counters, key, args.kernel, os.path.join(ROOT, "profiles"),
                           args.commands, args.skip_first)
        return
    if args.summarize_trace:
        key = args.workload.replace(":", "_")
        summarize_trace(args.summarize_trace[0], key, args.kernel, os.path.join(ROOT, "profiles"),
                        args.trace_command, args.skip_first)
        return
    ws = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    pool = None
    workers = host_workers()
    if not args.no_cpu_baseline and args.objective == "default":
        if under_profiler():
            _log("under a profiler: no oracle worker processes, cpu_baseline left out")
        else:
            _log(f"starting {workers} oracle worker processes")
            pool = start_pool(workers)
    try:
        if args.workload == "all":
            run_all(args, pool, workers)
        else:
            run_single(args, pool, workers)
    finally:
        if pool is not None:
            pool.terminate()


if __name__ == "__main__":
    main()
