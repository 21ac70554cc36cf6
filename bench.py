"""Benchmark of the GRPO loss hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--objective NAME]

One step is one grpo_loss_fwd_bwd call (advantages and weights, the fused
vocabulary pass with the analytic gradient, the fixed-order reductions) over
one batch of synthetic inputs already resident in HBM.  The default workload
is the Qwen-size vocabulary: B = 32 (4 prompts x 8 samples), T = 2048,
V = 151,936, bf16 logits, full mask, token-mean reduction.

Prints one JSON line with tokens/s (all B*T slots per second), the roofline of
the vocabulary kernel (algorithmic bytes over its own HIP-event-timed
duration, against 8 TB/s HBM), and the fp64 CPU oracle's rate on a bounded
sample of the same workload.

--objective selects another per-token or sequence-level objective on the same
workload (default: the clipped surrogate with k3 the workload names).  The
sequence-level ones (gspo, real) run a forward row pass, the per-sequence
phase and a gradient pass; the timed "vocabulary kernel" then spans all three
and the byte model is unchanged (policy read twice, reference once, gradient
written once).

Auxiliary modes (for the HBM-traffic counters, see profiles/):
  --calibrate-only       run only a plain elementwise kernel over 2 GiB that
                         reads and writes known bytes (counter scale)
  --summarize-pmc F W CF CW
                         write profiles/<kernel>_<workload>_pmc.json from four
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
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "tokens/s for fused GRPO fwd+bwd from [B,T,V] logits; % of MI355X peak HBM GB/s"
ROW_KERNEL = "grpo_rows_kernel"
KERNEL_SOURCES = ["rl_post_loss_amd/csrc/grpo_rows.hip", "rl_post_loss_amd/csrc/grpo_rows_resident.hip",
                  "rl_post_loss_amd/csrc/grpo_rowcore.hpp", "rl_post_loss_amd/csrc/grpo_device.hpp",
                  "rl_post_loss_amd/csrc/grpo_internal.hpp", "rl_post_loss_amd/csrc/grpo_objective.hpp",
                  "rl_post_loss_amd/csrc/grpo_api.hip"]
CALIB_BYTES = 1 << 31   # 2 GiB copy for counter calibration

# objective presets: (keyword overrides, needs generating log-probs)
OBJECTIVES = {
    "default": ({}, False),
    "cispo": (dict(pg_loss="cispo"), False),
    "gspo": (dict(pg_loss="gspo", reduction="sequence_mean"), False),
    "real": (dict(pg_loss="real", reduction="token_mean"), False),
    "seq_mask": (dict(tis_type="seq_mask", tis_ratio_min=0.8, tis_ratio_max=1.25), True),
}


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def byte_model(wl, mask_active_rows, rows):
    """Algorithmic HBM bytes of one vocabulary-kernel launch: every active row
    reads the policy row twice and the reference row once and writes the
    gradient row once; a masked row only writes its zero gradient; plus the
    per-slot side inputs (action id, old log-prob, mask byte)."""
    bx = 4 if wl.dtype == "f32" else 2
    bg = bx
    V = wl.V
    ids_bytes = 8
    side = rows * (ids_bytes + 4 + 1)
    return mask_active_rows * V * (3 * bx + bg) + (rows - mask_active_rows) * V * bg + side


def cpu_baseline(wl, inp, target_s=12.0, rows_per_chunk=32):
    """The fp64 oracle as it stands, on successive row chunks of this batch
    until about ``target_s`` seconds of host compute have run."""
    import numpy as np
    import oracle
    h_mask = inp["mask"].cpu().numpy()
    h_rew = inp["rewards"].cpu().numpy()
    groups = wl.groups_kwargs()
    off = oracle.group_offsets(wl.B, groups.get("samples_per_prompt"), groups.get("group_boundaries"))
    A = oracle.group_advantages(h_rew, off, groups.get("leave_one_out", False),
                                groups.get("scale_by_std", True))
    cfg = oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
                            reduction=wl.reductions[0], alpha=wl.alpha)
    _, _, w = oracle.sequence_weights(h_mask, cfg.reduction, cfg.alpha)
    B, T, V = wl.B, wl.T, wl.V
    pol = inp["policy"].view(B * T, V)
    ref = inp["ref"].view(B * T, V)
    ids = inp["action_ids"].view(-1).cpu().numpy()
    old = inp["old_logps"].view(-1).cpu().numpy()
    mflat = h_mask.reshape(-1)
    rows_done = 0
    compute = 0.0
    r0 = 0
    while compute < target_s and r0 < B * T:
        r1 = min(B * T, r0 + rows_per_chunk)
        sel = np.nonzero(mflat[r0:r1])[0] + r0
        x = pol[r0:r1].float().cpu().numpy()[sel - r0]
        y = ref[r0:r1].float().cpu().numpy()[sel - r0]
        seq = sel // T
        t0 = time.perf_counter()
        oracle.logits_rows(x, y, ids[sel], old[sel], A[seq], w[seq], cfg)
        compute += time.perf_counter() - t0
        rows_done += r1 - r0
        r0 = r1
    return dict(value=rows_done / compute, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{rows_done} of {B * T} slots (rows {0}..{r0 - 1}) of the same batch, "
                       f"float64 numpy, single thread, {compute:.1f} s of compute; host copies excluded")


def cpu_baseline_groups(wl, inp, call, target_s=12.0, groups_per_chunk=16):
    """The fp64 oracle as it stands on a [B, T] log-prob batch: ``call`` runs
    it on host arrays of whole groups, a chunk at a time in batch order and
    starting over at the end of the batch, until about ``target_s`` seconds
    of host compute have run.  Each chunk is its own oracle call, so its
    sequence weights and any global statistic are the chunk's; the work per
    slot is the same."""
    h = {k: v.cpu().numpy() for k, v in inp.items()}
    B, T = h["mask"].shape
    size = wl.group_size * groups_per_chunk
    compute = 0.0
    done = 0                      # sequences processed, over all passes
    while compute < target_s:
        start = done % B
        sl = slice(start, min(B, start + size))
        part = {k: v[sl] for k, v in h.items()}
        t0 = time.perf_counter()
        call(part)
        compute += time.perf_counter() - t0
        done += sl.stop - sl.start
    return dict(value=done * T / compute, unit="tokens/s", cores=1, kind="oracle",
                sample=f"{done} sequences ({done * T} slots, {done / B:.2f} passes over the batch of "
                       f"{B}) in chunks of {size} sequences, float64 numpy, single thread, "
                       f"{compute:.1f} s of compute; host copies excluded")


class HipEvents:
    """hipEvent_t pairs created through the HIP runtime (the vocabulary kernel
    is launched by the library on torch's current stream; the library records
    these events right around that launch)."""

    def __init__(self, n):
        import ctypes as C
        self.C = C
        self.hip = C.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = C.c_void_p(), C.c_void_p()
            assert self.hip.hipEventCreate(C.byref(a)) == 0 and self.hip.hipEventCreate(C.byref(b)) == 0
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


def load_traffic(workload):
    """HBM traffic per launch from the committed counter summary, if it was
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{ROW_KERNEL}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


GRAPH_TIMING = ("GPU time per call: the calls captured in one HIP graph per replay (each input "
                "copy in turn), replays timed back to back")


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


def run_token(args):
    """Logprob-level token loss (no vocabulary).  The 71 MB working set fits
    the memory-side cache, so the timed loop rotates over enough input copies
    (each call reads a different one) to keep it from being served there."""
    import torch
    import rl_post_loss_amd as rpl
    from workloads import TOKEN_WORKLOADS, make_token_inputs

    rpl.load_library()
    dev = torch.device("cuda:0")
    wl = TOKEN_WORKLOADS[args.workload]
    copies = [make_token_inputs(wl, device=dev, seed=args.seed + k) for k in range(args.copies)]
    outs = [torch.empty((wl.B, wl.T), dtype=torch.float32, device=dev) for _ in range(args.copies)]
    kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
              samples_per_prompt=wl.group_size, reduction=wl.reduction)

    results = [None] * len(copies)

    def step(k):
        j = k % len(copies)
        c = copies[j]
        results[j] = rpl.grpo_token_loss(c["logp"], c["old_logps"], c["ref_logp"], c["rewards"],
                                         c["mask"], out=results[j], **kw)

    for k in range(max(args.warmup, len(copies))):
        step(k)
    torch.cuda.synchronize()
    # eager calls (Python binding overhead included)
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    ms, ms_graph_per_call = _graph_times(step, len(copies), args.steps)
    m = copies[0]["mask"]
    active = int(m.sum())
    rows = wl.B * wl.T
    alg = active * 17 + (rows - active) * 5
    out = {"metric": "tokens/s for the logprob-level GRPO token loss (forward + dlogp)",
           "value": rows / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": f"{wl.name}: B={wl.B} ({wl.num_groups} groups of {wl.group_size}), "
                                  f"T={wl.T}, {wl.reduction}, input copies rotated: {args.copies}",
                      "active_tokens": active, "algorithmic_bytes": alg,
                      "step_GBps": alg / (ms * 1e-3) / 1e9, "timing": GRAPH_TIMING,
                      "ms_per_step_graph_per_call": ms_graph_per_call,
                      "ms_per_step_eager_python": ms_eager}}
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        import oracle
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cfg = oracle.LossConfig(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta,
                                reduction=wl.reduction)
        out["cpu_baseline"] = cpu_baseline_groups(
            wl, copies[0], lambda h: oracle.grpo_token_loss(
                h["logp"], h["old_logps"], h["ref_logp"], h["mask"], h["rewards"],
                groups=dict(samples_per_prompt=wl.group_size), cfg=cfg),
            target_s=args.cpu_seconds)
    print(json.dumps(out), flush=True)


ADV_WORKLOADS = {"adv_reinforce_pp": "reinforce_pp", "adv_reinforce_pp_baseline": "reinforce_pp_baseline"}


def run_adv(args):
    """Token-level advantage estimator over the log-prob workload's shape
    (B = 1024 in groups of 16, T = 4096, ragged lengths): REINFORCE++
    returns (k1 shaping 0.01, gamma 1) or the inclusive group baseline, with
    the global masked normalization.  Input copies are rotated as for the
    token loss; timed as the token loss is."""
    import torch
    import rl_post_loss_amd as rpl
    from workloads import TOKEN_WORKLOADS, make_token_inputs

    rpl.load_library()
    dev = torch.device("cuda:0")
    est = ADV_WORKLOADS[args.workload]
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    copies = [make_token_inputs(wl, device=dev, seed=args.seed + k) for k in range(args.copies)]
    kw = dict(kl_coef=0.01, gamma=1.0, normalize=True)
    if est == "reinforce_pp_baseline":
        kw = dict(samples_per_prompt=wl.group_size, normalize=True)
    outs = [None] * len(copies)

    def step(k):
        j = k % len(copies)
        c = copies[j]
        extra = dict(old_logps=c["old_logps"], ref_logps=c["ref_logp"]) if est == "reinforce_pp" else {}
        outs[j] = rpl.grpo_token_advantages(est, c["rewards"], c["mask"], **extra, **kw)

    for k in range(max(args.warmup, len(copies))):
        step(k)
    torch.cuda.synchronize()
    ms, ms_graph_per_call = _graph_times(step, len(copies), args.steps)
    rows = wl.B * wl.T
    # minimum bytes: old, ref f32 and the mask read once (REINFORCE++), the output written once
    per_slot = (4 + 4 + 1 + 4) if est == "reinforce_pp" else (1 + 4)
    alg = rows * per_slot
    out = {"metric": "tokens/s for the token-level advantage estimator (returns + global normalization)",
           "value": rows / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f64", "data": "synthetic",
           "config": {"workload": f"{args.workload}: B={wl.B} (groups of {wl.group_size}), T={wl.T}, "
                                  f"ragged lengths, {est}, normalized; input copies rotated: {args.copies}",
                      "algorithmic_bytes": alg, "step_GBps": alg / (ms * 1e-3) / 1e9,
                      "timing": GRAPH_TIMING, "ms_per_step_graph_per_call": ms_graph_per_call}}
    out["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        import oracle
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        if est == "reinforce_pp":
            call = lambda h: oracle.token_advantages(est, h["rewards"], h["old_logps"], h["ref_logp"],
                                                     h["mask"], **kw)
        else:
            call = lambda h: oracle.token_advantages(est, h["rewards"], None, None, h["mask"],
                                                     groups=dict(samples_per_prompt=wl.group_size),
                                                     normalize=True)
        out["cpu_baseline"] = cpu_baseline_groups(wl, copies[0], call, target_s=args.cpu_seconds)
    print(json.dumps(out), flush=True)


def run(args):
    import torch
    import rl_post_loss_amd as rpl
    from workloads import WORKLOADS, make_gen_logps, make_logits_inputs

    rpl.load_library()
    dev = torch.device("cuda:0")
    wl = WORKLOADS[args.workload]
    print(f"[bench] generating {wl.name}: B={wl.B} T={wl.T} V={wl.V} {wl.dtype}", file=sys.stderr,
          flush=True)
    t_gen = time.perf_counter()
    inp = make_logits_inputs(wl, device=dev, seed=args.seed)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    B, T, V = wl.B, wl.T, wl.V
    gdt = inp["policy"].dtype
    grad = torch.empty((B, T, V), dtype=gdt, device=dev)
    kw = dict(eps_low=wl.eps_low, eps_high=wl.eps_high, beta=wl.beta, reduction=wl.reductions[0],
              alpha=wl.alpha)
    kw.update(wl.groups_kwargs())
    obj, needs_gen = OBJECTIVES[args.objective]
    kw.update(obj)
    gen = make_gen_logps(inp["old_logps"], seed=args.seed) if needs_gen else None

    def step():
        return rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                     inp["rewards"], inp["mask"], grad_out=grad, gen_logps=gen, **kw)

    for _ in range(args.warmup):
        res = step()
    torch.cuda.synchronize()
    ref_scalars = res.scalars.clone() if args.warmup else None
    ref_grad_sum = int(grad.view(torch.int16 if grad.element_size() == 2 else torch.int32)
                       .sum(dtype=torch.int64)) if args.warmup else None

    ev = HipEvents(args.steps)
    lib = rpl.load_library()
    step_scalars = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        lib.grpo_set_timing_events(ev.pairs[k][0], ev.pairs[k][1])
        res = step()
        step_scalars.append(res.scalars)  # each call returns its own scalar tensor
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.grpo_set_timing_events(None, None)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = [ev.elapsed_ms(k) for k in range(args.steps)]
    ev.close()
    kern_avg = sum(kern_ms) / len(kern_ms)
    kern_median = sorted(kern_ms)[len(kern_ms) // 2]
    # bit reproducibility: every timed step's scalars equal the warm-up's, and
    # the gradient left by the last step has the warm-up gradient's checksum
    repro = ref_scalars is None or (
        all(torch.equal(ref_scalars.view(torch.int32), sc.view(torch.int32)) for sc in step_scalars)
        and int(grad.view(torch.int16 if grad.element_size() == 2 else torch.int32)
                .sum(dtype=torch.int64)) == ref_grad_sum)

    active = int(inp["mask"].sum())
    rows = B * T
    alg_bytes = byte_model(wl, active, rows)
    achieved = alg_bytes / (kern_avg * 1e-3) / 1e9
    traffic = load_traffic(wl.name) if args.objective == "default" else None
    value = rows / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: B={B} ({len(wl.group_sizes)} groups), T={T}, V={V}, "
                        f"{wl.dtype} logits and gradient, {kw['reduction']}, "
                        f"{'full mask' if wl.len_range is None else 'ragged lengths %d..%d' % wl.len_range}"
                        + ("" if args.objective == "default" else f", objective {args.objective}"),
            "objective": {k: v for k, v in obj.items()},
            "B": B, "T": T, "V": V, "storage": wl.dtype, "active_slots": active,
            "active_tokens_per_s": active / (ms_per_step * 1e-3),
            "hbm_fraction_of_step": alg_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "bit_reproducible": bool(repro),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS,
            "traffic": traffic,
            "kernel": ROW_KERNEL,
            "kernel_ms": kern_avg,
            "kernel_ms_median": kern_median,
            "algorithmic_bytes": alg_bytes,
        },
    }
    if not args.no_cpu_baseline and args.objective == "default":
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, inp, target_s=args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


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


def _pmc_values(d, counter, name_part):
    """Per-dispatch counter values (summed over the csv rows of a dispatch)
    of kernels whose name contains ``name_part``."""
    import csv
    per = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter or name_part not in row.get("Kernel_Name", ""):
                    continue
                did = row.get("Dispatch_Id")
                per[did] = per.get(did, 0.0) + float(row["Counter_Value"])
    return list(per.values())


def summarize_pmc(dirs, workload, out_dir):
    """Combine the four rocprofv3 --pmc runs into profiles/<kernel>_<workload>_pmc.json.
    The counters read over the calibration kernel, which moves a known number
    of bytes each way, give the scale from counter units to bytes."""
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = dirs
    res = {}
    for counter, run_dir, cal_dir in (("FETCH_SIZE", fetch_dir, cal_fetch_dir),
                                      ("WRITE_SIZE", write_dir, cal_write_dir)):
        cal = _pmc_values(cal_dir, counter, "_add<float>")
        rows = _pmc_values(run_dir, counter, ROW_KERNEL)
        if not cal or not rows:
            raise SystemExit(f"missing {counter} values (calibration {len(cal)}, row kernel {len(rows)})")
        c = max(cal)
        scale = CALIB_BYTES / c
        res[counter] = dict(calibration_counter=c, calibration_bytes=CALIB_BYTES,
                            scale_bytes_per_unit=scale,
                            row_kernel_counter_per_dispatch=rows,
                            row_kernel_bytes_avg=sum(rows) / len(rows) * scale)
    traffic = res["FETCH_SIZE"]["row_kernel_bytes_avg"] + res["WRITE_SIZE"]["row_kernel_bytes_avg"]
    summary = dict(kernel=ROW_KERNEL, workload=workload, kernel_source_hash=kernel_source_hash(),
                   counters=res, traffic_bytes_per_launch=traffic,
                   commands=["rocprofv3 --pmc FETCH_SIZE --kernel-include-regex grpo_rows -f csv "
                             f"-d {fetch_dir} -o run -- python3 bench.py --workload {workload} "
                             "--steps 3 --warmup 1 --no-cpu-baseline",
                             "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex grpo_rows -f csv "
                             f"-d {write_dir} -o run -- python3 bench.py --workload {workload} "
                             "--steps 3 --warmup 1 --no-cpu-baseline",
                             "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex elementwise -f csv "
                             f"-d {cal_fetch_dir} -o run -- python3 bench.py --calibrate-only",
                             "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex elementwise -f csv "
                             f"-d {cal_write_dir} -o run -- python3 bench.py --calibrate-only",
                             f"python bench.py --workload {workload} --summarize-pmc "
                             f"{fetch_dir} {write_dir} {cal_fetch_dir} {cal_write_dir}"])
    os.makedirs(out_dir, exist_ok=True)
    base = os.path.join(out_dir, f"{ROW_KERNEL}_{workload}_pmc")
    with open(base + ".json", "w") as f:
        json.dump(summary, f, indent=1)
    print(json.dumps(summary, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="logits_v151936")
    ap.add_argument("--objective", default="default", choices=sorted(OBJECTIVES))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copies", type=int, default=6, help="input copies rotated by the token-loss bench")
    ap.add_argument("--calibrate-only", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=4, default=None)
    args = ap.parse_args()
    if args.calibrate_only:
        calibrate_only()
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.workload, os.path.join(ROOT, "profiles"))
        return
    ws = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.workload.startswith("token_loss"):
        run_token(args)
    elif args.workload in ADV_WORKLOADS:
        run_adv(args)
    else:
        run(args)


if __name__ == "__main__":
    main()
