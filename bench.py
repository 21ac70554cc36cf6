"""Benchmark of the GRPO loss hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME]

One step is one grpo_loss_fwd_bwd call (advantages and weights, the fused
vocabulary pass with the analytic gradient, the fixed-order reductions) over
one batch of synthetic inputs already resident in HBM.  The default workload
is the Qwen-size vocabulary: B = 32 (4 prompts x 8 samples), T = 2048,
V = 151,936, bf16 logits, full mask, token-mean reduction.

Prints one JSON line with tokens/s (all B*T slots per second), the roofline of
the vocabulary kernel (algorithmic bytes over its own HIP-event-timed
duration, against 8 TB/s HBM), and the fp64 CPU oracle's rate on a bounded
sample of the same workload.

Auxiliary modes:
  --calibrate            also run a plain device copy of known size (for the
                         counter scaling of rocprofv3 --pmc runs)
  --summarize-pmc DIR... write a profiles/ summary from rocprofv3 csv output
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
KERNEL_SOURCES = ["rl_post_loss_amd/csrc/grpo_rows.hip", "rl_post_loss_amd/csrc/grpo_device.hpp",
                  "rl_post_loss_amd/csrc/grpo_internal.hpp", "rl_post_loss_amd/csrc/grpo_api.hip"]
CALIB_BYTES = 1 << 31   # 2 GiB copy for counter calibration


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


def run(args):
    import torch
    import rl_post_loss_amd as rpl
    from workloads import WORKLOADS, make_logits_inputs

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

    def step():
        return rpl.grpo_loss_fwd_bwd(inp["policy"], inp["ref"], inp["action_ids"], inp["old_logps"],
                                     inp["rewards"], inp["mask"], grad_out=grad, **kw)

    if args.calibrate:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        res = step()
    torch.cuda.synchronize()
    ref_scalars = res.scalars.clone() if args.warmup else None

    ev = HipEvents(args.steps)
    lib = rpl.load_library()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        lib.grpo_set_timing_events(ev.pairs[k][0], ev.pairs[k][1])
        res = step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    lib.grpo_set_timing_events(None, None)
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = [ev.elapsed_ms(k) for k in range(args.steps)]
    ev.close()
    kern_avg = sum(kern_ms) / len(kern_ms)
    repro = ref_scalars is None or torch.equal(ref_scalars.view(torch.int32), res.scalars.view(torch.int32))

    active = int(inp["mask"].sum())
    rows = B * T
    alg_bytes = byte_model(wl, active, rows)
    achieved = alg_bytes / (kern_avg * 1e-3) / 1e9
    traffic = load_traffic(wl.name)
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
                        f"{wl.dtype} logits and gradient, {wl.reductions[0]}, "
                        f"{'full mask' if wl.len_range is None else 'ragged lengths %d..%d' % wl.len_range}",
            "B": B, "T": T, "V": V, "storage": wl.dtype, "active_slots": active,
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
            "algorithmic_bytes": alg_bytes,
        },
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, inp, target_s=args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


def summarize_pmc(dirs, workload, out_dir):
    """Combine a FETCH_SIZE run and a WRITE_SIZE run (rocprofv3 csv output
    under ``dirs``) into profiles/<kernel>_<workload>_pmc.json + .txt.  The
    counters of the calibration copy (2 GiB read, 2 GiB written) give the
    scale from counter units to bytes."""
    import csv
    vals = {"FETCH_SIZE": {}, "WRITE_SIZE": {}}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(path) as f:
                for row in csv.DictReader(f):
                    name = row.get("Counter_Name")
                    if name not in vals:
                        continue
                    kern = row.get("Kernel_Name", "")
                    key = "copy" if ("copy" in kern.lower() or "elementwise" in kern.lower()) else \
                          ("rows" if ROW_KERNEL in kern else None)
                    if key is None:
                        continue
                    did = row.get("Dispatch_Id")
                    vals[name].setdefault(key, {}).setdefault(did, 0.0)
                    vals[name][key][did] += float(row["Counter_Value"])
    res = {}
    for name, per in vals.items():
        copy = max(per.get("copy", {}).values(), default=None)
        rows = list(per.get("rows", {}).values())
        if copy is None or not rows:
            raise SystemExit(f"missing {name} data for the copy or the row kernel")
        scale = CALIB_BYTES / copy          # bytes per counter unit
        res[name] = dict(copy_counter=copy, scale_bytes_per_unit=scale,
                         row_kernel_counter_avg=sum(rows) / len(rows),
                         row_kernel_bytes_avg=sum(rows) / len(rows) * scale, dispatches=len(rows))
    traffic = res["FETCH_SIZE"]["row_kernel_bytes_avg"] + res["WRITE_SIZE"]["row_kernel_bytes_avg"]
    summary = dict(kernel=ROW_KERNEL, workload=workload, kernel_source_hash=kernel_source_hash(),
                   counters=res, traffic_bytes_per_launch=traffic)
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
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate", action="store_true")
    ap.add_argument("--summarize-pmc", nargs="+", default=None)
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.workload, os.path.join(ROOT, "profiles"))
        return
    ws = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    run(args)


if __name__ == "__main__":
    main()
