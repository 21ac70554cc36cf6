"""Host logic of bench.py, without a GPU: the refusal of more than one GPU,
the byte models of the vocabulary and token kernels, the counter summary's
scaling from counter units to bytes, the tie of the reported traffic to the
kernel sources, and the CPU-oracle baselines over worker processes."""

import csv
import json
import os
import subprocess
import sys

import bench
from workloads import TOKEN_WORKLOADS, WORKLOADS, make_logits_inputs, make_token_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, "bench.py", *args], cwd=ROOT, capture_output=True,
                           text=True, timeout=300, env={**os.environ, **env})
        assert r.returncode == 2, (args, env, r.stderr)
        assert "one GPU" in r.stderr
        assert r.stdout == ""


def test_byte_model():
    wl = WORKLOADS["logits_v151936"]
    rows = wl.B * wl.T
    # every row active: policy twice, reference once, gradient once, bf16
    # (2 bytes each), plus 13 bytes of side inputs per slot
    assert bench.byte_model(wl, rows, rows) == rows * wl.V * 8 + rows * 13 == 79_659_073_536
    # a masked row only writes its zero gradient row
    assert bench.byte_model(wl, 0, rows) == rows * wl.V * 2 + rows * 13
    tiny = WORKLOADS["tiny_logits"]   # float32
    n = tiny.B * tiny.T
    assert bench.byte_model(tiny, 10, n) == 10 * tiny.V * 16 + (n - 10) * tiny.V * 4 + n * 13
    # the resident kernel reads an active policy row once: one policy pass fewer
    v32 = WORKLOADS["logits_v32000"]
    n = v32.B * v32.T
    assert bench.byte_model(v32, 100, n) - bench.min_bytes(v32, 100, n, True) == 100 * v32.V * 2
    # the streaming kernel keeps HELD_CHUNKS chunks of each active policy row in LDS
    # (rows above 64 KB: the 1024-thread kernel); shorter streaming rows hold none
    held = min(wl.V * 2 // 16, bench.HELD_CHUNKS) * 16
    assert bench.min_bytes(wl, rows, rows, False) == bench.byte_model(wl, rows, rows) - rows * held
    assert bench.min_bytes(tiny, 10, n, False) == bench.byte_model(tiny, 10, n)
    assert bench._resident(v32)
    assert not bench._resident(WORKLOADS["logits_csr_v128256"])
    assert not bench._resident(wl) and not bench._resident(tiny)
    # token loss: 17 B per active token, 5 B per masked one
    assert bench.token_bytes(4_194_304, 4_194_304) == 71_303_168
    assert bench.token_bytes(10, 30) == 10 * 17 + 20 * 5


def _counter_csv(d, kernel, counter, values):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for did, parts in enumerate(values):
            for v in parts:          # one row per hardware instance, summed per dispatch
                w.writerow(dict(Dispatch_Id=did, Kernel_Name=kernel, Counter_Name=counter,
                                Counter_Value=v))


def test_summarize_pmc_scales_by_the_calibration_kernel(tmp_path):
    row = "void grpo::grpo_rows_kernel<unsigned short>(grpo::RowArgs)"
    cal = "void at::native::elementwise_kernel<_add<float>>(...)"
    dirs = [str(tmp_path / n) for n in ("f", "w", "cf", "cw")]
    # dispatch 0 is the warm-up, left out of the average
    _counter_csv(dirs[0], row, "FETCH_SIZE", [[1.0], [10.0, 20.0], [40.0, 20.0]])   # 30, 60
    _counter_csv(dirs[1], row, "WRITE_SIZE", [[1.0], [5.0], [7.0]])
    _counter_csv(dirs[2], cal, "FETCH_SIZE", [[1000.0, 24.0]])             # 1024 units
    _counter_csv(dirs[3], cal, "WRITE_SIZE", [[2048.0]])
    out = tmp_path / "profiles"
    bench.summarize_pmc(dirs, "wl", "grpo_rows_kernel", str(out))
    d = json.load(open(out / "grpo_rows_kernel_wl_pmc.json"))
    fetch = 45.0 * bench.CALIB_BYTES / 1024.0
    write = 6.0 * bench.CALIB_BYTES / 2048.0
    per = d["per_kernel"]["grpo_rows_kernel<unsigned short>"]["FETCH_SIZE"]
    assert per["counter_per_dispatch"] == [1.0, 30.0, 60.0]
    assert per["dispatches_averaged"] == 2
    assert abs(d["traffic_bytes_per_launch"] - (fetch + write)) <= 1e-9 * (fetch + write)
    assert d["kernel_source_hash"] == bench.kernel_source_hash("grpo_rows_kernel")
    assert (out / "grpo_rows_kernel_wl_pmc.md").read_text().count("| FETCH_SIZE |") == 1


def test_summarize_pmc_sums_a_kernel_family(tmp_path):
    """The estimator's traffic per call: the averages of its kernels, summed."""
    scan = "grpo::grpo_tokadv_kernel(grpo::TokAdvArgs)"
    norm = "void grpo::grpo_tokadv_norm_kernel<true>(grpo::TokAdvArgs, int)"
    cal = "void at::native::elementwise_kernel<_add<float>>(...)"
    dirs = [str(tmp_path / n) for n in ("f", "w", "cf", "cw")]
    import csv
    for d, counter, vals in ((dirs[0], "FETCH_SIZE", (4.0, 2.0)), (dirs[1], "WRITE_SIZE", (1.0, 3.0))):
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                              "Counter_Value"])
            w.writeheader()
            for call in range(3):   # call 0 is the warm-up
                w.writerow(dict(Dispatch_Id=2 * call, Kernel_Name=scan, Counter_Name=counter,
                                Counter_Value=vals[0] * (1 + call)))
                w.writerow(dict(Dispatch_Id=2 * call + 1, Kernel_Name=norm, Counter_Name=counter,
                                Counter_Value=vals[1] * (1 + call)))
    _counter_csv(dirs[2], cal, "FETCH_SIZE", [[1024.0]])
    _counter_csv(dirs[3], cal, "WRITE_SIZE", [[1024.0]])
    out = tmp_path / "profiles"
    bench.summarize_pmc(dirs, "wl", "grpo_tokadv_kernels", str(out), regex="grpo_tokadv")
    d = json.load(open(out / "grpo_tokadv_kernels_wl_pmc.json"))
    unit = bench.CALIB_BYTES / 1024.0
    want = (4.0 + 2.0) * 2.5 * unit + (1.0 + 3.0) * 2.5 * unit   # calls 1 and 2 averaged
    assert abs(d["traffic_bytes_per_launch"] - want) <= 1e-9 * want
    assert d["members"] == ["grpo_tokadv_kernel(", "grpo_tokadv_norm_kernel"]   # the members launched


def test_summarize_trace_skips_the_warmup(tmp_path):
    import csv
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Start_Timestamp",
                                          "End_Timestamp"])
        w.writeheader()
        for k, us in enumerate((50.0, 10.0, 12.0, 11.0)):
            w.writerow(dict(Dispatch_Id=k, Kernel_Name="void grpo::grpo_token_kernel<false, 2>(x)",
                            Start_Timestamp=1000 * k * 100, End_Timestamp=int(1000 * (k * 100 + us))))
        w.writerow(dict(Dispatch_Id=9, Kernel_Name="other_kernel", Start_Timestamp=0, End_Timestamp=5))
    out = tmp_path / "profiles"
    bench.summarize_trace(str(d), "wl", "grpo_token_kernel", str(out), "rocprofv3 ...", 1)
    text = (out / "grpo_token_kernel_wl_kernel_trace.md").read_text()
    assert "| grpo_token_kernel<false, 2> | 4 | 11.0 | 11.0 | 10.0 | 12.0 | 20.8 |" in text
    assert "other_kernel" not in text


def test_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    path = prof / "grpo_token_kernel_wl_pmc.json"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda kernel=None: "abc")
    assert bench.load_traffic("grpo_token_kernel", "wl") is None
    path.write_text(json.dumps(dict(kernel_source_hash="abc", traffic_bytes_per_launch=123.0)))
    assert bench.load_traffic("grpo_token_kernel", "wl") == 123.0
    path.write_text(json.dumps(dict(kernel_source_hash="old", traffic_bytes_per_launch=123.0)))
    assert bench.load_traffic("grpo_token_kernel", "wl") is None


def test_cpu_baselines_over_worker_processes():
    """The oracle baselines run on spawned worker processes: the token loss
    and the advantage estimators over whole groups, the logits rows from
    float32 sample files."""
    import torch
    pool = bench.start_pool(2)
    try:
        wl = TOKEN_WORKLOADS["token_loss_ragged"]
        inp = make_token_inputs(wl, device="cpu", seed=0, B=48, T=32)
        res = bench.cpu_baseline_tokens(pool, 2, wl, inp, target_s=0.05)
        assert res["kind"] == "oracle" and res["cores"] == 2 and res["value"] > 0
        assert "jobs of 16 sequences" in res["sample"]
        lw = WORKLOADS["logits_v32000"].scaled(T=8, V=300, prompts=2)
        linp = make_logits_inputs(lw, device="cpu", seed=1)
        res = bench.cpu_baseline_logits(pool, 2, lw, linp, "token_mean", {}, 0.05, 64)
        assert res["value"] > 0 and res["cores"] == 2 and "slots 0..63" in res["sample"]
        for est in ("reinforce_pp", "reinforce_pp_baseline"):
            res = bench.cpu_baseline_adv(pool, 2, wl, est, inp, 0.05)
            assert res["value"] > 0 and res["cores"] == 2 and "one group (16 sequences)" in res["sample"]
    finally:
        pool.terminate()


def test_profiler_guard(monkeypatch):
    monkeypatch.delenv("LD_PRELOAD", raising=False)
    for k in list(os.environ):
        if k.startswith("ROCPROF"):
            monkeypatch.delenv(k)
    assert not bench.under_profiler()
    monkeypatch.setenv("LD_PRELOAD", "/opt/rocm/lib/librocprofiler-sdk-tool.so")
    assert bench.under_profiler()


def test_source_hash_follows_the_family(tmp_path, monkeypatch):
    """An edit to the estimator's source leaves the logits kernels' profiles
    current and makes the estimator's stale; an edit to a shared header makes
    every family's stale."""
    import shutil
    for rel in bench.KERNEL_SOURCES:
        dst = tmp_path / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(bench.ROOT, rel), dst)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    fams = ("grpo_rows_kernel", "grpo_token_kernel", "grpo_tokadv_kernels")
    before = {k: bench.kernel_source_hash(k) for k in fams}
    with open(tmp_path / "rl_post_loss_amd/csrc/grpo_adv.hip", "a") as f:
        f.write("\n// edited\n")
    after = {k: bench.kernel_source_hash(k) for k in fams}
    assert after["grpo_rows_kernel"] == before["grpo_rows_kernel"]
    assert after["grpo_token_kernel"] == before["grpo_token_kernel"]
    assert after["grpo_tokadv_kernels"] != before["grpo_tokadv_kernels"]
    with open(tmp_path / "rl_post_loss_amd/csrc/grpo_device.hpp", "a") as f:
        f.write("\n// edited\n")
    assert all(bench.kernel_source_hash(k) != after[k] for k in fams)
