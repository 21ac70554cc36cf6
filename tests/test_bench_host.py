"""Host logic of bench.py, without a GPU: the refusal of more than one GPU,
the byte model of the vocabulary kernel, the counter summary's scaling from
counter units to bytes, the tie of the reported traffic to the kernel
sources, and the CPU-oracle baseline over whole groups."""

import csv
import json
import os
import subprocess
import sys

import bench
from workloads import TOKEN_WORKLOADS, WORKLOADS, make_token_inputs

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
    row = f"void grpo::{bench.ROW_KERNEL}<unsigned short>(grpo::RowArgs)"
    cal = "void at::native::elementwise_kernel<_add<float>>(...)"
    dirs = [str(tmp_path / n) for n in ("f", "w", "cf", "cw")]
    _counter_csv(dirs[0], row, "FETCH_SIZE", [[10.0, 20.0], [40.0, 20.0]])   # 30, 60 per dispatch
    _counter_csv(dirs[1], row, "WRITE_SIZE", [[5.0], [7.0]])
    _counter_csv(dirs[2], cal, "FETCH_SIZE", [[1000.0, 24.0]])             # 1024 units
    _counter_csv(dirs[3], cal, "WRITE_SIZE", [[2048.0]])
    out = tmp_path / "profiles"
    bench.summarize_pmc(dirs, "wl", str(out))
    d = json.load(open(out / f"{bench.ROW_KERNEL}_wl_pmc.json"))
    fetch = 45.0 * bench.CALIB_BYTES / 1024.0
    write = 6.0 * bench.CALIB_BYTES / 2048.0
    assert d["counters"]["FETCH_SIZE"]["row_kernel_counter_per_dispatch"] == [30.0, 60.0]
    assert abs(d["traffic_bytes_per_launch"] - (fetch + write)) <= 1e-9 * (fetch + write)
    assert d["kernel_source_hash"] == bench.kernel_source_hash()


def test_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    path = prof / f"{bench.ROW_KERNEL}_wl_pmc.json"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc")
    assert bench.load_traffic("wl") is None
    path.write_text(json.dumps(dict(kernel_source_hash="abc", traffic_bytes_per_launch=123.0)))
    assert bench.load_traffic("wl") == 123.0
    path.write_text(json.dumps(dict(kernel_source_hash="old", traffic_bytes_per_launch=123.0)))
    assert bench.load_traffic("wl") is None


def test_cpu_baseline_over_whole_groups():
    wl = TOKEN_WORKLOADS["token_loss_ragged"]
    inp = make_token_inputs(wl, device="cpu", seed=0, B=48, T=32)
    sizes = []

    def call(h):
        sizes.append(h["mask"].shape[0])
        assert all(v.shape[0] == h["mask"].shape[0] for v in h.values())
        sum(float(v.sum()) for v in h.values())   # some host work to time

    res = bench.cpu_baseline_groups(wl, inp, call, target_s=0.01, groups_per_chunk=2)
    assert sizes and all(n % wl.group_size == 0 for n in sizes)
    assert res["kind"] == "oracle" and res["cores"] == 1 and res["value"] > 0
    assert f"{sum(sizes)} sequences" in res["sample"]
