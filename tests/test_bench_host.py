"""Host-side logic of bench.py (no GPU): the one-GPU guard, the choice of
dominant kernel per workload, and the counter summariser that turns
rocprofv3 FETCH_SIZE / WRITE_SIZE readings into HBM bytes per launch."""
import csv
import importlib.util
import os
import subprocess
import sys

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_dominant_kernel_per_workload():
    b = _bench()
    kern = {name: b.dominant_kernel(workloads.layer_specs(name)[0]) for name in workloads.WORKLOADS}
    # batch 1 at 4096^2 fits the single-launch layer; 16 rows take the GEMV;
    # 2048 and 4096 rows the 8-wave GEMM (k a multiple of 64); the float32
    # workload its own kernel
    assert kern == {"small": "gemv_f32<2>", "gemv": "layer_small<2>", "batch16": "gemv_bf16<4>",
                    "prefill_up": "gemm8_bf16<3>", "dit_block": "gemm8_bf16<4>"}
    assert b.single_launch(workloads.layer_specs("gemv")[0])
    assert not b.single_launch(workloads.layer_specs("batch16")[0])
    assert b.operand_layout(workloads.layer_specs("batch16")[0])


def test_committed_traffic_profiles_name_the_dominant_kernels():
    # every committed counter profile parses and names the kernel the bench
    # prices for that workload (the bench drops it if the source hash differs)
    b = _bench()
    for name in ("gemv", "batch16", "prefill_up", "dit_block"):
        p = b._profile_path(name)
        assert os.path.exists(p), p
        kv = dict(line.split(":", 1) for line in open(p) if ":" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        assert kv["workload"] == name
        assert kv["kernel"] == b.dominant_kernel(workloads.layer_specs(name)[0])
        assert float(kv["hbm_bytes_per_dispatch"]) > 0
        assert len(kv["kernel_source_sha256_16"]) == 16


def _counter_dir(tmp_path, name, rows):
    d = tmp_path / name
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kname, counter, value in rows:
            w.writerow({"Kernel_Name": kname, "Counter_Name": counter, "Counter_Value": value})
    return str(d)


def test_pmc_summary_scales_by_the_copy_and_takes_medians(tmp_path, monkeypatch):
    # synthetic counter files: the copy reads half its bytes on FETCH_SIZE
    # (factor 2) and all of them on WRITE_SIZE (factor 1); the kernel's
    # medians are 300 and 50 KiB, so HBM bytes = (300 * 2 + 50) * 1024
    b = _bench()
    copy_kib = b.COPY_BYTES / 1024.0
    cf = _counter_dir(tmp_path, "cf", [("copy", "FETCH_SIZE", copy_kib / 2), ("copy", "FETCH_SIZE", 10.0)])
    cw = _counter_dir(tmp_path, "cw", [("copy", "WRITE_SIZE", copy_kib)])
    bf = _counter_dir(tmp_path, "bf", [("k<4>", "FETCH_SIZE", v) for v in (100.0, 300.0, 900.0)] +
                      [("other", "FETCH_SIZE", 1e9)])
    bw = _counter_dir(tmp_path, "bw", [("k<4>", "WRITE_SIZE", v) for v in (50.0, 50.0, 70.0)])
    monkeypatch.setattr(b, "PROFILE_DIR", str(tmp_path / "profiles"))
    args = type("A", (), {"pmc_summary": (cf, cw, bf, bw), "pmc_kernel": "k<4>", "pmc_kernel_label": "k<4>",
                          "copy_kernel": "copy", "pmc_commands": "synthetic", "workload": "unit"})()
    b.pmc_summary(args)
    kv = dict(line.split(":", 1) for line in open(b._profile_path("unit")) if not line.startswith("#"))
    assert float(kv["hbm_bytes_per_dispatch"]) == pytest.approx((300.0 * 2 + 50.0) * 1024.0, rel=1e-6)
    assert float(kv["copy_fetch_factor"]) == pytest.approx(2.0)
    # the bench reads it back only while the kernel source is unchanged
    assert b.read_traffic("unit", "k<4>") == pytest.approx((300.0 * 2 + 50.0) * 1024.0, rel=1e-6)
    assert b.read_traffic("unit", "other<4>") is None
    monkeypatch.setattr(b, "kernel_source_hash", lambda: "0" * 16)
    assert b.read_traffic("unit", "k<4>") is None


def test_invalid_step_counts_exit_with_a_message():
    for args in (["--steps", "0"], ["--warmup", "-1"], ["--warm-seconds", "-0.5"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                           text=True, timeout=120)
        assert r.returncode == 2, args
        assert "--steps" in r.stderr
