"""Benchmark of the fused E8-decode linear layer on one MI355X.

Default (--workload suite): the headline is the diffusion-transformer block,
the largest workload: Q, K, V, O 3072x3072, up 12288x3072, down 3072x12288,
4 bpw, 4096 bf16 activation rows per linear. One step is the full forward
y = U^T (s W^) (V x) of all six linears (input RHT, fused decode-GEMM, output
RHT each), all in libglq.so; exactly --steps steps are timed (HIP-graph
replays, HIP events around them) after --warmup eager steps and
--warm-seconds of untimed replays, rotating through distinct copies of the
index planes (10 x 57 MB, twice the 256 MB Infinity Cache) so each step
streams its compressed weights from HBM. value = 2 m n k summed over the
block per second (TFLOP/s). Beside it, in "workloads": the batch-1 4096x4096
2 bpw layer (GB/s of compressed weights, sustained and single-call), the
batch-16 4 bpw layer and the 2048-token 16384x4096 3 bpw prefill layer, each
timed the same way with its own step count.

roofline = the dominant kernel (the decode-GEMM / GEMV / whole-layer kernel)
timed alone with HIP events on its launch stream (graph replays): its
algorithmic work per launch (2 m n k flops against 2.5 PFLOP/s bf16 MFMA, or
compressed bytes against 8 TB/s HBM at m <= 16) / its mean launch duration;
for the block, summed over its six linears. traffic = HBM bytes per launch
from rocprofv3 FETCH_SIZE + WRITE_SIZE counters (profiles/), scaled by what
the counters read for a plain copy of known size; null if the kernel source
has changed since those counters were taken.
cpu_baseline = the oracle's float64 forward on the host (decode, both RHTs,
matmul), on a bounded sample of the same workload.
vs_uncompressed_bf16 = the same six products as torch.matmul (hipBLASLt) on
dense bf16 weights.

Other modes (profiling helpers and single workloads):
  --workload gemv|batch16|prefill_up|dit_block|small   one workload as the line
  --copy-calibration                              a plain device copy of known size
  --row-scale                                     layers encoded with per-row scales
  --achievable                                    stream-read, copy and bf16 matmul ceilings
  --encoder                                       CPU encoder: plain vs LDLQ time and proxy loss
  --ep-decode BPP                                 entropy-coded format: decode time at that rate
  --pmc-summary DIR                               turn rocprofv3 counter CSVs into a profile file
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KERNEL_SRC = os.path.join(ROOT, "dequant_e8_codebook_amd", "csrc", "glq_kernels.hip")
PROFILE_DIR = os.path.join(ROOT, "profiles")
COPY_BYTES = 256 << 20


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _profile_path(workload):
    return os.path.join(PROFILE_DIR, f"pmc_traffic_{workload}.txt")


def read_traffic(workload, dominant):
    """HBM bytes per launch of the dominant kernel from the committed counter
    profile, or None if absent or taken on a different kernel source."""
    p = _profile_path(workload)
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash() or kv.get("kernel") != dominant:
        return None
    try:
        return float(kv["hbm_bytes_per_dispatch"])
    except (KeyError, ValueError):
        return None


# ------------------------------------------------------------------ workload

def build_layers(workload, n_layers, device, row_scale=False):
    import numpy as np
    import torch
    from dequant_e8_codebook_amd import glq
    import workloads as wl

    specs = wl.layer_specs(workload)
    cb = glq.device_codebook(device)
    built = []
    for spec in specs:
        w = wl.weights(spec).astype(np.float32)
        sn, sk = wl.sign_n(spec), wl.sign_k(spec)
        i1, i2, s = glq.encode_ref(w, spec.bpw, sn, sk, per_row=row_scale)
        base = glq.Layer.from_numpy(i1, i2, s, sn, sk, cb, device=device)
        copies = [base]
        for _ in range(n_layers - 1):
            copies.append(glq.Layer(base.n, base.k, base.bpw, base.scale, base.idx1.clone(),
                                    None if base.idx2 is None else base.idx2.clone(),
                                    base.sign_k, base.sign_n, cb, base.row_scale))
        x = wl.activations(spec)
        xdt = torch.float32 if spec.x_dtype == "f32" else torch.bfloat16
        ydt = torch.float32 if spec.y_dtype == "f32" else torch.bfloat16
        xt = torch.from_numpy(x).to(device=device, dtype=xdt)
        y = torch.empty((spec.m, spec.n), device=device, dtype=ydt)
        ws = torch.zeros(glq.workspace_bytes(base, spec.m), device=device, dtype=torch.uint8)
        built.append(dict(spec=spec, layers=copies, x=xt, y=y, ws=ws, idx=(i1, i2, s, sn, sk), xnp=x))
    return built


def single_launch(spec):
    """True when a full layer forward of this shape is one kernel (the
    small-batch whole-layer kernel): bf16 x, m <= 4, m*k and m*n <= 16384,
    k/8 a multiple of 8."""
    return (spec.x_dtype == "bf16" and spec.m <= 4 and spec.m * spec.k <= 16384
            and spec.m * spec.n <= 16384 and (spec.k // 8) % 8 == 0)


def operand_layout(spec):
    """True when the library writes x~ in the small-batch GEMV's operand
    layout (its input transform does it): bf16 x, m <= 16 and k a multiple of
    256 and at most 16384, outside the single-launch shapes."""
    return (spec.x_dtype == "bf16" and spec.m <= 16 and spec.k % 256 == 0 and spec.k <= 16384
            and not single_launch(spec))


def dominant_kernel(spec):
    if spec.x_dtype == "f32":
        return f"gemv_f32<{spec.bpw}>"
    if single_launch(spec):
        return f"layer_small<{spec.bpw}>"
    if spec.m <= 16:
        return f"gemv_bf16<{spec.bpw}>"
    # k a multiple of 64: the 8-wave GEMM; other k: the 4-wave one
    return f"gemm8_bf16<{spec.bpw}>" if spec.k % 64 == 0 else f"gemm_bf16<{spec.bpw}>"


def _event():
    import torch
    return torch.cuda.Event(enable_timing=True)


def _graph_seconds(g, reps):
    """Seconds for `reps` replays of a captured graph (one warm replay first)."""
    import torch
    g.replay()
    torch.cuda.synchronize()
    k0, k1 = _event(), _event()
    k0.record()
    for _ in range(reps):
        g.replay()
    k1.record()
    torch.cuda.synchronize()
    return k0.elapsed_time(k1) * 1e-3


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def layer_bytes(L):
    """Algorithmic bytes of a layer: its index planes, plus the row-scale
    vector when there is one."""
    return (L.idx1.numel() * 2 + (0 if L.idx2 is None else L.idx2.numel() * L.idx2.element_size())
            + (0 if L.row_scale is None else L.row_scale.numel() * 4))


def time_workload(name, steps, warmup, copies, row_scale=False, kernel_launches=1024, built=None, warm_s=0.1):
    """Time exactly `steps` whole-layer forward steps of a workload (every
    linear of it per step), rotating through `copies` distinct copies of the
    index planes, plus its dominant kernel alone. Untimed first: `warmup`
    eager steps, one replay of each captured graph, and graph replays for
    `warm_s` seconds. Returns (result, built)."""
    import torch
    from dequant_e8_codebook_amd import glq

    if built is None:
        built = build_layers(name, copies, "cuda:0", row_scale=row_scale)
    per_graph = len(built[0]["layers"])
    comp_bytes = sum(layer_bytes(b["layers"][0]) for b in built)
    flops = sum(2.0 * b["spec"].m * b["spec"].n * b["spec"].k for b in built)

    def step(i):
        for b in built:
            glq.fused_linear(b["layers"][i % per_graph], b["x"], b["y"], b["ws"])

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    # Exactly `steps` steps: full graphs of one step per layer copy, then one
    # graph of the remaining steps. HIP-graph replays, so the time is GPU time,
    # not Python/ctypes launch cost.
    full, rem = divmod(steps, per_graph)
    g_full = _capture(lambda: [step(i) for i in range(per_graph)]) if full else None
    g_rem = _capture(lambda: [step(i) for i in range(rem)]) if rem else None
    for g in (g_full, g_rem):
        if g is not None:
            g.replay()
    torch.cuda.synchronize()
    # untimed graph replays until warm_s of wall time has passed, so that the
    # timed steps start at the clock the GPU holds under this load (the first
    # ~50 ms of a run measured 1-3% slower than the rest)
    warm_steps = max(warmup, 1) + (per_graph if full else 0) + rem
    gw, gw_steps = (g_full, per_graph) if full else (g_rem, rem)
    w0 = time.perf_counter()
    while time.perf_counter() - w0 < warm_s:
        gw.replay()
        torch.cuda.synchronize()
        warm_steps += gw_steps
    t0, t1 = _event(), _event()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(full):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1)
    ms_step = ms / steps
    gbs = comp_bytes * steps / (ms * 1e-3) / 1e9
    tflops = flops * steps / (ms * 1e-3) / 1e12

    # eager (no graph) steps for reference
    n_eager = min(steps, 64)
    e0, e1 = _event(), _event()
    e0.record()
    for i in range(n_eager):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_ms_step = e0.elapsed_time(e1) / n_eager

    spec0 = built[0]["spec"]
    hbm_bound = spec0.m <= 16
    dom = dominant_kernel(spec0)
    one_kernel = single_launch(spec0) and len(built) == 1
    per_linear = []
    for b in built:
        spec = b["spec"]
        Ls = b["layers"]
        reps = max(1, kernel_launches // len(Ls))
        xr = b["x"].clone()
        zt = torch.empty_like(b["y"])
        if one_kernel:
            # the whole layer is one kernel: its launches are the timed steps
            k_mean = ms_step * 1e-3
            how = (f"the timed steps themselves ({steps} whole-layer launches in HIP-graph replays, "
                   "HIP events around them)")
        elif spec.x_dtype == "f32":
            glq.rht_apply(b["x"], xr, Ls[0].sign_k, False)
            flags = glq.FLAG_NO_INPUT_RHT | glq.FLAG_NO_OUTPUT_RHT
            g = _capture(lambda: [glq.fused_linear(L, xr, zt, b["ws"], flags) for L in Ls])
            k_mean = _graph_seconds(g, reps) / (reps * len(Ls))
            how = f"HIP events around {reps} replays of a graph of {len(Ls)} launches (x pre-rotated)"
        else:
            # the kernel reads x~ as the library's own input transform writes it
            # (with row sums at 3/4 bpw, or in the GEMV's operand layout), which
            # a pre-rotated x cannot give: time (input transform + kernel) and
            # subtract the row-major input transform of the same rows alone
            ga = _capture(lambda: [glq.fused_linear(L, b["x"], zt, b["ws"], glq.FLAG_NO_OUTPUT_RHT) for L in Ls])
            gb = _capture(lambda: [glq.rht_apply(b["x"], xr, L.sign_k, False) for L in Ls])
            k_mean = (_graph_seconds(ga, reps) - _graph_seconds(gb, reps)) / (reps * len(Ls))
            how = (f"HIP events around {reps} replays of a graph of {len(Ls)} (input transform + kernel) "
                   f"launch pairs, minus the same for the input transform alone")
        kb = layer_bytes(Ls[0])
        kf = 2.0 * spec.m * spec.n * spec.k
        per_linear.append({"layer": f"{spec.n}x{spec.k}", "kernel_mean_us": round(k_mean * 1e6, 3),
                           "algorithmic_bytes": kb, "algorithmic_flops": kf, "timing": how})
    k_total = sum(p["kernel_mean_us"] for p in per_linear) * 1e-6
    k_bytes = sum(p["algorithmic_bytes"] for p in per_linear)
    k_flops = sum(p["algorithmic_flops"] for p in per_linear)
    if hbm_bound:
        achieved = k_bytes / k_total / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
    else:
        achieved = k_flops / k_total / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / MFMA_BF16_PEAK_TFLOPS, 4))
    roof["traffic"] = read_traffic(name, dom)
    roof["kernel"] = dom
    roof["kernel_mean_us"] = round(k_total * 1e6 / len(per_linear), 3)
    roof["algorithmic_bytes_per_launch"] = round(k_bytes / len(per_linear))
    roof["algorithmic_flops_per_launch"] = k_flops / len(per_linear)
    if len(per_linear) == 1:
        roof["timing"] = per_linear[0]["timing"]
    else:
        roof["timing"] = ("mean over the block's linears, one launch of each per step; "
                          "achieved = their summed work / their summed mean launch time")
        roof["per_linear"] = per_linear
    res = {
        "value": round(gbs, 2) if hbm_bound else round(tflops, 3),
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "steps": steps, "ms_per_step": round(ms_step, 5), "warmup_steps_run": warm_steps,
        "config": {"workload": name, "layers": [f"{b['spec'].n}x{b['spec'].k}" for b in built],
                   "bpw": spec0.bpw, "m": spec0.m, "x_dtype": spec0.x_dtype,
                   "distinct_layer_copies": per_graph, "row_scales": bool(row_scale),
                   "step": "full layer forward of every linear: input RHT + fused decode-matmul + output RHT"},
        "tflops": round(tflops, 4), "compressed_gbs": round(gbs, 2),
        "eager_ms_per_step": round(eager_ms_step, 5), "wall_s_timed": round(wall, 4),
        "roofline": roof,
    }
    if one_kernel:
        res["single_call_us"], res["single_call_host_us"] = single_call_us(built[0])
        res["single_call_note"] = ("medians of isolated calls (host waits for each), each on a different layer "
                                   "copy: single_call_us is the call's own GPU time (events enqueued behind a "
                                   "spin kernel), single_call_host_us adds the binding and launch submission; "
                                   "the sustained rate (value) is over back-to-back launches")
    return res, built


def single_call_us(b, calls=200):
    """One isolated whole-layer call, each on another layer copy, the host
    synchronised before and after each: (GPU, host) medians in microseconds.
    GPU: a spin kernel (~100 us) holds the stream while the host enqueues
    event, call, event, so the events bracket the call alone, started on an
    idle GPU with nothing else in flight. Host: the events recorded around
    the Python call on an idle GPU, so the binding's marshalling and the
    launch submission are inside."""
    import statistics
    import torch
    from dequant_e8_codebook_amd import glq
    gpu, host = [], []
    Ls = b["layers"]
    for i in range(calls):
        L = Ls[i % len(Ls)]
        e0, e1 = _event(), _event()
        torch.cuda.synchronize()
        torch.cuda._sleep(200000)
        e0.record()
        glq.fused_linear(L, b["x"], b["y"], b["ws"])
        e1.record()
        torch.cuda.synchronize()
        gpu.append(e0.elapsed_time(e1) * 1e3)
        e0, e1 = _event(), _event()
        e0.record()
        glq.fused_linear(L, b["x"], b["y"], b["ws"])
        e1.record()
        torch.cuda.synchronize()
        host.append(e0.elapsed_time(e1) * 1e3)
    return round(statistics.median(gpu), 3), round(statistics.median(host), 3)


def bf16_matmul_step_ms(built, reps=20):
    """Uncompressed comparison: torch.matmul (hipBLASLt) on dense bf16 weights
    of the same shapes, one product per linear, summed (ms per step)."""
    import torch
    tot = 0.0
    per = []
    for b in built:
        spec = b["spec"]
        x = torch.randn(spec.m, spec.k, device="cuda:0").to(torch.bfloat16)
        wt = torch.randn(spec.k, spec.n, device="cuda:0").to(torch.bfloat16)
        for _ in range(3):
            torch.matmul(x, wt)
        torch.cuda.synchronize()
        e0, e1 = _event(), _event()
        e0.record()
        for _ in range(reps):
            torch.matmul(x, wt)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tot += ms
        per.append({"layer": f"{spec.n}x{spec.k}", "ms": round(ms, 4)})
        del x, wt
    return round(tot, 4), per


def cpu_baseline_layer(built, budget_s):
    """The oracle's float64 layer forward on the host, on a bounded sample
    (a few activation rows of the first linear), in compressed bytes per second."""
    import numpy as np
    from oracle import glq as og
    b = built[0]
    spec = b["spec"]
    i1, i2, s, sn, sk = b["idx"]
    x = b["xnp"]
    rows = min(spec.m, 4)
    n_done = 0
    t0 = time.perf_counter()
    while True:
        ref = og.layer_reference(x[:rows], i1, i2, spec.bpw, s, sn, sk)
        n_done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    comp = i1.size * 2 + (0 if i2 is None else i2.size * i2.itemsize) + (4 * np.size(s) if np.ndim(s) else 0)
    return {"value": round(n_done * comp / dt / 1e9, 5), "unit": "GB/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{n_done} layer forwards of {spec.n}x{spec.k} at {spec.bpw} bpw, {rows} activation row(s) "
                      f"each (decode + float64 RHTs + matmul), {dt:.1f} s; compressed bytes per second",
            "accuracy": [_accuracy(og, b, ref)]}


def cpu_baseline_block(built, rows):
    """The oracle's float64 forward of every linear of the workload on the
    host, on the first `rows` activation rows of each (decode, both RHTs and
    the matrix product all inside the timed region), in TFLOP/s of 2 rows n k."""
    from oracle import glq as og
    fl, t = 0.0, 0.0
    acc = []
    for b in built:
        spec = b["spec"]
        i1, i2, s, sn, sk = b["idx"]
        x = b["xnp"][:rows]
        t0 = time.perf_counter()
        ref = og.layer_reference(x, i1, i2, spec.bpw, s, sn, sk)
        t += time.perf_counter() - t0
        fl += 2.0 * len(x) * spec.n * spec.k
        acc.append(_accuracy(og, b, ref))
    names = ", ".join(f"{b['spec'].n}x{b['spec'].k}" for b in built)
    return {"value": round(fl / t / 1e12, 6), "unit": "TFLOP/s", "cores": _blas_threads(), "kind": "oracle",
            "sample": f"{rows} of {built[0]['spec'].m} activation rows through each linear ({names}) at "
                      f"{built[0]['spec'].bpw} bpw: decode + float64 RHTs + matmul, {t:.1f} s",
            "cpu_model": _cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0)), "accuracy": acc}


def _accuracy(og, b, ref):
    """The timed runs' own output (y of the last replay; every copy of a
    linear holds the same indices) against the oracle on the sampled rows:
    max|y - y_ref| / max|y_ref| and its row-normalised maximum."""
    y = b["y"][:len(ref)].float().cpu().numpy()
    return {"layer": f"{b['spec'].n}x{b['spec'].k}", "rows": len(ref),
            "rel_max": float(f"{og.relative_error(y, ref):.3e}"),
            "row_rel_max": float(f"{og.row_relative_error(y, ref):.3e}"), "tolerance": 1e-2}


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return 1


METRIC = "fused E8-decode linear TFLOP/s + compressed-weight GB/s (% roofline), 1 MI355X"


def run_suite(args):
    """The default bench line: the DiT block (the largest workload) as the
    headline, timed for exactly --steps steps; the batch-1, batch-16 and
    prefill workloads beside it, each with its own dominant-kernel roofline."""
    import torch
    torch.cuda.set_device(0)
    head, built = time_workload("dit_block", args.steps, args.warmup, 10, args.row_scale, args.kernel_launches,
                                warm_s=args.warm_seconds)
    mm_ms, mm_per = bf16_matmul_step_ms(built)
    out = {"metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
           "steps": head["steps"], "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic", "config": head["config"]}
    out.update({k: v for k, v in head.items() if k not in out and k != "config"})
    out["vs_uncompressed_bf16"] = {
        "bf16_matmul_ms_per_step": mm_ms, "decode_gemm_ms_per_step": head["ms_per_step"],
        "ratio": round(head["ms_per_step"] / mm_ms, 4), "per_linear": mm_per,
        "note": "torch.matmul (hipBLASLt) on dense bf16 weights of the same six shapes; the step "
                "includes both row transforms of every linear"}
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline_block(built, args.cpu_rows)
    del built
    torch.cuda.empty_cache()
    others = {}
    for name, steps in (("gemv", 2048), ("batch16", 1024), ("prefill_up", 100)):
        copies = 128 if name in ("gemv", "batch16") else 24
        r, b = time_workload(name, steps, 16, copies, args.row_scale, args.kernel_launches, warm_s=args.warm_seconds)
        if name == "gemv" and not args.no_cpu_baseline:
            r["cpu_baseline"] = cpu_baseline_layer(b, 3.0)
        others[name] = r
        del b
        torch.cuda.empty_cache()
    out["workloads"] = others
    return out


def run_one(args):
    """One workload as the bench line (profiling runs and the other configurations)."""
    import torch
    torch.cuda.set_device(0)
    copies = args.layers if len(__import__("workloads").layer_specs(args.workload)) == 1 else max(1, args.layers // 16)
    res, built = time_workload(args.workload, args.steps, args.warmup, copies, args.row_scale, args.kernel_launches,
                               warm_s=args.warm_seconds)
    out = {"metric": METRIC, "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": res["steps"],
           "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32" if built[0]["spec"].x_dtype == "f32" else "bf16",
           "data": "synthetic", "config": res["config"]}
    out.update({k: v for k, v in res.items() if k not in out})
    if args.no_cpu_baseline:
        out["cpu_baseline"] = None
    elif len(built) > 1 or built[0]["spec"].m > 16:
        out["cpu_baseline"] = cpu_baseline_block(built, min(args.cpu_rows, built[0]["spec"].m))
    else:
        out["cpu_baseline"] = cpu_baseline_layer(built, args.cpu_budget)
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ profiling helpers

def achievable_peaks():
    """Measured ceilings on this GPU, for context beside the published peaks:
    a stream read of 2 GiB (torch sum of float32), a 2 GiB device copy
    (bytes read plus written) and bf16 torch.matmul
    (hipBLASLt) on uncompressed weights of the workload shapes."""
    import torch
    dev = "cuda:0"
    out = {}
    a = torch.ones(512 << 20, dtype=torch.float32, device=dev)      # 2 GiB
    for _ in range(3):
        a.sum()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        a.sum()
    e1.record()
    torch.cuda.synchronize()
    out["stream_read_gbs"] = round(a.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    out["copy_read_plus_write_gbs"] = round(2 * a.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a, b
    shapes = [(2048, 16384, 4096), (4096, 3072, 3072), (4096, 12288, 3072), (4096, 3072, 12288)]
    mm = {}
    for m, n, k in shapes:
        x = torch.randn(m, k, device=dev).to(torch.bfloat16)
        w = torch.randn(n, k, device=dev).to(torch.bfloat16)
        wt = w.t().contiguous()
        for _ in range(3):
            torch.matmul(x, wt)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            torch.matmul(x, wt)
        e1.record()
        torch.cuda.synchronize()
        mm[f"{m}x{n}x{k}"] = round(2.0 * m * n * k * 20 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    out["bf16_matmul_tflops"] = mm
    print(json.dumps(out))


def encoder_bench(workload, budget_s):
    """The library's CPU encoders on one layer of the workload: nearest
    rounding (glq_encode_ref) against LDLQ error feedback (glq_encode_ldlq)
    with a synthetic Hessian of 2k calibration rows; proxy loss
    tr((X^ - X) H~ (X^ - X)^T) of both (computed here in float64 from the
    indices); and the oracle's LDLQ encoder timed on a bounded sample of rows
    (the first rows of W with the first entries of sign_n)."""
    import numpy as np
    import workloads as wl
    from dequant_e8_codebook_amd import glq
    from oracle import glq as og, ldlq as ol, rht
    spec = wl.layer_specs(workload)[0]
    w = wl.weights(spec).astype(np.float32)
    sn, sk = wl.sign_n(spec), wl.sign_k(spec)
    h = ol.hessian_from_inputs(wl.calibration(spec, 2 * spec.k))
    t0 = time.perf_counter()
    p1, p2, ps = glq.encode_ref(w, spec.bpw, sn, sk)
    t_plain = time.perf_counter() - t0
    t0 = time.perf_counter()
    l1, l2, ls = glq.encode_ldlq(w, spec.bpw, sn, sk, h)
    t_ldlq = time.perf_counter() - t0
    x = rht.rotate_weights(w.astype(np.float64), sn, sk) / np.float64(ps)
    ht = ol.damp_hessian(ol.rotate_hessian(h, sk))
    loss_plain = ol.proxy_loss(og.decode_values(p1, p2, spec.bpw), x, ht)
    loss_ldlq = ol.proxy_loss(og.decode_values(l1, l2, spec.bpw), x, ht)
    # oracle: row samples of 16, 64, 256 ... rows while they stay within the budget
    rows_s, t_or, rows = 0, 0.0, 16
    while rows <= spec.n:
        t0 = time.perf_counter()
        ol.encode_ldlq(w[:rows].astype(np.float64), spec.bpw, sn[:rows], sk, h)
        t_or, rows_s = time.perf_counter() - t0, rows
        if 4 * t_or > budget_s:
            break
        rows *= 4
    out = {"workload": workload, "n": spec.n, "k": spec.k, "bpw": spec.bpw, "threads": os.cpu_count(),
           "cpp_plain_s": round(t_plain, 3), "cpp_ldlq_s": round(t_ldlq, 3),
           "cpp_ldlq_weights_per_s": round(spec.n * spec.k / t_ldlq, 1),
           "proxy_loss_plain": loss_plain, "proxy_loss_ldlq": loss_ldlq,
           "loss_ratio": round(loss_ldlq / loss_plain, 4),
           "indices_changed_frac": round(float((l1 != p1).mean()), 4),
           "oracle_ldlq_sample": f"{rows_s} rows x {spec.k}", "oracle_ldlq_s": round(t_or, 3),
           "oracle_ldlq_weights_per_s": round(rows_s * spec.k / t_or, 1)}
    print(json.dumps(out))


def ep_step_for_rate(w, sn, sk, target_bpp, lane_groups):
    """Quantiser step whose encoding lands nearest the target actual_bpp
    (bisection on log(step); the rate falls as the step grows)."""
    import numpy as np
    from dequant_e8_codebook_amd import glq
    n, k = w.shape
    lo, hi = np.log(0.02), np.log(2.0)
    best = None
    for _ in range(14):
        mid = 0.5 * (lo + hi)
        try:
            h = glq.ep_encode(w, sn, sk, float(np.exp(mid)), lane_groups)
        except glq.GlqError:
            lo = mid
            continue
        bpp = ep_actual_bpp(h)
        if best is None or abs(bpp - target_bpp) < abs(best[1] - target_bpp):
            best = (h, bpp)
        if bpp > target_bpp:
            lo = mid
        else:
            hi = mid
    return best


def ep_actual_bpp(h):
    """Every stored byte of an entropy-coded layer per weight, times 8."""
    b = (2 * len(h.words) + 4 * h.states.size + 4 * len(h.offsets) + 40 + 2 * sum(h.model.nsym)
         + 4 * h.n + 4 + (h.n + 7) // 8 + (h.k + 7) // 8)
    return 8.0 * b / (h.n * h.k)


def ep_decode_bench(workload, target_bpp, lane_groups, launches):
    """Fused symbol decode + weight reconstruction of the entropy-coded format
    on the workload's layer shapes: step chosen for the target rate, kernel
    time from HIP events around back-to-back launches on one stream."""
    import numpy as np
    import torch
    import workloads as wl
    from dequant_e8_codebook_amd import glq
    res = []
    seen = set()
    for spec in wl.layer_specs(workload):
        if (spec.n, spec.k) in seen:
            continue
        seen.add((spec.n, spec.k))
        w = wl.weights(spec).astype(np.float32)
        sn, sk = wl.sign_n(spec), wl.sign_k(spec)
        h, bpp = ep_step_for_rate(w, sn, sk, target_bpp, lane_groups)
        L = glq.EpLayer.from_host(h)
        out = torch.empty((spec.n, spec.k), device="cuda", dtype=torch.bfloat16)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            for _ in range(5):
                glq.ep_decode_weights(L, out, stream=s)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            for _ in range(launches):
                glq.ep_decode_weights(L, out, stream=s)
            e1.record(s)
            s.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        stored = bpp * spec.n * spec.k / 8.0
        moved = stored + 2.0 * spec.n * spec.k
        # the whole layer y = U^T W^ (V x) at the workload's batch (bf16 in/out)
        L.sign_k, L.sign_n = (torch.from_numpy(np.ascontiguousarray(a, np.int8)).to("cuda") for a in (sk, sn))
        L.__dict__.pop("_st", None)
        x = torch.randn(spec.m, spec.k, device="cuda").to(torch.bfloat16)
        y = torch.empty(spec.m, spec.n, device="cuda", dtype=torch.bfloat16)
        ws = torch.zeros(glq.ep_workspace_bytes(L, spec.m), device="cuda", dtype=torch.uint8)
        reps = max(3, min(50, launches // 4))
        with torch.cuda.stream(s):
            for _ in range(3):
                glq.ep_fused_linear(L, x, y, ws, stream=s)
            e0.record(s)
            for _ in range(reps):
                glq.ep_fused_linear(L, x, y, ws, stream=s)
            e1.record(s)
            s.synchronize()
        lus = e0.elapsed_time(e1) * 1e3 / reps
        res.append({"shape": f"{spec.n}x{spec.k}", "step": h.step, "actual_bpp": round(bpp, 4),
                    "nblocks": h.nblocks, "kernel_us": round(us, 2),
                    "weights_per_s": round(spec.n * spec.k / (us * 1e-6), 1),
                    "stored_gbs": round(stored / (us * 1e-6) / 1e9, 1),
                    "hbm_gbs": round(moved / (us * 1e-6) / 1e9, 1), "hbm_frac": round(moved / (us * 1e-6) / 8e12, 4),
                    "layer_m": spec.m, "layer_us": round(lus, 2),
                    "layer_tflops": round(2.0 * spec.m * spec.n * spec.k / (lus * 1e-6) / 1e12, 1)})
    print(json.dumps({"mode": "ep_decode", "workload": workload, "target_bpp": target_bpp,
                      "lane_groups": lane_groups, "layers": res}))


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES (for counter calibration)."""
    import torch
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "launches": 5}))


def _read_counters(d):
    """{(kernel_name, counter): [values per dispatch]} from rocprofv3 counter CSVs."""
    vals = {}
    for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(p) as f:
            for row in csv.DictReader(f):
                key = (row.get("Kernel_Name", ""), row.get("Counter_Name", ""))
                try:
                    vals.setdefault(key, []).append(float(row.get("Counter_Value", "nan")))
                except ValueError:
                    pass
    return vals


def pmc_summary(args):
    """Write profiles/pmc_traffic_<workload>.txt from four counter runs:
    copy FETCH, copy WRITE, bench FETCH, bench WRITE (directories given)."""
    cf, cw, bf, bw = args.pmc_summary
    kernel_pat = args.pmc_kernel
    def pick(d, counter, pat):
        v = _read_counters(d)
        sel = [x for (k, c), xs in v.items() if c == counter and pat in k for x in xs]
        if not sel:
            raise SystemExit(f"no {counter} values for kernels matching {pat!r} in {d}")
        return sel
    copy_kib = COPY_BYTES / 1024.0
    cfetch = pick(cf, "FETCH_SIZE", args.copy_kernel)
    cwrite = pick(cw, "WRITE_SIZE", args.copy_kernel)
    f_fac = copy_kib / max(cfetch)          # the largest dispatch is the full copy
    w_fac = copy_kib / max(cwrite)
    kf = pick(bf, "FETCH_SIZE", kernel_pat)
    kw = pick(bw, "WRITE_SIZE", kernel_pat)
    import statistics
    mf, mw = statistics.median(kf), statistics.median(kw)
    hbm = (mf * f_fac + mw * w_fac) * 1024.0
    os.makedirs(PROFILE_DIR, exist_ok=True)
    with open(_profile_path(args.workload), "w") as f:
        f.write("# HBM traffic of the dominant kernel from rocprofv3 counters (KiB per dispatch),\n"
                "# scaled by copy_bytes / counter reading of a plain device copy of known size.\n")
        f.write(f"# commands: {args.pmc_commands}\n" if args.pmc_commands else "")
        f.write(f"workload: {args.workload}\nkernel: {args.pmc_kernel_label}\n")
        f.write(f"kernel_source_sha256_16: {kernel_source_hash()}\n")
        f.write(f"dispatches_fetch: {len(kf)}\ndispatches_write: {len(kw)}\n")
        f.write(f"fetch_kib_per_dispatch_median: {mf:.1f}\nwrite_kib_per_dispatch_median: {mw:.1f}\n")
        f.write(f"copy_fetch_factor: {f_fac:.4f}\ncopy_write_factor: {w_fac:.4f}\n")
        f.write(f"hbm_bytes_per_dispatch: {hbm:.0f}\n")
    print(open(_profile_path(args.workload)).read())


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--warm-seconds", type=float, default=0.1,
                    help="untimed graph replays for this long after the warm-up steps (0: none)")
    ap.add_argument("--workload", default="suite", choices=["suite", "small", "gemv", "batch16", "prefill_up",
                                                            "dit_block"],
                    help="suite (default): the DiT block as the headline, the other workloads beside it")
    ap.add_argument("--layers", type=int, default=128, help="distinct copies of the index planes rotated through")
    ap.add_argument("--kernel-launches", type=int, default=1024)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU work (small-batch runs)")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="activation rows per linear in the oracle's timed sample (prefill / DiT runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--achievable", action="store_true", help="measure stream-read and bf16 matmul ceilings")
    ap.add_argument("--row-scale", action="store_true", help="encode with per-row scales")
    ap.add_argument("--encoder", action="store_true", help="time the CPU encoders (plain and LDLQ)")
    ap.add_argument("--ep-decode", type=float, default=0.0, metavar="BPP",
                    help="time the entropy-coded format's decode at this storage rate")
    ap.add_argument("--ep-lane-groups", type=int, default=32)
    ap.add_argument("--pmc-summary", nargs=4, metavar=("COPY_FETCH", "COPY_WRITE", "BENCH_FETCH", "BENCH_WRITE"))
    ap.add_argument("--pmc-kernel", default="gemv_bf16")
    ap.add_argument("--pmc-kernel-label", default="gemv_bf16<2>")
    ap.add_argument("--copy-kernel", default="")
    ap.add_argument("--pmc-commands", default="")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(args)
        return 0
    if args.steps < 1 or args.warmup < 0 or args.warm_seconds < 0:
        print("bench.py: --steps must be at least 1, --warmup and --warm-seconds at least 0", file=sys.stderr)
        return 2
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(rows of x or output features would shard across GPUs with no exchange).",
              file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.achievable:
        achievable_peaks()
        return 0
    if args.encoder:
        encoder_bench("gemv" if args.workload == "suite" else args.workload, args.cpu_budget)
        return 0
    if args.ep_decode > 0:
        ep_decode_bench("gemv" if args.workload == "suite" else args.workload, args.ep_decode,
                        args.ep_lane_groups, args.kernel_launches)
        return 0
    out = run_suite(args) if args.workload == "suite" else run_one(args)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
