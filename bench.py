"""Benchmark of the fused E8-decode linear layer on one MI355X.

Default workload: the 4096x4096, 2 bpw, batch-1 layer (bf16 activations with
8 outlier channels at 20x, Student-t(5) weights of std 0.02). One step is one
full layer forward y = U^T (s W^) (V x): input RHT, fused decode-GEMV, output
RHT, all in libglq.so. Steps rotate through --layers distinct copies of the
layer's index planes (128 x 4 MiB = 512 MiB, twice the 256 MB Infinity
Cache), so each step streams its compressed weights from HBM.

value = compressed-weight bytes moved per second (GB/s) over the timed steps,
which replay a HIP graph of one step per layer copy (no host launch cost).
roofline = the dominant kernel of the step, timed with HIP events on its
launch stream (graph replays): compressed bytes per launch / mean launch
duration against 8 TB/s HBM (small batch), or 2 M N K per launch / duration
against 2.5 PFLOP/s bf16 MFMA (prefill). At batch 1 the whole layer is one
kernel, so its launches are the timed steps. traffic = HBM bytes per launch from
rocprofv3 FETCH_SIZE + WRITE_SIZE counters (profiles/), scaled by what the
counters read for a plain copy of known size; null if the kernel source has
changed since those counters were taken.
cpu_baseline = the oracle's layer forward on the host (float64), on a bounded
sample of layer forwards of the same workload.

Other modes (profiling helpers, not bench lines):
  --workload batch16|prefill_up|dit_block|small   time another workload
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
    return f"gemv_bf16<{spec.bpw}>" if spec.m <= 16 else f"gemm_bf16<{spec.bpw}>"


def run_bench(args):
    import numpy as np
    import torch
    from dequant_e8_codebook_amd import glq
    from workloads import layer_specs

    dev = "cuda:0"
    torch.cuda.set_device(0)
    specs = layer_specs(args.workload)
    per_step_layers = len(specs)
    n_rot = args.layers if per_step_layers == 1 else max(1, args.layers // 16)
    built = build_layers(args.workload, n_rot, dev, row_scale=args.row_scale)

    def layer_bytes(L):
        # index planes, plus the row-scale vector when there is one
        return (L.idx1.numel() * 2 + (0 if L.idx2 is None else L.idx2.numel() * L.idx2.element_size())
                + (0 if L.row_scale is None else L.row_scale.numel() * 4))
    comp_bytes = sum(layer_bytes(b["layers"][0]) for b in built)
    flops = sum(2.0 * b["spec"].m * b["spec"].n * b["spec"].k for b in built)

    def step(i):
        for b in built:
            L = b["layers"][i % len(b["layers"])]
            glq.fused_linear(L, b["x"], b["y"], b["ws"])

    # The timed steps replay a HIP graph holding one step per distinct layer
    # copy (captured through torch's CUDA-graph API, on its capture stream), so
    # the measurement sees GPU time, not Python/ctypes launch overhead.
    per_graph = len(built[0]["layers"])
    for i in range(max(args.warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(per_graph):
            step(i)
    replays = max(1, args.steps // per_graph)
    steps_timed = replays * per_graph
    for _ in range(max(1, args.warmup // per_graph)):
        graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(replays):
        graph.replay()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1)
    ms_step = ms / steps_timed
    gbs = comp_bytes * steps_timed / (ms * 1e-3) / 1e9
    tflops = flops * steps_timed / (ms * 1e-3) / 1e12

    # eager (no graph) rate of the same steps, for reference
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    n_eager = min(steps_timed, 256)
    e0.record()
    for i in range(n_eager):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_ms_step = e0.elapsed_time(e1) / n_eager

    # dominant kernel alone (x pre-rotated, output left rotated): a graph of
    # one launch per layer copy, replayed; mean launch = time / launches
    b0 = built[0]
    spec0 = b0["spec"]
    xr = b0["x"].clone()
    sk = b0["layers"][0].sign_k
    glq.rht_apply(b0["x"], xr, sk, False)
    z = torch.empty_like(b0["y"])
    flags = glq.FLAG_NO_INPUT_RHT | glq.FLAG_NO_OUTPUT_RHT
    for L in b0["layers"]:
        glq.fused_linear(L, xr, z, b0["ws"], flags)
    torch.cuda.synchronize()
    kgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(kgraph):
        for L in b0["layers"]:
            glq.fused_linear(L, xr, z, b0["ws"], flags)
    krep = max(1, args.kernel_launches // len(b0["layers"]))

    def graph_seconds(g):
        g.replay()
        torch.cuda.synchronize()
        k0 = torch.cuda.Event(enable_timing=True)
        k1 = torch.cuda.Event(enable_timing=True)
        k0.record()
        for _ in range(krep):
            g.replay()
        k1.record()
        torch.cuda.synchronize()
        return k0.elapsed_time(k1) * 1e-3

    core_mean = graph_seconds(kgraph) / (krep * len(b0["layers"]))
    tiled = operand_layout(spec0)
    if tiled:
        # the step's GEMV reads x~ in the operand layout its input transform
        # writes, which a pre-rotated x cannot give: time input transform +
        # GEMV and subtract the row-major transform of the same rows (the
        # same kernel writing row-major, without the row sums)
        zt = torch.empty_like(b0["y"])
        for L in b0["layers"]:
            glq.fused_linear(L, b0["x"], zt, b0["ws"], glq.FLAG_NO_OUTPUT_RHT)
        ga = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ga):
            for L in b0["layers"]:
                glq.fused_linear(L, b0["x"], zt, b0["ws"], glq.FLAG_NO_OUTPUT_RHT)
        gb = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gb):
            for L in b0["layers"]:
                glq.rht_apply(b0["x"], xr, L.sign_k, False)
        core_mean = (graph_seconds(ga) - graph_seconds(gb)) / (krep * len(b0["layers"]))
    # the whole-layer kernel is the step itself: its mean launch is the step time
    k_mean = ms_step * 1e-3 if single_launch(spec0) and len(built) == 1 else core_mean
    # rotated-basis launches of 3/4 bpw also run a small row-sum kernel
    L0 = b0["layers"][0]
    k_bytes = layer_bytes(L0)
    k_flops = 2.0 * spec0.m * spec0.n * spec0.k
    dom = dominant_kernel(spec0)
    hbm_bound = spec0.m <= 16
    if hbm_bound:
        achieved = k_bytes / k_mean / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 2), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4))
    else:
        achieved = k_flops / k_mean / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / MFMA_BF16_PEAK_TFLOPS, 4))
    traffic = read_traffic(args.workload, dom)
    roof["traffic"] = traffic
    roof["kernel"] = dom
    roof["kernel_mean_us"] = round(k_mean * 1e6, 3)
    if single_launch(spec0) and len(built) == 1:
        roof["timing"] = (f"HIP events around {replays} replays of a graph of {per_graph} whole-layer launches "
                          "(the timed steps)")
        roof["matmul_core"] = {"kernel": f"gemv_bf16<{spec0.bpw}>", "mean_us": round(core_mean * 1e6, 3),
                               "achieved_gbs": round(k_bytes / core_mean / 1e9, 2),
                               "note": "decode-GEMV alone (x already rotated, z left rotated), as in the multi-kernel path"}
    elif tiled:
        roof["timing"] = (f"HIP events around {krep} replays of a graph of {len(b0['layers'])} (input transform into "
                          "the operand layout + GEMV) pairs, minus the same for the row-major input transform alone")
    else:
        roof["timing"] = f"HIP events around {krep} replays of a graph of {len(b0['layers'])} launches"
    roof["algorithmic_bytes_per_launch"] = k_bytes
    roof["algorithmic_flops_per_launch"] = k_flops

    out = {
        "metric": "fused E8-decode linear TFLOP/s + compressed-weight GB/s (% roofline), 1 MI355X",
        "value": round(gbs, 2) if hbm_bound else round(tflops, 3),
        "unit": "GB/s" if hbm_bound else "TFLOP/s",
        "n_gpus": 1, "steps": steps_timed, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload,
                   "layers": [f"{b['spec'].n}x{b['spec'].k}" for b in built],
                   "bpw": spec0.bpw, "m": spec0.m, "x_dtype": spec0.x_dtype,
                   "distinct_layer_copies": len(b0["layers"]), "row_scales": bool(args.row_scale),
                   "step": "full layer forward: input RHT + fused decode-matmul + output RHT"},
        "tflops": round(tflops, 4), "compressed_gbs": round(gbs, 2),
        "eager_ms_per_step": round(eager_ms_step, 5),
        "wall_s_timed": round(wall, 4),
        "roofline": roof,
    }
    return out, built


def cpu_baseline(built, budget_s):
    """The oracle's float64 layer forward on the host, timed on a bounded sample."""
    import numpy as np
    from oracle import glq as og
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = 1
    b = built[0]
    spec = b["spec"]
    i1, i2, s, sn, sk = b["idx"]
    x = b["xnp"]
    rows = min(spec.m, 4)
    n_done = 0
    t0 = time.perf_counter()
    while True:
        og.layer_reference(x[:rows], i1, i2, spec.bpw, s, sn, sk)
        n_done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    comp = i1.size * 2 + (0 if i2 is None else i2.size * i2.itemsize) + (4 * np.size(s) if np.ndim(s) else 0)
    gbs = n_done * comp / dt / 1e9
    # the oracle's decode alone (float32 weights from the indices), a quarter of the budget
    n_dec = 0
    t1 = time.perf_counter()
    while True:
        og.decode_f32(i1, i2, spec.bpw, s)
        n_dec += 1
        if time.perf_counter() - t1 >= budget_s / 4:
            break
    dd = time.perf_counter() - t1
    return {"value": round(gbs, 5), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_done} layer forwards of {spec.n}x{spec.k} at {spec.bpw} bpw, {rows} activation row(s) "
                      f"each (decode + float64 RHTs + matmul), {dt:.1f} s; compressed bytes per second",
            "decode_only": {"value": round(n_dec * comp / dd / 1e9, 5), "unit": "GB/s",
                            "sample": f"{n_dec} float32 decodes of the layer, {dd:.1f} s"},
            "cpu_model": _cpu_model(), "affinity_cpus": len(os.sched_getaffinity(0))}


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
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--workload", default="gemv", choices=["small", "gemv", "batch16", "prefill_up", "dit_block"])
    ap.add_argument("--layers", type=int, default=128, help="distinct copies of the index planes rotated through")
    ap.add_argument("--kernel-launches", type=int, default=1024)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle CPU work")
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
        encoder_bench(args.workload, args.cpu_budget)
        return 0
    if args.ep_decode > 0:
        ep_decode_bench(args.workload, args.ep_decode, args.ep_lane_groups, args.kernel_launches)
        return 0
    out, built = run_bench(args)
    out["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(built, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
