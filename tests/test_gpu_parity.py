"""GPU parity: the HIP path (through the C ABI) against the oracle.

Bars: decoded weights bit-exact (compared as integer bit patterns); RHT within
float32 rounding; layer outputs within max|y - y_ref| / max|y_ref| <= 1e-5 on
the float32 path and <= 1e-2 on the bf16 matrix-core path.

Inputs: the five layer workloads of `workloads` (seeded). At reduced sizes the
indices come from the oracle encoder applied to the workload's weight
distribution; at full sizes the indices are seeded uniform draws (any index
array is a valid compressed layer, and running the nearest-neighbour encoder
on 10^7 groups does not fit a test), and whole output rows are checked for a
sample of rows.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
from oracle import glq as og, rht  # noqa: E402
import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 1e-2


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dequant_e8_codebook_amd import glq
    return glq


@pytest.fixture(scope="module")
def cb(G):
    return G.device_codebook("cuda")


def _t(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to("cuda") if dtype is None else t.to(device="cuda", dtype=dtype)


def _bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def _random_layer(n, k, bpw, seed):
    g = k // 8
    i1 = workloads.random_indices((n, g), seed)
    i2 = None
    if bpw == 3:
        i2 = workloads.random_indices((n, g), seed + 1, 256, np.uint8)
    elif bpw == 4:
        i2 = workloads.random_indices((n, g), seed + 1)
    return i1, i2


def _run_linear(G, cb, i1, i2, s, sn, sk, x, x_dt, y_dt, flags=0):
    L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb)
    m = x.shape[0]
    xt = _t(x.astype(np.float32), torch.float32 if x_dt == "f32" else torch.bfloat16)
    # NaN-filled so that an output element no kernel writes fails the finiteness checks
    y = torch.full((m, L.n), float("nan"), device="cuda", dtype=torch.float32 if y_dt == "f32" else torch.bfloat16)
    ws = torch.zeros(max(G.workspace_bytes(L, max(m, 1)), 256), device="cuda", dtype=torch.uint8)
    G.fused_linear(L, xt, y, ws, flags)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


# --------------------------------------------------------------- decode ----

@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_decode_every_index_bitexact(G, cb, bpw, out):
    # all 65536 stage-1 indices (and random residual indices) in one call
    n, k = 4096, 128
    i1 = np.arange(65536, dtype=np.uint16).reshape(n, k // 8)
    _, i2 = _random_layer(n, k, bpw, 90 + bpw)
    s = np.float32(0.0123)
    L = G.Layer.from_numpy(i1, i2, s, None, None, cb)
    w = torch.empty((n, k), device="cuda", dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    G.decode_weights(L, w)
    torch.cuda.synchronize()
    ref = og.decode_bf16_bits(i1, i2, bpw, s) if out == "bf16" else og.decode_f32(i1, i2, bpw, s).view(np.uint32)
    assert np.array_equal(_bits(w), ref)


@pytest.mark.parametrize("n,k,bpw", [(1, 8, 2), (33, 24, 3), (300, 4104, 4), (17, 520, 2)])
def test_decode_ragged_shapes(G, cb, n, k, bpw):
    i1, i2 = _random_layer(n, k, bpw, 7 * n + k)
    s = np.float32(3.75e-3)
    L = G.Layer.from_numpy(i1, i2, s, None, None, cb)
    for dt in (torch.bfloat16, torch.float32):
        w = torch.empty((n, k), device="cuda", dtype=dt)
        G.decode_weights(L, w)
        torch.cuda.synchronize()
        ref = og.decode_bf16_bits(i1, i2, bpw, s) if dt == torch.bfloat16 else og.decode_f32(i1, i2, bpw, s).view(np.uint32)
        assert np.array_equal(_bits(w), ref)


def test_decode_oracle_encoded_layer(G, cb):
    spec = workloads.layer_specs("small")[0]
    w = workloads.weights(spec)
    sn, sk = workloads.sign_n(spec), workloads.sign_k(spec)
    for bpw in (2, 3, 4):
        i1, i2, s = og.encode(w, bpw, sn, sk)
        L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb)
        out = torch.empty((spec.n, spec.k), device="cuda", dtype=torch.bfloat16)
        G.decode_weights(L, out)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(out), og.decode_bf16_bits(i1, i2, bpw, s))


# ------------------------------------------------------------------ RHT ----

@pytest.mark.parametrize("n", [8, 12, 7, 256, 3072, 4096, 12288, 16384, 130])
@pytest.mark.parametrize("rows", [1, 5])
@pytest.mark.parametrize("transpose", [0, 1])
def test_rht_f32(G, n, rows, transpose):
    rng = np.random.default_rng(n * 7 + rows)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    sig = workloads.signs(n, n + 1)
    out = torch.empty((rows, n), device="cuda", dtype=torch.float32)
    G.rht_apply(_t(x), out, _t(sig), bool(transpose))
    torch.cuda.synchronize()
    ref = (rht.rht_transpose if transpose else rht.rht_forward)(x.astype(np.float64), sig)
    got = out.cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref)) * np.log2(max(rht.block_size(n), 2))


@pytest.mark.parametrize("n", [1024, 2048, 8192])
@pytest.mark.parametrize("rows", [1, 16, 64])
@pytest.mark.parametrize("transpose", [0, 1])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rht_few_rows_whole_block(G, n, rows, transpose, dt):
    # a few rows that are one block filling 1024 threads with 1, 2 or 8
    # elements a thread: the register kernel's full-block variant
    x = np.random.default_rng(n + rows + 5 * transpose).standard_normal((rows, n)).astype(np.float32)
    if dt == "bf16":
        x = workloads.bf16_round_trip(x)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    sig = workloads.signs(n, n + 11)
    out = torch.empty((rows, n), device="cuda", dtype=tdt)
    G.rht_apply(_t(x, tdt), out, _t(sig), bool(transpose))
    torch.cuda.synchronize()
    ref = (rht.rht_transpose if transpose else rht.rht_forward)(x.astype(np.float64), sig)
    got = out.float().cpu().numpy()
    if dt == "f32":
        assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref)) * np.log2(n)
    else:
        assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-3)) <= 2.0 ** -8   # one bf16 rounding


@pytest.mark.parametrize("n", [3072, 4096, 16384, 8200, 1024, 8192])
@pytest.mark.parametrize("transpose", [0, 1])
def test_rht_many_rows(G, n, transpose):
    # more rows than the few-row path takes: the block kernel (3072), the LDS
    # radix-16 kernel (8200) and the full-block register kernel on 256 .. 1024
    # threads (1024, 4096, 8192, 16384)
    rows = 96
    rng = np.random.default_rng(n + transpose)
    x = rng.standard_normal((rows, n)).astype(np.float32)
    sig = workloads.signs(n, n + 3)
    out = torch.empty((rows, n), device="cuda", dtype=torch.float32)
    G.rht_apply(_t(x), out, _t(sig), bool(transpose))
    torch.cuda.synchronize()
    ref = (rht.rht_transpose if transpose else rht.rht_forward)(x.astype(np.float64), sig)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-6 * np.max(np.abs(ref)) * np.log2(rht.block_size(n))


@pytest.mark.parametrize("n", [3072, 12288])
@pytest.mark.parametrize("transpose", [0, 1])
def test_rht_many_rows_bf16(G, n, transpose):
    # bf16 rows of several blocks (the block kernel: 3 x 1024, 3 x 4096)
    rows = 96
    x = workloads.bf16_round_trip(np.random.default_rng(n + 7 * transpose).standard_normal((rows, n)).astype(np.float32))
    sig = workloads.signs(n, n + 9)
    out = torch.empty((rows, n), device="cuda", dtype=torch.bfloat16)
    G.rht_apply(_t(x, torch.bfloat16), out, _t(sig), bool(transpose))
    torch.cuda.synchronize()
    ref = (rht.rht_transpose if transpose else rht.rht_forward)(x.astype(np.float64), sig)
    got = out.float().cpu().numpy()
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-3)) <= 2.0 ** -8   # one bf16 rounding


@pytest.mark.parametrize("n,rows", [(3072, 2600), (12288, 600), (6144, 300), (5120, 40), (15360, 70),
                                    (10240, 33), (20480, 9)])
@pytest.mark.parametrize("transpose", [0, 1])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_rht_multi_block_rows(G, n, rows, transpose, dt):
    # rows of several Hadamard blocks of 1024 (3072, 5120, 15360), 2048 (6144,
    # 10240) or 4096 (12288): one workgroup per row, one to four waves per
    # block; more rows than resident workgroups at 3072 and 12288 (the
    # grid-stride loop with the next row in flight); 20480 = 5 x 4096 needs
    # 20 waves and takes the LDS kernel
    x = np.random.default_rng(n + rows + transpose).standard_normal((rows, n)).astype(np.float32)
    if dt == "bf16":
        x = workloads.bf16_round_trip(x)
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    sig = workloads.signs(n, n + 13)
    out = torch.full((rows, n), float("nan"), device="cuda", dtype=tdt)
    G.rht_apply(_t(x, tdt), out, _t(sig), bool(transpose))
    torch.cuda.synchronize()
    ref = (rht.rht_transpose if transpose else rht.rht_forward)(x.astype(np.float64), sig)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    if dt == "f32":
        assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref)) * np.log2(rht.block_size(n))
    else:
        assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-3)) <= 2.0 ** -8   # one bf16 rounding


def test_rht_bf16_in_out(G):
    n, rows = 4096, 3
    x = workloads.bf16_round_trip(np.random.default_rng(1).standard_normal((rows, n)).astype(np.float32))
    sig = workloads.signs(n, 5)
    out = torch.empty((rows, n), device="cuda", dtype=torch.bfloat16)
    G.rht_apply(_t(x, torch.bfloat16), out, _t(sig), False)
    torch.cuda.synchronize()
    ref = rht.rht_forward(x.astype(np.float64), sig)
    got = out.float().cpu().numpy()
    assert np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-3)) <= 2.0 ** -8   # one bf16 rounding


# ------------------------------------------------------- fused linear ----

def _encoded(spec, n, k, m):
    """Reduced-size layer of the workload: weights of its distribution, oracle-encoded."""
    sub = workloads.LayerSpec(spec.name + ".reduced", n, k, spec.bpw, m, spec.w_dist, spec.x_dtype,
                              spec.y_dtype, spec.outliers and max(1, spec.outliers * k // spec.k),
                              spec.seed_base)
    w = workloads.weights(sub)
    sn, sk = workloads.sign_n(sub), workloads.sign_k(sub)
    i1, i2, s = og.encode(w, sub.bpw, sn, sk)
    x = workloads.activations(sub)
    return sub, i1, i2, s, sn, sk, x


def test_small_workload_fp32_path(G, cb):
    spec = workloads.layer_specs("small")[0]           # 256x256, 2 bpw, M=4, fp32 in/out
    w = workloads.weights(spec)
    sn, sk = workloads.sign_n(spec), workloads.sign_k(spec)
    i1, i2, s = og.encode(w, 2, sn, sk)
    x = workloads.activations(spec)
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "f32", "f32")
    ref = og.layer_reference(x, i1, i2, 2, s, sn, sk)
    assert og.relative_error(y, ref) <= TOL_F32
    # and the decoded layer approximates the original one (sanity, not parity)
    assert og.relative_error(y, x.astype(np.float64) @ w.T) < 0.5


@pytest.mark.parametrize("name,n,k,m", [
    ("gemv", 512, 1024, 1), ("batch16", 512, 512, 16), ("prefill_up", 1024, 512, 256),
    ("dit_block", 768, 768, 192)])
def test_workloads_reduced_oracle_encoded(G, cb, name, n, k, m):
    spec = workloads.layer_specs(name)[0]
    sub, i1, i2, s, sn, sk, x = _encoded(spec, n, k, m)
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, sub.x_dtype, sub.y_dtype)
    ref = og.layer_reference(x, i1, i2, sub.bpw, s, sn, sk)
    assert og.relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("m", [1, 3, 16, 17, 33, 129])
def test_fused_shapes_bf16(G, cb, bpw, m):
    # ragged n (not a multiple of 16 or 128), k not a multiple of 256
    n, k = 150, 264
    i1, i2 = _random_layer(n, k, bpw, 1000 + 10 * bpw + m)
    s = np.float32(0.02)
    sn, sk = workloads.signs(n, 11), workloads.signs(k, 12)
    x = workloads.bf16_round_trip(np.random.default_rng(m).standard_normal((m, k)).astype(np.float32))
    for y_dt in ("bf16", "f32"):
        y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "bf16", y_dt)
        ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
        assert og.relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("m,k", [(3, 256), (16, 136)])
def test_gemv_many_row_tiles(G, cb, m, k):
    # 2 bpw with more than 1024 tiles of 16 rows: four tiles per workgroup,
    # the last workgroup ragged
    n, bpw = 16400, 2
    i1, i2 = _random_layer(n, k, bpw, 4000 + m + k)
    s = np.float32(0.013)
    sn, sk = workloads.signs(n, 51), workloads.signs(k, 52)
    x = workloads.bf16_round_trip(np.random.default_rng(k).standard_normal((m, k)).astype(np.float32))
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    for y_dt in ("bf16", "f32"):
        y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "bf16", y_dt)
        assert og.relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("m,n,k", [(300, 320, 512), (257, 264, 160), (64, 512, 4160), (40, 136, 72),
                                   (512, 1024, 136), (1000, 1024, 264)])
def test_prefill_tiles(G, cb, bpw, m, n, k):
    # several 256 x 256 output tiles with ragged row and column tails, the
    # 16-byte-store epilogue (n * element size % 16 == 0) and its per-element
    # fallback, a k that is not a multiple of the 64-input k-step, and 8 and
    # 16 tiles (every XCD dealt whole tiles), all rows checked
    i1, i2 = _random_layer(n, k, bpw, 3000 + m + n + k)
    s = np.float32(0.017)
    sn, sk = workloads.signs(n, 41), workloads.signs(k, 42)
    x = workloads.bf16_round_trip(np.random.default_rng(m + k).standard_normal((m, k)).astype(np.float32))
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    for y_dt in ("bf16", "f32"):
        y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "bf16", y_dt)
        assert og.relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("m,n,k", [(17, 300, 64), (40, 1000, 128), (257, 33, 192), (520, 600, 1088)])
def test_gemm_whole_k_steps(G, cb, bpw, m, n, k):
    # k a multiple of 64 (the 8-wave GEMM, 32 weight rows a wave): one, two and
    # an odd number of k-steps; n not a multiple of 32, so one wave's rows end
    # inside it and whole waves lie past n; m just above the GEMV range, a
    # single activation row in the last tile, and several tiles both ways
    i1, i2 = _random_layer(n, k, bpw, 7000 + m + n + k)
    s = np.float32(0.019)
    sn, sk = workloads.signs(n, 71), workloads.signs(k, 72)
    x = workloads.bf16_round_trip(np.random.default_rng(m * k).standard_normal((m, k)).astype(np.float32))
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    for y_dt in ("bf16", "f32"):
        y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "bf16", y_dt)
        assert np.isfinite(y).all()
        assert og.relative_error(y, ref) <= TOL_BF16
        assert og.row_relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("bpw", [3, 4])
def test_gemm_long_k(G, cb, bpw):
    # 384 whole k-steps (k = 3 x 8192): the loop's buffer offsets reach
    # 48 KiB per index row and 12 MiB across the x~ tile
    m, n, k = 20, 96, 24576
    i1, i2 = _random_layer(n, k, bpw, 7700 + bpw)
    s = np.float32(0.011)
    sn, sk = workloads.signs(n, 77), workloads.signs(k, 78)
    x = workloads.bf16_round_trip(np.random.default_rng(bpw).standard_normal((m, k)).astype(np.float32))
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "bf16", "f32")
    assert np.isfinite(y).all()
    assert og.relative_error(y, ref) <= TOL_BF16
    assert og.row_relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("bpw", [2, 3, 4])
def test_gemm_k_split(G, cb, bpw):
    # long rows and fewer 256 x 256 tiles than CUs: every tile's k-steps are
    # split between two workgroups that meet through partial sums and a tile
    # counter in the control words (12 ragged tiles, 128 k-steps, remainders
    # of 64); all rows checked, both output types, and a repeat call on the
    # same workspace (the counters must be back at zero) bit-identical
    m, n, k = 600, 1000, 8192
    i1, i2 = _random_layer(n, k, bpw, 8100 + bpw)
    s = np.float32(0.013)
    sn, sk = workloads.signs(n, 81), workloads.signs(k, 82)
    x = workloads.bf16_round_trip(np.random.default_rng(bpw + 81).standard_normal((m, k)).astype(np.float32))
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb)
    xt = _t(x, torch.bfloat16)
    ws = torch.zeros(G.workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
    for y_dt in (torch.bfloat16, torch.float32):
        outs = []
        for _ in range(2):
            y = torch.full((m, n), float("nan"), device="cuda", dtype=y_dt)
            G.fused_linear(L, xt, y, ws)
            torch.cuda.synchronize()
            outs.append(y.float().cpu().numpy())
        assert np.isfinite(outs[0]).all()
        assert og.relative_error(outs[0], ref) <= TOL_BF16
        assert og.row_relative_error(outs[0], ref) <= TOL_BF16
        assert np.array_equal(outs[0], outs[1])
    assert not ws[:4352].any().item()                 # control words left zero


_LDS_ORDER_SCRIPT = r"""
import numpy as np, torch
from dequant_e8_codebook_amd import glq
import workloads
cb = glq.device_codebook("cuda")
for bpw in (4, 3, 2):
    n, k, m = 256, 256, 64
    i1 = workloads.random_indices((n, k // 8), 5)
    i2 = None if bpw == 2 else workloads.random_indices((n, k // 8), 6, 256 if bpw == 3 else 65536,
                                                         np.uint8 if bpw == 3 else np.uint16)
    L = glq.Layer.from_numpy(i1, i2, 0.01, workloads.signs(n, 1), workloads.signs(k, 2), cb)
    x = torch.randn(m, k, device="cuda").to(torch.bfloat16)
    for y_dt in (torch.float32, torch.bfloat16):
        y = torch.empty(m, n, device="cuda", dtype=y_dt)
        ws = torch.zeros(glq.workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
        glq.fused_linear(L, x, y, ws)
torch.cuda.synchronize()
print("ok", flush=True)
"""


def test_lds_limit_any_call_order(G):
    # a fresh process whose first prefill call needs the most LDS (4 bpw) and
    # whose later calls need less: each kernel gets its own LDS limit
    import os, subprocess, sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _LDS_ORDER_SCRIPT], cwd=root, capture_output=True, text=True,
                       timeout=110)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("m,n,k", [(1, 1, 8), (4, 17, 24), (6, 64, 520), (2, 300, 256)])
def test_fused_shapes_f32(G, cb, bpw, m, n, k):
    i1, i2 = _random_layer(n, k, bpw, 2000 + n + k + m)
    s = np.float32(0.011)
    sn, sk = workloads.signs(n, 21), workloads.signs(k, 22)
    x = np.random.default_rng(n + k).standard_normal((m, k)).astype(np.float32)
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "f32", "f32")
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    assert og.relative_error(y, ref) <= TOL_F32


@pytest.mark.parametrize("flags", [1, 2, 3])
@pytest.mark.parametrize("x_dt,m", [("f32", 3), ("bf16", 2), ("bf16", 40)])
def test_fused_flags(G, cb, flags, x_dt, m):
    n, k, bpw = 96, 128, 4
    i1, i2 = _random_layer(n, k, bpw, 77 + flags)
    s = np.float32(0.05)
    sn, sk = workloads.signs(n, 31), workloads.signs(k, 32)
    x = np.random.default_rng(9).standard_normal((m, k)).astype(np.float32)
    if x_dt == "bf16":
        x = workloads.bf16_round_trip(x)
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, x_dt, "f32", flags)
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk, input_rht=not (flags & 1), output_rht=not (flags & 2))
    assert og.relative_error(y, ref) <= (TOL_F32 if x_dt == "f32" else TOL_BF16)


def test_m_zero_is_noop(G, cb):
    i1, i2 = _random_layer(16, 64, 2, 5)
    L = G.Layer.from_numpy(i1, i2, 1.0, workloads.signs(16, 1), workloads.signs(64, 2), cb)
    x = torch.empty((0, 64), device="cuda", dtype=torch.bfloat16)
    y = torch.empty((0, 16), device="cuda", dtype=torch.bfloat16)
    ws = torch.zeros(256, device="cuda", dtype=torch.uint8)
    G.fused_linear(L, x, y, ws)


# ------------------------------------------------- full-size workloads ----

def _tile_rows(m, tile=256):
    """One row in every 256-row output tile (the prefill GEMM's M tiles, at a
    different offset in each), the last row, and a few more."""
    rows = {min(m - 1, t + (t // tile * 37 + 11) % tile) for t in range(0, m, tile)}
    return sorted(rows | {0, m - 1, m // 2})


def _full_check(G, cb, spec, rows):
    i1, i2 = _random_layer(spec.n, spec.k, spec.bpw, spec.seed_base + 7)
    s = np.float32(0.02)
    sn, sk = workloads.sign_n(spec), workloads.sign_k(spec)
    x = workloads.activations(spec)
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, spec.x_dtype, spec.y_dtype)
    assert np.all(np.isfinite(y))                      # every element written (y starts as NaN)
    rows = sorted(set(r % spec.m for r in rows))
    ref = og.layer_reference(x[rows], i1, i2, spec.bpw, s, sn, sk)
    assert og.relative_error(y[rows], ref) <= TOL_BF16


@pytest.mark.parametrize("name", ["gemv", "batch16", "prefill_up"])
def test_full_size_workload(G, cb, name):
    spec = workloads.layer_specs(name)[0]
    rows = range(spec.m) if spec.m <= 16 else _tile_rows(spec.m) + [977]
    _full_check(G, cb, spec, rows)


@pytest.mark.parametrize("which", range(6))
def test_full_size_dit_block(G, cb, which):
    spec = workloads.layer_specs("dit_block")[which]
    _full_check(G, cb, spec, _tile_rows(spec.m))


# ------------------------------------- single-launch layer at small batch ----

@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("n,k,m", [(150, 512, 1), (4100, 1024, 2), (64, 4096, 4), (4096, 4096, 1),
                                   (3072, 3072, 3)])
def test_small_batch_single_launch(G, cb, bpw, n, k, m):
    # eligible for the one-kernel layer: bf16 x, m <= 4, m*k and m*n <= 16384,
    # k/8 a multiple of 8; n = 4100 has more 16-row tiles than workgroups
    i1, i2 = _random_layer(n, k, bpw, 3000 + n + m)
    s = np.float32(0.017)
    sn, sk = workloads.signs(n, 41), workloads.signs(k, 42)
    L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb)
    ws = torch.zeros(G.workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
    ref = None
    for call in range(3):                      # the same workspace, three calls in a row
        x = workloads.bf16_round_trip(np.random.default_rng(call + m).standard_normal((m, k)).astype(np.float32))
        for y_dt in (torch.bfloat16, torch.float32):
            y = torch.empty((m, n), device="cuda", dtype=y_dt)
            G.fused_linear(L, _t(x, torch.bfloat16), y, ws)
            torch.cuda.synchronize()
            ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
            assert og.relative_error(y.float().cpu().numpy(), ref) <= TOL_BF16
            assert int(ws[:4352].count_nonzero().item()) == 0     # completion counters left at zero


@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("m,n,k,flags", [(2, 150, 512, 2), (7, 300, 768, 0), (16, 64, 2048, 0), (9, 1000, 256, 2),
                                         (1, 40, 4096, 2)])
def test_small_batch_operand_layout(G, cb, bpw, m, n, k, flags):
    # at most 16 rows, k a multiple of 256, bf16 x: the input transform writes
    # x~ in the GEMV's operand layout; the operand rows past m keep whatever
    # the workspace held (here all-ones bytes, NaN as bf16) and feed no stored
    # output. flags = 2 (no output transform) keeps m <= 4 off the
    # single-launch layer.
    i1, i2 = _random_layer(n, k, bpw, 4000 + m + k)
    s = np.float32(0.03)
    sn, sk = workloads.signs(n, 71), workloads.signs(k, 72)
    x = workloads.bf16_round_trip(np.random.default_rng(m + k).standard_normal((m, k)).astype(np.float32))
    L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb)
    ws = torch.full((G.workspace_bytes(L, m),), 255, device="cuda", dtype=torch.uint8)
    ws[:4352] = 0                                      # completion counters start at zero
    y = torch.empty((m, n), device="cuda", dtype=torch.float32)
    G.fused_linear(L, _t(x, torch.bfloat16), y, ws, flags)
    torch.cuda.synchronize()
    yy = y.cpu().numpy()
    assert np.all(np.isfinite(yy))
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk, output_rht=not (flags & 2))
    assert og.relative_error(yy, ref) <= TOL_BF16


@pytest.mark.parametrize("n,k,bpw", [(1024, 8192, 2), (8192, 1024, 4), (16384, 1024, 2)])
def test_one_row_whole_block_layers(G, cb, n, k, bpw):
    # one activation row whose Hadamard block is all of k (8192) or all of n
    # (8192, 16384): the single-launch layer's transforms with every stage
    # fixed at compile time (4096 is covered above, 16384 along k below)
    i1, i2 = _random_layer(n, k, bpw, 7000 + n + k)
    s = np.float32(0.013)
    sn, sk = workloads.signs(n, 51), workloads.signs(k, 52)
    x = workloads.bf16_round_trip(np.random.default_rng(n + k).standard_normal((1, k)).astype(np.float32))
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "bf16", "bf16")
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    assert og.relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("n", [1024, 2048, 4096, 8192, 16384])
@pytest.mark.parametrize("y_dt", ["bf16", "f32"])
def test_one_row_output_tail(G, cb, n, y_dt):
    # one row whose output Hadamard block is all of n: at 8192 and 16384 the
    # last workgroup's 16-byte loads of z and vector stores of y (8 or 16
    # waves of 1024 elements), below that the 16-wave path (NaN-filled y:
    # every element must be written)
    k, bpw = 512, 2
    i1, i2 = _random_layer(n, k, bpw, 7100 + n)
    s = np.float32(0.02)
    sn, sk = workloads.signs(n, 53), workloads.signs(k, 54)
    x = workloads.bf16_round_trip(np.random.default_rng(n).standard_normal((1, k)).astype(np.float32))
    L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb)
    ws = torch.zeros(G.workspace_bytes(L, 1), device="cuda", dtype=torch.uint8)
    y = torch.full((1, n), float("nan"), device="cuda", dtype=torch.float32 if y_dt == "f32" else torch.bfloat16)
    G.fused_linear(L, _t(x, torch.bfloat16), y, ws)
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    assert np.isfinite(got).all()
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    assert og.relative_error(got, ref) <= TOL_BF16


# ------------------------------------------------------ per-row scales ----

def _row_scale_layer(n, k, bpw, seed, scale=0.75):
    i1, i2 = _random_layer(n, k, bpw, seed)
    rs = np.random.default_rng(seed).uniform(0.005, 0.05, n).astype(np.float32)
    return i1, i2, np.float32(scale), rs


@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_decode_row_scales_bitexact(G, cb, bpw, out):
    n, k = 300, 264
    i1, i2, s, rs = _row_scale_layer(n, k, bpw, 500 + bpw)
    L = G.Layer.from_numpy(i1, i2, s, None, None, cb, row_scale=rs)
    w = torch.empty((n, k), device="cuda", dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    G.decode_weights(L, w)
    torch.cuda.synchronize()
    se = og.effective_scale(s, rs)
    ref = og.decode_bf16_bits(i1, i2, bpw, se) if out == "bf16" else og.decode_f32(i1, i2, bpw, se).view(np.uint32)
    assert np.array_equal(_bits(w), ref)


@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("m,x_dt", [(1, "bf16"), (3, "bf16"), (12, "bf16"), (40, "bf16"), (300, "bf16"), (3, "f32")])
def test_fused_row_scales(G, cb, bpw, m, x_dt):
    # the single-launch layer (m <= 4), the GEMV (m <= 16), the GEMM, the float32 path
    n, k = 272, 512
    i1, i2, s, rs = _row_scale_layer(n, k, bpw, 600 + bpw + m)
    sn, sk = workloads.signs(n, 61), workloads.signs(k, 62)
    x = np.random.default_rng(m).standard_normal((m, k)).astype(np.float32)
    if x_dt == "bf16":
        x = workloads.bf16_round_trip(x)
    L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb, row_scale=rs)
    xt = _t(x, torch.float32 if x_dt == "f32" else torch.bfloat16)
    ref = og.layer_reference(x, i1, i2, bpw, og.effective_scale(s, rs), sn, sk)
    for y_dt in (("f32",) if x_dt == "f32" else ("bf16", "f32")):
        y = torch.empty((m, n), device="cuda", dtype=torch.float32 if y_dt == "f32" else torch.bfloat16)
        ws = torch.zeros(G.workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
        G.fused_linear(L, xt, y, ws)
        torch.cuda.synchronize()
        assert og.relative_error(y.float().cpu().numpy(), ref) <= (TOL_F32 if x_dt == "f32" else TOL_BF16)


@pytest.mark.parametrize("bpw", [2, 4])
def test_fused_row_scales_k_split(G, cb, bpw):
    # per-row scales through the epilogue of the decode-GEMM split along k
    # (two 256-row tiles with a ragged second, 96 k-steps: remainders of 48)
    m, n, k = 300, 272, 6144
    i1, i2, s, rs = _row_scale_layer(n, k, bpw, 690 + bpw)
    sn, sk = workloads.signs(n, 69), workloads.signs(k, 70)
    x = workloads.bf16_round_trip(np.random.default_rng(bpw + 69).standard_normal((m, k)).astype(np.float32))
    L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb, row_scale=rs)
    ref = og.layer_reference(x, i1, i2, bpw, og.effective_scale(s, rs), sn, sk)
    y = torch.full((m, n), float("nan"), device="cuda", dtype=torch.bfloat16)
    ws = torch.zeros(G.workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
    G.fused_linear(L, _t(x, torch.bfloat16), y, ws)
    torch.cuda.synchronize()
    yn = y.float().cpu().numpy()
    assert np.isfinite(yn).all()
    assert og.relative_error(yn, ref) <= TOL_BF16
    assert og.row_relative_error(yn, ref) <= TOL_BF16


def test_fused_row_scales_oracle_encoded(G, cb):
    # rows of very different magnitude encoded with per-row scales by the oracle
    spec = workloads.layer_specs("batch16")[0]
    n, k, m = 256, 512, 16
    w = workloads.weights(workloads.LayerSpec("rs", n, k, 4, m, "normal", "bf16", "bf16", 0, spec.seed_base))
    w = w * np.logspace(-2, 0, n)[:, None]
    sn, sk = workloads.signs(n, 71), workloads.signs(k, 72)
    i1, i2, rs = og.encode(w, 4, sn, sk, per_row=True)
    x = workloads.bf16_round_trip(np.random.default_rng(3).standard_normal((m, k)).astype(np.float32))
    y = _run_linear(G, cb, i1, i2, rs, sn, sk, x, "bf16", "f32")
    ref = og.layer_reference(x, i1, i2, 4, rs, sn, sk)
    assert og.relative_error(y, ref) <= TOL_BF16


@pytest.mark.gpu
@pytest.mark.parametrize("bpw,m", [(2, 1), (3, 64)])
def test_fused_ldlq_encoded(G, cb, bpw, m):
    # indices from the oracle's LDLQ encoder (error feedback changes the
    # indices, not the decode): the fused path still matches the oracle layer
    from oracle import ldlq as ol
    n, k = 256, 512
    spec = workloads.LayerSpec("ldlq", n, k, bpw, m, "student_t", "bf16", "bf16", 4, 6100 + bpw)
    w = workloads.weights(spec)
    sn, sk = workloads.sign_n(spec), workloads.sign_k(spec)
    h = ol.hessian_from_inputs(workloads.calibration(spec, 1024))
    i1, i2, s = ol.encode_ldlq(w, bpw, sn, sk, h)
    x = workloads.activations(spec)
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, "bf16", "f32")
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    assert og.relative_error(y, ref) <= TOL_BF16


# ------------------------------------------- entropy-coded lattice layers ----

def _ep_weights(n, k, seed, dist="student_t"):
    spec = workloads.LayerSpec("ep", n, k, 2, 1, dist, "f32", "f32", 0, seed)
    return workloads.weights(spec).astype(np.float32), workloads.sign_n(spec), workloads.sign_k(spec)


def _ep_decode(G, layer, dt):
    out = torch.empty((layer.n, layer.k), device="cuda", dtype=dt)
    G.ep_decode_weights(layer, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("n,k,step,lane_groups", [(8, 64, 0.4, 1), (13, 96, 0.25, 3), (5, 8, 0.3, 2),
                                                  (64, 512, 0.2, 32), (100, 1032, 0.12, 5)])
def test_ep_decode_oracle_stream_bitexact(G, n, k, step, lane_groups):
    # the oracle's own stream (EntroPack readings R20-R23), decoded on the GPU,
    # gives the oracle's weights bit for bit
    from oracle import entropack as oep
    w, sn, sk = _ep_weights(n, k, 7 * n + k)
    o = oep.encode(w.astype(np.float64), sn, sk, step, lane_groups)
    h = G.EpHost(n, k, lane_groups, float(o.step), o.row_scale, G.EpModel(), o.states, o.offsets, o.words)
    for t in range(5):
        h.model.nsym[t] = len(o.model.freq[t])
        h.model.vmin[t] = int(o.model.vmin[t])
        for s_, f in enumerate(o.model.freq[t]):
            h.model.freq[t][s_] = int(f)
    L = G.EpLayer.from_host(h)
    z, s = oep.quantise_lattice(w.astype(np.float64), sn, sk, step)
    ref = oep.weights_f32(z, s, step)
    assert np.array_equal(_bits(_ep_decode(G, L, torch.float32)), ref.view(np.uint32))
    assert np.array_equal(_bits(_ep_decode(G, L, torch.bfloat16)), og.f32_to_bf16_bits(ref))


@pytest.mark.parametrize("n,k,step,lane_groups", [(256, 4096, 0.19, 32), (3072, 1024, 0.3, 7), (1, 8, 0.5, 1)])
def test_ep_decode_library_stream_lossless(G, n, k, step, lane_groups):
    # row scales 1 and step 2 make the float32 output z itself: the lattice
    # points come back exactly as the oracle's quantiser chose them
    from oracle import entropack as oep
    w, sn, sk = _ep_weights(n, k, n + k)
    h = G.ep_encode(w, sn, sk, step, lane_groups)
    L = G.EpLayer.from_host(h)
    L.row_scale.fill_(1.0)
    L.step = 2.0
    out = _ep_decode(G, L, torch.float32).cpu().numpy()
    z, s = oep.quantise_lattice(w.astype(np.float64), sn, sk, step)
    assert np.array_equal(out, z.reshape(n, k).astype(np.float32))
    assert np.array_equal(h.row_scale, s)


@pytest.mark.parametrize("shape,step", [((4096, 4096), 0.25), ((12288, 3072), 0.35)])
def test_ep_decode_full_size(G, shape, step):
    # full-size layers: every weight against the oracle's quantiser
    from oracle import entropack as oep
    n, k = shape
    w, sn, sk = _ep_weights(n, k, 7000 + n)
    h = G.ep_encode(w, sn, sk, step, 32)
    L = G.EpLayer.from_host(h)
    got = _bits(_ep_decode(G, L, torch.bfloat16))
    z, s = oep.quantise_lattice(w.astype(np.float64), sn, sk, step)
    assert np.array_equal(got, og.f32_to_bf16_bits(oep.weights_f32(z, s, step)))


def test_ep_decode_graph_replays(G):
    # several replays of a captured decode, each equal to the eager result
    w, sn, sk = _ep_weights(512, 2048, 99)
    L = G.EpLayer.from_host(G.ep_encode(w, sn, sk, 0.22, 16))
    ref = _ep_decode(G, L, torch.bfloat16)
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        G.ep_decode_weights(L, out, stream=s)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            G.ep_decode_weights(L, out, stream=s)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("m", [1, 16])
def test_ep_fused_linear_graph_replays(G, m):
    # a captured entropy-coded layer (m = 1: the fill kernel that clears z and
    # the fused decode-product with its atomic row sums; m = 16: decode then
    # GEMV), replayed with eager calls in between: every replay within the
    # tolerance of the oracle and close to the eager result (float32 atomics
    # may sum in another order)
    n, k = 768, 1024
    L, w32, sn, sk = _ep_layer_case(G, n, k, 0.27, 31 + m)
    x = workloads.bf16_round_trip(np.random.default_rng(m).standard_normal((m, k)).astype(np.float32))
    xt = _t(x, torch.bfloat16)
    ref = rht.rht_transpose(rht.rht_forward(x.astype(np.float64), sk) @ w32.T, sn)
    ws = torch.zeros(G.ep_workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
    y = torch.empty((m, n), device="cuda", dtype=torch.float32)
    eager = torch.empty_like(y)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        G.ep_fused_linear(L, xt, y, ws, stream=s)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            G.ep_fused_linear(L, xt, y, ws, stream=s)
    for _ in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        G.ep_fused_linear(L, xt, eager, ws)
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert og.relative_error(got, ref) <= TOL_BF16
        assert og.relative_error(got, eager.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("m,bpw", [(1, 2), (3, 4), (16, 4), (40, 3)])
def test_fused_graph_replays(G, cb, m, bpw):
    # a captured layer forward (single launch with its completion tickets at
    # m <= 4, transform + GEMV + transform at 16, the GEMM path at 40),
    # replayed several times with eager calls on the same workspace in
    # between: every replay and every eager call give the eager result bit
    # for bit, and the ticket counters are left at zero
    n, k = 512, 1024
    i1, i2 = _random_layer(n, k, bpw, 900 + m)
    s = np.float32(0.02)
    sn, sk = workloads.signs(n, 61), workloads.signs(k, 62)
    L = G.Layer.from_numpy(i1, i2, s, sn, sk, cb)
    x = _t(workloads.bf16_round_trip(np.random.default_rng(m).standard_normal((m, k)).astype(np.float32)),
           torch.bfloat16)
    ws = torch.zeros(G.workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
    ref = torch.empty((m, n), device="cuda", dtype=torch.bfloat16)
    G.fused_linear(L, x, ref, ws)
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    eager = torch.empty_like(ref)
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        G.fused_linear(L, x, out, ws, stream=st)
        st.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            G.fused_linear(L, x, out, ws, stream=st)
    for _ in range(4):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        G.fused_linear(L, x, eager, ws)
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), ref.view(torch.int16))
        assert int(ws[:4352].count_nonzero().item()) == 0
    y = ref.float().cpu().numpy()
    assert og.relative_error(y, og.layer_reference(x.float().cpu().numpy(), i1, i2, bpw, s, sn, sk)) <= TOL_BF16


def _ep_layer_case(G, n, k, step, seed, lane_groups=8):
    from oracle import entropack as oep
    w, sn, sk = _ep_weights(n, k, seed)
    h = G.ep_encode(w, sn, sk, step, lane_groups)
    L = G.EpLayer.from_host(h, sign_k=sk, sign_n=sn)
    z, s = oep.quantise_lattice(w.astype(np.float64), sn, sk, step)
    return L, oep.weights_f32(z, s, step).astype(np.float64), sn, sk


def _ep_run(G, L, x, x_dt, y_dt, flags=0):
    m = x.shape[0]
    xt = _t(x.astype(np.float32), torch.float32 if x_dt == "f32" else torch.bfloat16)
    ncol = L.n
    y = torch.empty((m, ncol), device="cuda", dtype=torch.float32 if y_dt == "f32" else torch.bfloat16)
    ws = torch.zeros(max(G.ep_workspace_bytes(L, max(m, 1)), 256), device="cuda", dtype=torch.uint8)
    G.ep_fused_linear(L, xt, y, ws, flags)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


@pytest.mark.parametrize("n,k,m,x_dt,y_dt", [(256, 512, 1, "bf16", "bf16"), (256, 512, 16, "f32", "f32"),
                                            (300, 264, 5, "bf16", "f32"), (40, 8, 3, "f32", "f32"),
                                            (300, 264, 37, "bf16", "f32"), (1024, 4096, 300, "bf16", "bf16"),
                                            (520, 3072, 257, "f32", "bf16"), (600, 1024, 40, "bf16", "f32")])
def test_ep_fused_linear(G, n, k, m, x_dt, y_dt):
    # y = U^T W^ (V x) on entropy-coded weights: bf16 matrix cores against
    # the float64 product of the oracle's weights and transforms
    L, w32, sn, sk = _ep_layer_case(G, n, k, 0.3, 11 * n + k)
    x = np.random.default_rng(n + m).standard_normal((m, k)).astype(np.float32)
    if x_dt == "bf16":
        x = workloads.bf16_round_trip(x)
    y = _ep_run(G, L, x, x_dt, y_dt)
    ref = rht.rht_transpose(rht.rht_forward(x.astype(np.float64), sk) @ w32.T, sn)
    assert og.relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("flags", [1, 2, 3])
def test_ep_fused_linear_flags(G, flags):
    n, k, m = 256, 1024, 24
    L, w32, sn, sk = _ep_layer_case(G, n, k, 0.25, 77)
    x = workloads.bf16_round_trip(np.random.default_rng(flags).standard_normal((m, k)).astype(np.float32))
    y = _ep_run(G, L, x, "bf16", "f32", flags)
    xt = x.astype(np.float64) if flags & 1 else rht.rht_forward(x.astype(np.float64), sk)
    ref = xt @ w32.T
    if not flags & 2:
        ref = rht.rht_transpose(ref, sn)
    assert og.relative_error(y, ref) <= TOL_BF16


@pytest.mark.parametrize("n,k,m,lg,x_dt,y_dt", [(4096, 4096, 1, 32, "bf16", "bf16"), (4096, 4096, 1, 8, "bf16", "f32"),
                                               (1000, 1024, 1, 8, "f32", "f32"), (513, 512, 1, 5, "bf16", "f32"),
                                               (257, 768, 1, 3, "f32", "bf16"), (96, 4096, 1, 64, "bf16", "f32"),
                                               (4096, 4096, 2, 8, "bf16", "f32"), (1000, 1024, 7, 8, "f32", "f32"),
                                               (512, 2048, 16, 32, "bf16", "bf16")])
def test_ep_fused_small_batch(G, n, k, m, lg, x_dt, y_dt):
    # m = 1 with k / 8 >= 64 takes the decode fused into the product (the
    # weights never stored): block sizes that end mid-row, blocks spanning
    # several rows (lg = 3, 5), 4- and 8-wave launches (4096 x 4096 at lg 8
    # has 4096 blocks); m = 2 .. 16 the decode + GEMV path
    L, w32, sn, sk = _ep_layer_case(G, n, k, 0.3, 13 * n + k + m, lane_groups=lg)
    x = np.random.default_rng(n + 3 * m).standard_normal((m, k)).astype(np.float32)
    if x_dt == "bf16":
        x = workloads.bf16_round_trip(x)
    y = _ep_run(G, L, x, x_dt, y_dt)
    ref = rht.rht_transpose(rht.rht_forward(x.astype(np.float64), sk) @ w32.T, sn)
    assert og.relative_error(y, ref) <= TOL_BF16
    # every row checked on its own (a row summed into the wrong output row
    # would move the total error little)
    for i in range(m):
        assert og.relative_error(y[i], ref[i]) <= TOL_BF16


@pytest.mark.parametrize("flags,y_dt", [(1, "f32"), (2, "f32"), (3, "f32"), (2, "bf16"), (3, "bf16")])
def test_ep_fused_small_batch_flags(G, flags, y_dt):
    # at m = 1 without the output transform a float32 y is summed into
    # directly, a bf16 y converted from the float32 sums
    n, k, m = 384, 1024, 1
    L, w32, sn, sk = _ep_layer_case(G, n, k, 0.25, 78 + flags)
    x = workloads.bf16_round_trip(np.random.default_rng(flags).standard_normal((m, k)).astype(np.float32))
    y = _ep_run(G, L, x, "bf16", y_dt, flags)
    xt = x.astype(np.float64) if flags & 1 else rht.rht_forward(x.astype(np.float64), sk)
    ref = xt @ w32.T
    if not flags & 2:
        ref = rht.rht_transpose(ref, sn)
    assert og.relative_error(y, ref) <= TOL_BF16


def test_ep_fused_small_batch_repeat_clears(G):
    # the float32 sums start from zero on every call (no carry-over between
    # calls sharing a workspace or an output)
    n, k, m = 256, 1024, 1
    L, w32, sn, sk = _ep_layer_case(G, n, k, 0.3, 5)
    x = workloads.bf16_round_trip(np.random.default_rng(9).standard_normal((m, k)).astype(np.float32))
    xt = _t(x, torch.bfloat16)
    ws = torch.zeros(G.ep_workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
    ref = rht.rht_forward(x.astype(np.float64), sk) @ w32.T
    for flags in (0, 2):
        y = torch.full((m, n), 7.0, device="cuda", dtype=torch.float32)
        for _ in range(3):
            G.ep_fused_linear(L, xt, y, ws, flags)
        torch.cuda.synchronize()
        want = ref if flags & 2 else rht.rht_transpose(ref, sn)
        assert og.relative_error(y.cpu().numpy(), want) <= TOL_BF16


def test_ep_fused_linear_full_size_sampled(G):
    # the prefill up-projection shape, 16384 x 4096 at m = 2048: sampled rows
    # of y against the oracle (row r of y needs only row r of x)
    n, k, m = 16384, 4096, 2048
    L, w32, sn, sk = _ep_layer_case(G, n, k, 0.28, 4242, lane_groups=32)
    x = workloads.bf16_round_trip(np.random.default_rng(5).standard_normal((m, k)).astype(np.float32))
    y = _ep_run(G, L, x, "bf16", "bf16")
    rows = np.array([0, 1, 255, 256, 1023, 1500, 2046, 2047])
    ref = rht.rht_transpose(rht.rht_forward(x[rows].astype(np.float64), sk) @ w32.T, sn)
    assert og.relative_error(y[rows], ref) <= TOL_BF16


def test_ep_decode_zero_layer(G):
    # a stream with no words (every symbol certain) decodes to zeros
    w = np.zeros((64, 256), np.float32)
    sn, sk = workloads.signs(64, 3), workloads.signs(256, 4)
    h = G.ep_encode(w, sn, sk, 0.25, 4)
    assert len(h.words) == 0
    L = G.EpLayer.from_host(h, sign_k=sk, sign_n=sn)
    out = _ep_decode(G, L, torch.float32)
    assert not out.any()
    y = _ep_run(G, L, np.ones((3, 256), np.float32), "f32", "f32")
    assert not np.any(y)
    # the same at k = 512, where m = 1 takes the fused decode-product
    w = np.zeros((64, 512), np.float32)
    sk = workloads.signs(512, 4)
    h = G.ep_encode(w, sn, sk, 0.25, 4)
    assert len(h.words) == 0
    L = G.EpLayer.from_host(h, sign_k=sk, sign_n=sn)
    for m in (1, 3, 16):
        y = _ep_run(G, L, np.ones((m, 512), np.float32), "f32", "f32")
        assert not np.any(y)


@pytest.mark.parametrize("m,x_dt,y_dt,bpw", [(1, "bf16", "bf16", 2), (3, "f32", "f32", 2), (16, "bf16", "f32", 4),
                                            (40, "bf16", "bf16", 3)])
def test_largest_hadamard_block_along_k(G, cb, m, x_dt, y_dt, bpw):
    # k = 16384: the largest supported Hadamard block, 2048 groups per row
    n, k = 64, 16384
    i1, i2 = _random_layer(n, k, bpw, 161 + bpw)
    s = np.float32(2.1e-3)
    sn, sk = workloads.signs(n, 5), workloads.signs(k, 6)
    x = np.random.default_rng(m).standard_normal((m, k)).astype(np.float32)
    if x_dt == "bf16":
        x = workloads.bf16_round_trip(x)
    y = _run_linear(G, cb, i1, i2, s, sn, sk, x, x_dt, y_dt)
    ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
    assert og.relative_error(y, ref) <= (TOL_F32 if x_dt == "f32" and y_dt == "f32" else TOL_BF16)


# ------------------------------------------------------ binding checks ----

def test_binding_rejects_bad_arguments(G, cb):
    # wrong shapes, strided or mismatched tensors raise ValueError in the
    # binding before any launch; the good call afterwards still works
    n, k, m = 32, 64, 3
    i1, i2 = _random_layer(n, k, 4, 5)
    L = G.Layer.from_numpy(i1, i2, 0.01, workloads.signs(n, 1), workloads.signs(k, 2), cb)
    x = torch.randn(m, k, device="cuda").to(torch.bfloat16)
    y = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
    ws = torch.zeros(G.workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
    bad = [
        dict(x=torch.randn(m, k + 8, device="cuda").to(torch.bfloat16)),          # k mismatch
        dict(x=torch.randn(k, device="cuda").to(torch.bfloat16)),                 # 1-D x
        dict(x=torch.randn(k, m, device="cuda").to(torch.bfloat16).t()),          # strided x
        dict(y=torch.empty(m, n + 1, device="cuda", dtype=torch.bfloat16)),       # y shape
        dict(y=torch.empty(m + 1, n, device="cuda", dtype=torch.bfloat16)),
        dict(x=x.cpu()),                                                          # host x
        dict(ws=ws[1:]),                                                          # misaligned workspace
        dict(y=ws[:m * n * 2].view(torch.bfloat16).view(m, n)),                   # y inside the workspace
    ]
    for b in bad:
        with pytest.raises(ValueError):
            G.fused_linear(L, b.get("x", x), b.get("y", y), b.get("ws", ws))
    short = G.Layer(L.n, L.k, L.bpw, L.scale, L.idx1, L.idx2, L.sign_k[:k - 1], L.sign_n, L.cb)
    with pytest.raises(ValueError):
        G.fused_linear(short, x, y, ws)
    G.fused_linear(short, x, y, ws, G.FLAG_NO_INPUT_RHT)          # signs along k not needed then
    with pytest.raises(ValueError):
        G.decode_weights(L, torch.empty(n, k + 8, device="cuda", dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        G.rht_apply(x, torch.empty(m, k, device="cuda"), torch.ones(k - 1, device="cuda", dtype=torch.int8), False)
    G.fused_linear(L, x, y, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all()
