"""The allocation-free entry point (glq_fused_linear_noalloc) against the
workspace entry point (glq_fused_linear) and the oracle: two calls in a row
on each path, the second on a smaller layer, outputs bit-identical to the
workspace entry point's and within the bf16 bar of the oracle."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")
from oracle import glq as og  # noqa: E402
import workloads  # noqa: E402

pytestmark = pytest.mark.gpu
TOL_BF16 = 1e-2


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dequant_e8_codebook_amd import glq
    return glq


def _layer(G, cb, n, k, bpw, seed):
    g = k // 8
    i1 = workloads.random_indices((n, g), seed)
    i2 = None
    if bpw == 3:
        i2 = workloads.random_indices((n, g), seed + 1, 256, np.uint8)
    elif bpw == 4:
        i2 = workloads.random_indices((n, g), seed + 1)
    s = np.float32(0.013)
    sn, sk = workloads.signs(n, seed + 2), workloads.signs(k, seed + 3)
    return G.Layer.from_numpy(i1, i2, s, sn, sk, cb), (i1, i2, s, sn, sk)


def _call_both(G, L, x):
    m = x.shape[0]
    xt = torch.from_numpy(x).to(device="cuda", dtype=torch.bfloat16)
    y0 = torch.full((m, L.n), float("nan"), device="cuda", dtype=torch.bfloat16)
    y1 = torch.full((m, L.n), float("nan"), device="cuda", dtype=torch.bfloat16)
    ws = torch.zeros(G.workspace_bytes(L, m), device="cuda", dtype=torch.uint8)
    G.fused_linear(L, xt, y0, ws)
    # through the C ABI directly: no workspace pointer, no size
    st = L.struct()
    rc = G.raw().glq_fused_linear_noalloc(ctypes.byref(st), xt.data_ptr(), G.GLQ_BF16, m, y1.data_ptr(),
                                          G.GLQ_BF16, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == G.GLQ_OK, G.raw().glq_last_error()
    torch.cuda.synchronize()
    return y0.view(torch.int16).cpu().numpy(), y1.view(torch.int16).cpu().numpy(), y1.float().cpu().numpy()


# (n, k, bpw, m): the single-launch small-batch layer, then the multi-kernel
# paths (16-row GEMV, the decode-GEMM, and the decode-GEMM split along k,
# whose tile counters live in the static scratch's control words), each pair
# ending with a smaller call
@pytest.mark.parametrize("first,second", [
    ((4096, 4096, 4, 3), (1024, 1024, 2, 1)),
    ((1000, 768, 3, 12), (300, 256, 4, 5)),
    ((640, 1024, 2, 300), (264, 160, 3, 40)),
    ((512, 4096, 4, 300), (300, 8192, 3, 100)),
])
def test_noalloc_matches_workspace_entry_point(G, first, second):
    cb = G.device_codebook("cuda")
    for idx, (n, k, bpw, m) in enumerate((first, second)):
        L, (i1, i2, s, sn, sk) = _layer(G, cb, n, k, bpw, 100 * idx + n + k + bpw)
        x = workloads.bf16_round_trip(np.random.default_rng(m + n).standard_normal((m, k)).astype(np.float32))
        b0, b1, y = _call_both(G, L, x)
        assert np.array_equal(b0, b1)                          # the same kernels, bit for bit
        assert np.all(np.isfinite(y))
        ref = og.layer_reference(x, i1, i2, bpw, s, sn, sk)
        assert og.relative_error(y, ref) <= TOL_BF16


def test_noalloc_rejects_layers_beyond_the_static_scratch(G):
    cb = G.device_codebook("cuda")
    L, _ = _layer(G, cb, 16384, 4096, 3, 7)
    x = torch.zeros((2048, 4096), device="cuda", dtype=torch.bfloat16)
    y = torch.zeros((2048, 16384), device="cuda", dtype=torch.bfloat16)
    with pytest.raises(G.GlqError):
        G.fused_linear_noalloc(L, x, y)
    st = L.struct()
    rc = G.raw().glq_fused_linear_noalloc(ctypes.byref(st), x.data_ptr(), G.GLQ_BF16, 2048, y.data_ptr(),
                                          G.GLQ_BF16, 0, None)
    assert rc == G.GLQ_ERR_WORKSPACE
    assert b"static scratch" in G.raw().glq_last_error()
    # a call that fits still works afterwards
    small = x[:4, :]
    out = torch.empty((4, 16384), device="cuda", dtype=torch.bfloat16)
    G.fused_linear_noalloc(L, small, out)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
