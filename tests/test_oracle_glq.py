"""Pins of the oracle's scale, encode, residual stage, decode and layer
reference: the page's bit-width and size tables, codebook-exact layers that
the encoder must invert, brute force on tiny inputs, torch's bfloat16 cast
for the rounding step, and an independent x @ W^T product."""
import os

import numpy as np
import pytest
import torch

from oracle import e8, glq, rht
import workloads

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    return [l.split() for l in open(os.path.join(GOLD, name))
            if l.strip() and not l.startswith("#")]


def _signs(n, seed):
    return workloads.signs(n, seed)


# ---------------------------------------------------------------- sizes ----

def test_bit_width_table():
    for bpw, s1, s2, _ in _golden("glq_bit_widths.txt"):
        bpw, s1, s2 = int(bpw), int(s1), int(s2)
        n, k = 64, 128
        assert glq.compressed_bytes(n, k, bpw) * 8 == (n * k // 8) * (s1 + s2)
        assert glq.compressed_bytes(n, k, bpw) * 8 / (n * k) == bpw     # nominal rate


def test_results_table_sizes_follow_nominal_rate():
    rows = {r[0]: (float(r[1]), float(r[2])) for r in _golden("glq_results_sizes.txt")}
    bf16_mb = rows["bf16"][1]
    for name, bpw in (("glq4", 4), ("glq3", 3), ("glq2", 2)):
        eff, mb = rows[name]
        assert eff == bpw
        assert abs(bf16_mb * bpw / 16 - mb) <= 1.0       # 1537.5, 1153.1, 768.75


@pytest.mark.parametrize("n,k,bpw", [(4096, 4096, 2), (37, 136, 3), (64, 256, 4), (1, 8, 2)])
def test_actual_bpw_is_the_serialised_length(n, k, bpw):
    # actual_bpw against the length of a layer actually written out (index
    # planes, scale, packed signs) and read back losslessly: the stored
    # bytes are enough to rebuild every weight, and they are all counted
    rng = np.random.default_rng(n + k + bpw)
    i1 = rng.integers(0, 65536, (n, k // 8)).astype(np.uint16)
    i2 = None
    if bpw == 3:
        i2 = rng.integers(0, 256, (n, k // 8)).astype(np.uint8)
    elif bpw == 4:
        i2 = rng.integers(0, 65536, (n, k // 8)).astype(np.uint16)
    s = np.float32(0.0173)
    sn = np.where(rng.random(n) < 0.5, -1, 1).astype(np.int8)
    sk = np.where(rng.random(k) < 0.5, -1, 1).astype(np.int8)
    blob = glq.serialise_layer(i1, i2, s, sn, sk)
    assert glq.actual_bpw(n, k, bpw) == 8.0 * len(blob) / (n * k)
    j1, j2, t, tn, tk = glq.deserialise_layer(blob, n, k, bpw)
    assert np.array_equal(j1, i1) and t == s and np.array_equal(tn, sn) and np.array_equal(tk, sk)
    if bpw > 2:
        assert np.array_equal(j2, i2)
    assert np.array_equal(glq.decode_bf16_bits(j1, j2, bpw, t), glq.decode_bf16_bits(i1, i2, bpw, s))
    with pytest.raises(ValueError):
        glq.deserialise_layer(blob[:-1], n, k, bpw)
    if n * k == 4096 * 4096:
        assert 2.0 < glq.actual_bpw(n, k, bpw) < 2.001


# ---------------------------------------------------------------- scale ----

def test_global_scale():
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, (64, 64))
    s = glq.global_scale(w)
    assert s.dtype == np.float32
    assert s == np.float32(np.sqrt(np.mean(w * w)))
    assert glq.global_scale(np.zeros((8, 8))) == np.float32(1.0)
    with pytest.raises(ValueError):
        glq.global_scale(np.array([[np.nan] * 8]))
    # the rotation is orthogonal, so the scale of W~ equals the rms of W
    sn, sk = _signs(64, 1), _signs(64, 2)
    wt = rht.rotate_weights(w, sn, sk)
    assert np.isclose(glq.global_scale(wt), s, rtol=1e-6)


# --------------------------------------------------------------- encode ----

def _codebook_exact_layer(n, k, bpw, seed, scale=0.0173):
    """W = U^T (s * decode(idx)) V for random indices: encode must return
    exactly these indices when given the same s."""
    rng = np.random.default_rng(seed)
    g = k // 8
    if bpw == 2:
        i1 = rng.integers(0, 65536, (n, g))
        i2 = None
    else:
        # residual entries among the 241 shortest vectors (origin + roots)
        i1 = rng.integers(0, 65536, (n, g))
        i2 = rng.integers(0, 241, (n, g))
    vt = glq.decode_values(i1.astype(np.uint16), None if i2 is None else i2, bpw)
    sn, sk = _signs(n, seed + 1), _signs(k, seed + 2)
    w = rht.unrotate_weights(np.float64(np.float32(scale)) * vt, sn, sk)
    return w, i1, i2, sn, sk, np.float32(scale)


@pytest.mark.parametrize("bpw", [2, 4])
def test_encode_inverts_codebook_exact_layer(bpw):
    # at 4 bpw the residual 2^-2 C[i2] (i2 < 241, |.| <= 0.354) lies strictly
    # inside the stage-1 Voronoi cell (packing radius 0.707)
    n, k = 16, 64
    w, i1, i2, sn, sk, s = _codebook_exact_layer(n, k, bpw, 40 + bpw)
    e1, e2, es = glq.encode(w, bpw, sn, sk, scale=s)
    assert es == s
    assert np.array_equal(e1, i1)
    if bpw == 2:
        assert e2 is None
    else:
        assert np.array_equal(e2.astype(np.int64), i2)
        assert e2.dtype == np.uint16


def test_encode_3bpw_facet_ties():
    # at 3 bpw, X = C[i1] + C[r]/2 with r a root is the centre of a Voronoi
    # facet: equidistant from C[i1] and C[i1] + C[r] and from no other lattice
    # point. Stage 1 must take the lower index of the two (when both are in
    # the codebook), and stage 2 the root that points back to X.
    n, k = 16, 64
    w, i1, i2, sn, sk, s = _codebook_exact_layer(n, k, 3, 43)
    e1, e2, _ = glq.encode(w, 3, sn, sk, scale=s)
    cb = e8.codebook().astype(np.int64)
    i1f, i2f = i1.reshape(-1), i2.reshape(-1)
    other = e8.index_of(cb[i1f] + cb[i2f])
    other = np.where(i2f == 0, i1f, other)
    exp1 = np.where(other >= 0, np.minimum(i1f, other), i1f)
    exp2 = np.where(exp1 == i1f, i2f, e8.index_of(-cb[i2f], 256))
    assert (i2f != 0).sum() > 50 and (exp1 != i1f).sum() > 5
    assert np.array_equal(e1.reshape(-1).astype(np.int64), exp1)
    assert np.array_equal(e2.reshape(-1).astype(np.int64), exp2)


def test_encode_matches_bruteforce_definition_tiny():
    rng = np.random.default_rng(17)
    w = rng.normal(0, 0.02, (4, 32))
    sn, sk = _signs(4, 3), _signs(32, 4)
    for bpw in (2, 3, 4):
        a = glq.encode(w, bpw, sn, sk)
        b = glq.encode(w, bpw, sn, sk, search=glq.nearest_bruteforce)
        assert np.array_equal(a[0], b[0]) and a[2] == b[2]
        if bpw > 2:
            assert np.array_equal(a[1], b[1])
        # brute force of the definition written out for the residual stage
        if bpw > 2:
            wt = rht.rotate_weights(w, sn, sk)
            x = glq.groups(wt).reshape(-1, 8) / np.float64(a[2])
            r = x - e8.codebook_f64()[a[0].reshape(-1)]
            kk = glq.RESID_SHIFT[bpw]
            cr = e8.codebook_f64()[:1 << glq.RESID_BITS[bpw]] * 2.0 ** -kk
            d = ((r[:, None, :] - cr[None]) ** 2).sum(2)
            assert np.array_equal(np.argmin(d, 1), a[1].reshape(-1).astype(np.int64))


def test_residual_stages_reduce_error():
    rng = np.random.default_rng(21)
    w = rng.normal(0, 0.02, (64, 256))
    sn, sk = _signs(64, 5), _signs(256, 6)
    wt = rht.rotate_weights(w, sn, sk)
    mse = []
    for bpw in (2, 3, 4):
        i1, i2, s = glq.encode(w, bpw, sn, sk)
        v = glq.decode_values(i1, i2, bpw) * np.float64(s)
        mse.append(np.mean((wt - v) ** 2) / np.mean(wt ** 2))
    assert mse[0] > mse[1] > mse[2]
    assert 0.07 < mse[0] < 0.11 and 0.02 < mse[1] < 0.04 and 0.006 < mse[2] < 0.014


def test_encode_rejects_bad_args():
    with pytest.raises(ValueError):
        glq.encode(np.zeros((4, 12)), 2, _signs(4, 1), _signs(12, 2))
    with pytest.raises(ValueError):
        glq.encode(np.zeros((4, 16)), 5, _signs(4, 1), _signs(16, 2))


# --------------------------------------------------------------- decode ----

def test_decode_values_exact_and_codebook_only_case():
    i1 = np.array([[0, 1, 241, 65535]], dtype=np.uint16)
    v = glq.decode_values(i1, None, 2)
    assert np.array_equal(v.reshape(4, 8), e8.codebook()[[0, 1, 241, 65535]] / 2.0)
    # s = 1: decoded float32 weights are exactly the small half-integers
    w = glq.decode_f32(i1, None, 2, 1.0)
    assert np.array_equal(w.reshape(4, 8), (e8.codebook()[[0, 1, 241, 65535]] / 2.0).astype(np.float32))
    # residual: v = C[i1] + 2^-k C[i2]
    i2 = np.array([[1, 2, 0, 255]], dtype=np.uint8)
    v3 = glq.decode_values(i1, i2, 3).reshape(4, 8)
    cb = e8.codebook() / 2.0
    assert np.array_equal(v3, cb[[0, 1, 241, 65535]] + 0.5 * cb[[1, 2, 0, 255]])
    i2w = np.array([[65535, 2, 0, 7]], dtype=np.uint16)
    v4 = glq.decode_values(i1, i2w, 4).reshape(4, 8)
    assert np.array_equal(v4, cb[[0, 1, 241, 65535]] + 0.25 * cb[[65535, 2, 0, 7]])
    with pytest.raises(ValueError):
        glq.decode_values(i1, np.array([[256, 0, 0, 0]]), 3)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(4)
    w = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 0.02,
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0, 0.0], np.float32)])
    ours = glq.f32_to_bf16_bits(w)
    ref = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_decode_single_fp32_multiply():
    # w32 must equal the correctly rounded product of s and v (v exact)
    rng = np.random.default_rng(8)
    i1 = rng.integers(0, 65536, (8, 16)).astype(np.uint16)
    i2 = rng.integers(0, 65536, (8, 16)).astype(np.uint16)
    s = np.float32(0.0123456)
    w = glq.decode_f32(i1, i2, 4, s)
    v = glq.decode_values(i1, i2, 4)
    exact = np.float64(s) * v
    assert np.array_equal(w, exact.astype(np.float32))       # one rounding of the exact product


# ----------------------------------------------------------- layer ref ----

@pytest.mark.parametrize("bpw,n,k", [(2, 32, 64), (3, 48, 96), (4, 64, 3072 // 16)])
def test_layer_reference_equals_plain_matmul(bpw, n, k):
    w, i1, i2, sn, sk, s = _codebook_exact_layer(n, k, bpw, 60 + bpw)
    x = np.random.default_rng(1).standard_normal((5, k))
    y = glq.layer_reference(x, i1.astype(np.uint16), i2, bpw, s, sn, sk)
    # the decoded float32 weights differ from s*v by at most one rounding;
    # compare against x @ W_hat^T with W_hat = U^T fl32(s v) V computed directly
    w32 = glq.decode_f32(i1.astype(np.uint16), i2, bpw, s).astype(np.float64)
    w_hat = rht.unrotate_weights(w32, sn, sk)
    assert np.allclose(y, x @ w_hat.T, rtol=0, atol=1e-12)
    # and against the original W (equal up to the float32 rounding of s*v)
    assert np.allclose(y, x @ w.T, rtol=1e-6, atol=1e-7)


def test_layer_reference_rotation_flags():
    w, i1, i2, sn, sk, s = _codebook_exact_layer(16, 32, 2, 70)
    x = np.random.default_rng(2).standard_normal((3, 32))
    z = glq.layer_reference(x, i1.astype(np.uint16), None, 2, s, sn, sk, input_rht=True, output_rht=False)
    y = glq.layer_reference(x, i1.astype(np.uint16), None, 2, s, sn, sk)
    assert np.allclose(rht.rht_transpose(z, sn), y, atol=1e-13)
    xt = rht.rht_forward(x, sk)
    y2 = glq.layer_reference(xt, i1.astype(np.uint16), None, 2, s, sn, sk, input_rht=False)
    assert np.allclose(y2, y, atol=1e-13)


def test_relative_error_measure():
    assert glq.relative_error(np.array([1.0, 2.0]), np.array([1.0, 2.0])) == 0.0
    assert glq.relative_error(np.array([1.5, 2.0]), np.array([1.0, 2.0])) == 0.25


def test_row_relative_error_measure():
    # hand-computed: row 0 error 0.5 of max 2 (0.25), row 1 error 0.1 of max
    # 0.2 (0.5); the global measure sees 0.5 / 2 = 0.25
    ref = np.array([[1.0, 2.0], [0.1, 0.2]])
    got = np.array([[1.5, 2.0], [0.1, 0.1]])
    assert glq.row_relative_error(got, ref) == pytest.approx(0.5)
    assert glq.relative_error(got, ref) == pytest.approx(0.25)
    # one row: the two measures agree; an all-zero reference row counts its
    # absolute error
    assert glq.row_relative_error(got[:1], ref[:1]) == glq.relative_error(got[:1], ref[:1])
    assert glq.row_relative_error(np.array([[0.0, 0.3]]), np.zeros((1, 2))) == pytest.approx(0.3)


# -------------------------------------------------------- per-row scales ----

def test_row_scales_equal_norm_rows_reduce_to_global_scale():
    # rows that are signed permutations of one dyadic vector have exactly equal
    # mean squares, so every row scale is the global scale and the per-row
    # encoding must give the global-scale indices
    rng = np.random.default_rng(11)
    n, k = 12, 64
    base = rng.integers(-40, 41, k) / 1024.0
    wt = np.stack([rng.permutation(base) * rng.choice([-1.0, 1.0], k) for _ in range(n)])
    sn, sk = _signs(n, 3), _signs(k, 4)
    w = rht.unrotate_weights(wt, sn, sk)
    rs = glq.row_scales(rht.rotate_weights(w, sn, sk))
    assert rs.dtype == np.float32 and rs.shape == (n,)
    g1, g2, gs = glq.encode(w, 4, sn, sk)
    p1, p2, ps = glq.encode(w, 4, sn, sk, per_row=True)
    assert np.all(np.abs(ps / gs - 1) < 1e-6)
    assert np.array_equal(p1, g1) and np.array_equal(p2, g2)


def test_row_scales_power_of_two_row_factors():
    # multiplying row r of W~ by 2^e_r multiplies its scale by 2^e_r and leaves
    # the indices unchanged
    rng = np.random.default_rng(12)
    n, k = 10, 96
    wt = rng.standard_normal((n, k)) * 0.02
    e = rng.integers(-6, 7, n)
    sn, sk = _signs(n, 5), _signs(k, 6)
    a1, a2, a_s = glq.encode(rht.unrotate_weights(wt, sn, sk), 3, sn, sk, per_row=True)
    b1, b2, b_s = glq.encode(rht.unrotate_weights(wt * np.ldexp(1.0, e)[:, None], sn, sk), 3, sn, sk, per_row=True)
    assert np.array_equal(a1, b1) and np.array_equal(a2, b2)
    assert np.allclose(b_s, a_s * np.ldexp(1.0, e), rtol=2 ** -22, atol=0)


def test_row_scales_keep_small_rows():
    # rows 1000x smaller than the rest vanish under one global scale but are
    # encoded to the same relative error as the others with row scales
    rng = np.random.default_rng(13)
    n, k = 16, 128
    wt = rng.standard_normal((n, k)) * 0.02
    wt[::4] *= 1e-3
    sn, sk = _signs(n, 7), _signs(k, 8)
    w = rht.unrotate_weights(wt, sn, sk)
    g1, g2, gs = glq.encode(w, 2, sn, sk)
    p1, p2, ps = glq.encode(w, 2, sn, sk, per_row=True)
    def rel(i1, s):
        wd = glq.decode_f32(i1, None, 2, s).astype(np.float64)
        return np.linalg.norm(wd - wt, axis=1) / np.linalg.norm(wt, axis=1)
    assert np.all(rel(g1, gs)[::4] > 0.99)                 # global: small rows decode to ~0
    assert np.all(rel(p1, ps) < 0.6)                        # per row: every row keeps its shape


def test_decode_with_row_scales_is_rowwise_global_decode():
    rng = np.random.default_rng(14)
    i1 = rng.integers(0, 65536, (6, 8)).astype(np.uint16)
    i2 = rng.integers(0, 256, (6, 8)).astype(np.uint8)
    s = glq.effective_scale(0.5, rng.uniform(0.01, 0.04, 6).astype(np.float32))
    w = glq.decode_f32(i1, i2, 3, s)
    for r in range(6):
        assert np.array_equal(w[r], glq.decode_f32(i1[r:r + 1], i2[r:r + 1], 3, s[r])[0])
    assert glq.effective_scale(0.5, np.float32([0.3]))[0] == np.float32(np.float32(0.5) * np.float32(0.3))
