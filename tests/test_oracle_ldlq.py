"""Pins of the oracle's LDLQ encoder (glq page, "How it works" items 2-3).

Each check rests on something other than the oracle's own formulas: the
block factorisation is rebuilt from a library Cholesky of the reversed
matrix; the first two blocks of the sweep are recomputed with brute-force
nearest neighbours and the 2x2 block Schur formula on explicitly built
dense rotation matrices; the proxy-loss identity (X^ - X)(I + U) = eta
holds only for the right feedback sign and operand order; a Hessian
proportional to the identity must give the plain encoder's indices.
"""
import numpy as np
import pytest
import scipy.linalg

import workloads as wl
from oracle import e8, glq, ldlq


def _spd(k, seed, cond=50.0):
    rng = np.random.default_rng(seed)
    q, _ = np.linalg.qr(rng.standard_normal((k, k)))
    ev = np.geomspace(1.0, cond, k)
    return (q * ev) @ q.T


def _spec(n, k, outliers=4, seed=77, bpw=2):
    return wl.LayerSpec("ldlq", n, k, bpw, 1, "normal", "f32", "f32", outliers, seed)


def _dense_v(sign_k):
    """V = (I (x) H_b) diag(sigma) / sqrt(b) as an explicit matrix."""
    k = len(sign_k)
    b = k & -k
    hb = scipy.linalg.hadamard(b).astype(np.float64)
    return np.kron(np.eye(k // b), hb) @ np.diag(sign_k.astype(np.float64)) / np.sqrt(b)


@pytest.mark.parametrize("k,seed", [(16, 1), (64, 2), (96, 3)])
def test_block_udu_matches_reversed_cholesky(k, seed):
    h = _spd(k, seed)
    u, d = ldlq.block_udu(h)
    # independent route: P H P = L L^T (library Cholesky), R = P L P upper
    # triangular with H = R R^T; M = R blockdiag(R_jj)^-1, D_j = R_jj R_jj^T
    p = np.eye(k)[::-1]
    r = p @ np.linalg.cholesky(p @ h @ p) @ p
    nb = k // 8
    rd = np.zeros((k, k))
    for j in range(nb):
        s = slice(8 * j, 8 * j + 8)
        rd[s, s] = r[s, s]
        np.testing.assert_allclose(d[j], r[s, s] @ r[s, s].T, rtol=1e-10, atol=1e-10)
    m = r @ np.linalg.inv(rd)
    np.testing.assert_allclose(np.eye(k) + u, m, rtol=0, atol=1e-9)
    # structure: U is zero on and below the diagonal blocks
    for i in range(nb):
        for j in range(nb):
            if j <= i:
                assert not u[8 * i:8 * i + 8, 8 * j:8 * j + 8].any()
    rec = (np.eye(k) + u) @ scipy.linalg.block_diag(*d) @ (np.eye(k) + u).T
    np.testing.assert_allclose(rec, h, rtol=0, atol=1e-10 * np.abs(h).max())


def test_block_udu_rejects_indefinite():
    h = _spd(16, 5)
    h[3, 3] = -1.0
    with pytest.raises(ValueError):
        ldlq.block_udu(h)


@pytest.mark.parametrize("bpw", [2, 3, 4])
@pytest.mark.parametrize("c", [1.0, 3.7])
def test_identity_hessian_gives_plain_encoder(bpw, c):
    spec = _spec(24, 64)
    w, sn, sk = wl.weights(spec), wl.sign_n(spec), wl.sign_k(spec)
    a1, a2, sa = ldlq.encode_ldlq(w, bpw, sn, sk, c * np.eye(64))
    b1, b2, sb = glq.encode(w, bpw, sn, sk)
    assert sa == sb
    np.testing.assert_array_equal(a1, b1)
    if bpw > 2:
        np.testing.assert_array_equal(a2, b2)


def test_first_two_blocks_by_brute_force():
    """k = 16: block 0 is the plain nearest point of X_0; block 1 is the
    nearest point of X_1 + (X_0 - X^_0) H~01 H~11^-1 (2x2 block Schur
    form), with H~ built from dense matrices."""
    n, k = 40, 16
    spec = _spec(n, k, outliers=2, seed=11)
    w, sn, sk = wl.weights(spec), wl.sign_n(spec), wl.sign_k(spec)
    h = ldlq.hessian_from_inputs(wl.calibration(spec, 256, rho=0.9))
    i1, _, s = ldlq.encode_ldlq(w, 2, sn, sk, h)

    v = _dense_v(sk)
    un = _dense_v(sn)
    wt = un @ np.asarray(w, np.float64) @ v.T
    assert s == np.float32(np.sqrt(np.mean(wt * wt)))
    x = wt / np.float64(s)
    ht = v @ h @ v.T
    ht = ht + 0.01 * np.mean(np.diag(ht)) * np.eye(k)
    cb = e8.codebook_f64()
    j0 = glq.nearest_bruteforce(x[:, :8])
    u01 = ht[:8, 8:] @ np.linalg.inv(ht[8:, 8:])
    t1 = x[:, 8:] + (x[:, :8] - cb[j0]) @ u01
    j1 = glq.nearest_bruteforce(t1)
    np.testing.assert_array_equal(i1[:, 0], j0)
    np.testing.assert_array_equal(i1[:, 1], j1)
    # the feedback must matter here, or the check above says little
    assert (j1 != glq.nearest_bruteforce(x[:, 8:])).sum() >= 5
    # and its transpose would give another answer
    t_bad = x[:, 8:] + (x[:, :8] - cb[j0]) @ u01.T
    assert (glq.nearest_bruteforce(t_bad) != j1).any()


@pytest.mark.parametrize("bpw", [2, 3, 4])
def test_proxy_loss_identity(bpw):
    spec = _spec(32, 128)
    w, sn, sk = wl.weights(spec), wl.sign_n(spec), wl.sign_k(spec)
    h = ldlq.hessian_from_inputs(wl.calibration(spec, 512))
    *_, tr = ldlq.encode_ldlq(w, bpw, sn, sk, h, trace=True)
    direct = ldlq.proxy_loss(tr["xhat"], tr["x"], tr["h"])
    eta = tr["xhat"] - tr["t"]
    summed = sum(float(np.einsum("ri,ij,rj->", eta[:, 8 * j:8 * j + 8], tr["d"][j], eta[:, 8 * j:8 * j + 8]))
                 for j in range(16))
    assert abs(direct - summed) <= 1e-9 * direct
    # X^ decodes from the returned indices
    i1, i2, _ = ldlq.encode_ldlq(w, bpw, sn, sk, h)
    np.testing.assert_array_equal(glq.decode_values(i1, i2, bpw), tr["xhat"])


@pytest.mark.parametrize("bpw,outliers,bound", [(2, 4, 0.5), (3, 4, 0.5), (4, 4, 0.5), (2, 0, 0.95)])
def test_ldlq_lowers_proxy_loss(bpw, outliers, bound):
    spec = _spec(48, 128, outliers=outliers, seed=21)
    w, sn, sk = wl.weights(spec), wl.sign_n(spec), wl.sign_k(spec)
    h = ldlq.hessian_from_inputs(wl.calibration(spec, 512))
    *_, tr = ldlq.encode_ldlq(w, bpw, sn, sk, h, trace=True)
    j1, j2, _ = glq.encode(w, bpw, sn, sk)
    plain = ldlq.proxy_loss(glq.decode_values(j1, j2, bpw), tr["x"], tr["h"])
    assert ldlq.proxy_loss(tr["xhat"], tr["x"], tr["h"]) < bound * plain


def test_hessian_scale_does_not_change_indices():
    spec = _spec(16, 64)
    w, sn, sk = wl.weights(spec), wl.sign_n(spec), wl.sign_k(spec)
    h = ldlq.hessian_from_inputs(wl.calibration(spec, 256))
    a = ldlq.encode_ldlq(w, 3, sn, sk, h)
    b = ldlq.encode_ldlq(w, 3, sn, sk, 4.0 * h)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_per_row_power_of_two_rows():
    """n odd makes U a pure sign flip (block b(n) = 1), so scaling row r of W
    by 2^p scales row r of W~ exactly: with per-row scales, s_r scales by
    2^p and the indices stay the same."""
    spec = _spec(15, 64)
    w, sn, sk = wl.weights(spec), wl.sign_n(spec), wl.sign_k(spec)
    h = ldlq.hessian_from_inputs(wl.calibration(spec, 256))
    f = 2.0 ** np.arange(-7, 8)
    a1, a2, sa = ldlq.encode_ldlq(w, 4, sn, sk, h, per_row=True)
    b1, b2, sb = ldlq.encode_ldlq(np.asarray(w) * f[:, None], 4, sn, sk, h, per_row=True)
    np.testing.assert_array_equal(a1, b1)
    np.testing.assert_array_equal(a2, b2)
    np.testing.assert_array_equal(sb, (sa * f).astype(np.float32))
