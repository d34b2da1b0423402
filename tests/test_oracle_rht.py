"""Pins of the oracle's randomized Hadamard transform against the closed
form H[i, j] = (-1)^popcount(i & j) of the Sylvester matrix, H H = b I,
orthogonality, and explicit unit-vector images that fix the order of the
sign flip and the Hadamard product."""
import os

import numpy as np
import pytest

from oracle import rht

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def h_closed_form(b):
    i = np.arange(b)[:, None]
    j = np.arange(b)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    return np.where(pc % 2 == 0, 1.0, -1.0)


def test_golden_h8():
    rows = [l.split() for l in open(os.path.join(GOLD, "hadamard_8.txt"))
            if l.strip() and not l.startswith("#")]
    h8 = np.array(rows, dtype=np.float64)
    assert np.array_equal(rht.hadamard(8), h8)
    assert np.array_equal(h_closed_form(8), h8)


@pytest.mark.parametrize("b", [1, 2, 4, 16, 64, 256, 1024, 4096])
def test_hadamard_square_is_b_identity(b):
    h = rht.hadamard(b)
    assert np.array_equal(h @ h, b * np.eye(b))
    if b <= 256:
        assert np.array_equal(h, h_closed_form(b))


def test_block_size():
    assert [rht.block_size(n) for n in (256, 4096, 3072, 12288, 16384, 12, 7, 8)] == \
        [256, 4096, 1024, 4096, 16384, 4, 1, 8]


@pytest.mark.parametrize("n", [8, 256, 3072, 8192, 16384])
def test_forward_transform_explicit(n):
    # V e_j = sigma_j * H_b[:, j mod b] / sqrt(b) placed in block j // b:
    # the sign of input j multiplies the whole column (sign first).
    rng = np.random.default_rng(n)
    sigma = (1 - 2 * rng.integers(0, 2, n)).astype(np.int8)
    b = rht.block_size(n)
    for j in (0, 1, n // 2 + 3, n - 1):
        e = np.zeros(n)
        e[j] = 1.0
        out = rht.rht_forward(e, sigma)
        blk, jj = divmod(j, b)
        expect = np.zeros(n)
        col = np.array([(-1.0) ** bin(i & jj).count("1") for i in range(b)])
        expect[blk * b:(blk + 1) * b] = sigma[j] * col / np.sqrt(b)
        assert np.allclose(out, expect, rtol=0, atol=1e-15)
        # transpose: H first, then the sign of each OUTPUT entry
        out_t = rht.rht_transpose(e, sigma)
        expect_t = np.zeros(n)
        expect_t[blk * b:(blk + 1) * b] = col / np.sqrt(b)
        expect_t *= sigma
        assert np.allclose(out_t, expect_t, rtol=0, atol=1e-15)


@pytest.mark.parametrize("n", [256, 3072, 16384])
def test_orthogonal_and_inverse(n):
    rng = np.random.default_rng(1 + n)
    sigma = (1 - 2 * rng.integers(0, 2, n)).astype(np.int8)
    x = rng.standard_normal((3, n))
    fx = rht.rht_forward(x, sigma)
    assert np.allclose(np.linalg.norm(fx, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(rht.rht_transpose(fx, sigma), x, rtol=0, atol=1e-12)


def test_large_block_factored_path_matches_closed_form():
    # b = 16384 uses the Kronecker factoring; compare a few outputs with the
    # closed-form sum over all inputs.
    n = 16384
    rng = np.random.default_rng(5)
    v = rng.standard_normal(n)
    ones = np.ones(n, dtype=np.int8)
    out = rht.rht_forward(v, ones) * np.sqrt(n)
    j = np.arange(n)
    for i in (0, 1, 777, 16383):
        sgn = np.array([1.0 if bin(i & int(t)).count("1") % 2 == 0 else -1.0 for t in j])
        assert np.isclose(out[i], (sgn * v).sum(), rtol=1e-12, atol=1e-9)


def test_weight_rotation_round_trip_and_conventions():
    rng = np.random.default_rng(9)
    n, k = 48, 64
    w = rng.standard_normal((n, k))
    sn = (1 - 2 * rng.integers(0, 2, n)).astype(np.int8)
    sk = (1 - 2 * rng.integers(0, 2, k)).astype(np.int8)
    wt = rht.rotate_weights(w, sn, sk)
    # explicit matrices: V = H_bk diag(sk)/sqrt(bk) blockwise, U likewise
    def mat(n_, s):
        b = rht.block_size(n_)
        m = np.kron(np.eye(n_ // b), h_closed_form(b)) @ np.diag(s.astype(float)) / np.sqrt(b)
        return m
    U, V = mat(n, sn), mat(k, sk)
    assert np.allclose(wt, U @ w @ V.T, atol=1e-12)
    assert np.allclose(rht.unrotate_weights(wt, sn, sk), w, atol=1e-12)
    assert np.isclose(np.linalg.norm(wt), np.linalg.norm(w), rtol=1e-13)
