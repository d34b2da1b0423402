"""Randomized Hadamard transform (RHT) of the oracle, float64.

[glq] "How it works", item 2: random sign flips followed by a fast
Walsh-Hadamard transform, applied to the weights so the Hessian becomes
roughly proportional to the identity and Euclidean nearest neighbour is
close to optimal. Readings of what the pages leave open:

R4  Hadamard matrix: Sylvester construction in natural order,
    H_1 = [1], H_2b = [[H_b, H_b], [H_b, -H_b]]  (= scipy.linalg.hadamard).
R5  Length n that is not a power of two: block-diagonal Hadamard with block
    b(n) = largest power of two dividing n (the Walsh-Hadamard transform is
    defined only for powers of two); the sign flips cover all n entries.
R6  Normalisation 1/sqrt(b), so the transform is orthogonal:
      V = (I (x) H_b) diag(sigma) / sqrt(b)      (sign first, then Hadamard)
    applied as x~ = V x along the input axis, and its transpose
      V^T = diag(sigma) (I (x) H_b) / sqrt(b)    (Hadamard first, then sign)
    The layer is W~ = U W V^T, and at run time y = U^T (s W^) (V x).
"""
from __future__ import annotations

import functools

import numpy as np
import scipy.linalg

DENSE_MAX = 4096


def block_size(n: int) -> int:
    """b(n): the largest power of two dividing n (R5)."""
    if n <= 0:
        raise ValueError("length must be positive")
    return n & -n


@functools.lru_cache(maxsize=16)
def hadamard(b: int) -> np.ndarray:
    """Dense Sylvester Hadamard matrix H_b (R4), float64, b <= DENSE_MAX."""
    if b > DENSE_MAX:
        raise ValueError("dense Hadamard limited to 4096")
    h = scipy.linalg.hadamard(b).astype(np.float64)
    h.setflags(write=False)
    return h


def _apply_h(v: np.ndarray, b: int) -> np.ndarray:
    """Multiply every length-b block of the last axis by H_b.

    For b > 4096 the Sylvester identity H_{b1 b2} = H_{b1} (x) H_{b2} is used:
    the block is viewed as a b1 x b2 matrix and multiplied by H_{b1} on the
    left and H_{b2} on the right (the same matrix product, factored).
    """
    shp = v.shape
    n = shp[-1]
    blocks = v.reshape(-1, n // b, b)
    if b <= DENSE_MAX:
        # H symmetric: row-vector form, every block one row of a single product
        out = blocks.reshape(-1, b) @ hadamard(b)
    else:
        # H_b1 on the left, H_b2 on the right of each b1 x b2 block, each as
        # one matrix product over all blocks
        b2 = DENSE_MAX
        b1 = b // b2
        m = blocks.reshape(-1, b2) @ hadamard(b2)                        # rows of every block times H_b2
        m = m.reshape(-1, b1, b2).transpose(0, 2, 1).reshape(-1, b1) @ hadamard(b1)
        out = m.reshape(-1, b2, b1).transpose(0, 2, 1)                   # back to b1 x b2 blocks
    return out.reshape(shp)


def rht_forward(v: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """V v along the last axis: sign flips, then block Hadamard, / sqrt(b)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if sigma.shape != (n,):
        raise ValueError("sign vector length")
    b = block_size(n)
    return _apply_h(v * sigma.astype(np.float64), b) / np.sqrt(b)


def rht_transpose(v: np.ndarray, sigma: np.ndarray) -> np.ndarray:
    """V^T v along the last axis: block Hadamard, then sign flips, / sqrt(b)."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    if sigma.shape != (n,):
        raise ValueError("sign vector length")
    b = block_size(n)
    return _apply_h(v, b) * sigma.astype(np.float64) / np.sqrt(b)


def rotate_weights(w: np.ndarray, sign_n: np.ndarray, sign_k: np.ndarray) -> np.ndarray:
    """W~ = U W V^T for W [n, k] (R6)."""
    w = np.asarray(w, dtype=np.float64)
    wv = rht_forward(w, sign_k)                 # rows: W V^T  (V acting on each row)
    return rht_forward(wv.T, sign_n).T          # columns: U (W V^T)


def unrotate_weights(wt: np.ndarray, sign_n: np.ndarray, sign_k: np.ndarray) -> np.ndarray:
    """W = U^T W~ V, the inverse of rotate_weights."""
    wt = np.asarray(wt, dtype=np.float64)
    a = rht_transpose(wt.T, sign_n).T           # U^T W~
    return rht_transpose(a, sign_k)             # (U^T W~) V
