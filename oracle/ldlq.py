"""LDLQ error feedback of the oracle (encoder side), float64.

TEST INFRASTRUCTURE ONLY: see the package header; the library never imports
this module.

[glq] "How it works", item 3: a block LDL decomposition of the Hessian
drives a sequential sweep over 8-weight blocks, and the quantisation error
of each block is carried forward to correct the blocks after it (the error
feedback of GPTQ, "Acknowledgments", with 8-dimensional blocks in place of
single columns). Item 2: the Hessian is rotated by the same randomized
Hadamard transform as the weights. Readings of what the pages leave open
(R15: the error feedback is optional; the plain encoder rounds every group
on its own, this one adds the feedback below given a Hessian):

R17 Hessian: H [k, k], symmetric positive semi-definite, over the input
    features in the original basis (H = X^T X / m for calibration inputs
    X [m, k]). Rotated like the weights: H~ = V H V^T. Damped as in GPTQ:
    H~ + delta * mean(diag H~) * I, delta = 0.01 unless given (the mean of
    the diagonal does not change under the orthogonal V, so damping before
    or after the rotation is the same).
R18 Decomposition: H~ = (I + U) D (I + U)^T, U strictly block upper
    triangular and D block diagonal, with blocks of 8 input features (the
    groups of R8). It is unique for a positive definite H~. Computed from
    the last block backward: D_last = H~_last,last; U_i,last =
    H~_i,last D_last^-1; the leading part is replaced by its Schur
    complement and the step repeats.
R19 Sweep: blocks j = 0, 1, ..., k/8 - 1 in order along k, every row
    independently: T_j = X_j + sum_{i<j} (X_i - X^_i) U_ij, X^_j = Q(T_j),
    with X = W~ / s (global or per-row scale, computed as without LDLQ) and
    Q the nearest-neighbour / residual quantiser of R9 / R10. Then
    (X^ - X)(I + U) = eta with eta_j = X^_j - T_j, so the proxy loss
    tr((X^ - X) H~ (X^ - X)^T) equals sum_j eta_j D_j eta_j^T.
"""
from __future__ import annotations

import numpy as np

from . import glq, rht

BLOCK = 8
DEFAULT_DAMP = 0.01


def hessian_from_inputs(x: np.ndarray) -> np.ndarray:
    """H = X^T X / m for calibration inputs X [m, k] (R17)."""
    x = np.asarray(x, dtype=np.float64)
    return (x.T @ x) / x.shape[0]


def rotate_hessian(h: np.ndarray, sign_k: np.ndarray) -> np.ndarray:
    """H~ = V H V^T (R17): the weight rotation of R6 with U = V."""
    h = np.asarray(h, dtype=np.float64)
    if h.ndim != 2 or h.shape[0] != h.shape[1]:
        raise ValueError("Hessian must be square")
    return rht.rotate_weights(h, sign_k, sign_k)


def damp_hessian(h: np.ndarray, damp: float = DEFAULT_DAMP) -> np.ndarray:
    """H + damp * mean(diag H) * I (R17)."""
    h = np.array(h, dtype=np.float64, copy=True)
    h[np.diag_indices_from(h)] += damp * np.mean(np.diag(h))
    return h


def block_udu(h: np.ndarray, b: int = BLOCK):
    """H = (I + U) D (I + U)^T with U strictly block upper triangular (R18).

    Returns U [k, k] (zero on and below the diagonal blocks) and D [k/b, b, b].
    Raises ValueError when a diagonal block of a Schur complement is not
    positive definite (H not positive definite).
    """
    a = np.array(h, dtype=np.float64, copy=True)
    k = a.shape[0]
    if a.shape != (k, k) or k % b:
        raise ValueError("Hessian must be square with a side that is a multiple of the block")
    nb = k // b
    u = np.zeros((k, k))
    d = np.zeros((nb, b, b))
    for j in range(nb - 1, -1, -1):
        s = slice(j * b, (j + 1) * b)
        dj = a[s, s]
        try:
            np.linalg.cholesky(dj)
        except np.linalg.LinAlgError:
            raise ValueError("Hessian is not positive definite") from None
        d[j] = dj
        top = slice(0, j * b)
        if j == 0:
            break
        uj = a[top, s] @ np.linalg.inv(dj)          # U_i,j = H_i,j D_j^-1 for i < j
        u[top, s] = uj
        a[top, top] = a[top, top] - uj @ dj @ uj.T   # Schur complement of block j
    return u, d


def encode_ldlq(w: np.ndarray, bpw: int, sign_n: np.ndarray, sign_k: np.ndarray,
                hessian: np.ndarray, damp: float = DEFAULT_DAMP, scale: float | None = None,
                per_row: bool = False, search=glq.nearest, trace: bool = False):
    """Quantise W [n, k] (original basis) with LDLQ error feedback (R17-R19).

    Returns (idx1 u16, idx2 | None, s) like glq.encode; with trace=True a
    fourth item holds the sweep's targets T, decoded X^, the scaled weights X,
    the damped rotated Hessian and its factors U, D.
    """
    if bpw not in (2, 3, 4):
        raise ValueError("bpw must be 2, 3 or 4")
    wt = rht.rotate_weights(w, sign_n, sign_k)
    n, k = wt.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 8")
    if per_row:
        s = glq.row_scales(wt)
        x = wt / s.astype(np.float64)[:, None]
    else:
        s = glq.global_scale(wt) if scale is None else np.float32(scale)
        x = wt / np.float64(s)
    ht = damp_hessian(rotate_hessian(hessian, sign_k), damp)
    u, d = block_udu(ht)
    xhat = np.zeros((n, k))
    t_all = np.zeros((n, k))
    g = k // BLOCK
    i1 = np.zeros((n, g), dtype=np.int64)
    i2 = np.zeros((n, g), dtype=np.int64) if bpw > 2 else None
    for j in range(g):
        cols = slice(j * BLOCK, (j + 1) * BLOCK)
        prev = slice(0, j * BLOCK)
        t = x[:, cols] + (x[:, prev] - xhat[:, prev]) @ u[prev, cols]
        a1, a2, v = glq.quantise(t, bpw, search)
        i1[:, j] = a1
        if i2 is not None:
            i2[:, j] = a2
        xhat[:, cols] = v
        t_all[:, cols] = t
    idx2 = None if i2 is None else i2.astype(np.uint8 if bpw == 3 else np.uint16)
    out = (i1.astype(np.uint16), idx2, (s if per_row else np.float32(s)))
    if trace:
        out = out + ({"t": t_all, "xhat": xhat, "x": x, "h": ht, "u": u, "d": d},)
    return out


def proxy_loss(xhat: np.ndarray, x: np.ndarray, h: np.ndarray) -> float:
    """tr((X^ - X) H (X^ - X)^T), the layer-output error the feedback
    minimises (GPTQ's objective), in the scaled rotated units."""
    e = np.asarray(xhat, dtype=np.float64) - np.asarray(x, dtype=np.float64)
    return float(np.sum((e @ np.asarray(h, dtype=np.float64)) * e))
