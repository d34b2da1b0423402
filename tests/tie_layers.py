"""Layers whose rotated weights are exact ties of the quantisers (helper of
the tie tests; not collected by pytest).

W = U^T W~ V is built so that every step of the rotation is exact in
float32 and float64: n odd (Hadamard block 1 along n, U = diag(sign_n)),
k = 16 q with q odd (block 16 along k, 1/sqrt(16) = 1/4), W~ entries
multiples of 1/16 times a power of two. Then rotating W gives W~ back
bit for bit in any summation order, and a quantiser sees exactly the
tie points put into W~.
"""
import os

import numpy as np

from oracle import rht

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e8_lattice_ties.txt")


def lattice_ties():
    """(names, x [T, 8], z [T, 8]) of the golden tie file."""
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    names = [r[0] for r in rows]
    x = np.array([[float(v) for v in r[1:9]] for r in rows])
    z = np.array([[int(v) for v in r[9:17]] for r in rows], dtype=np.int64)
    return names, x, z


def exact_layer(wt: np.ndarray, sign_n: np.ndarray, sign_k: np.ndarray) -> np.ndarray:
    """float32 W with rotate_weights(W) == wt exactly."""
    n, k = wt.shape
    assert n % 2 == 1 and k % 16 == 0 and (k // 16) % 2 == 1
    w = rht.unrotate_weights(wt, sign_n, sign_k)
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w)
    assert np.array_equal(rht.rotate_weights(w32, sign_n, sign_k), np.asarray(wt, dtype=np.float64))
    return w32


def _filler(sum_sq: float) -> np.ndarray:
    """8 multiples of 1/4 whose squares sum to sum_sq (a multiple of 1/16)."""
    target = int(round(sum_sq * 16))
    assert target == sum_sq * 16 and target >= 0

    def split(rem, slots):
        if rem == 0:
            return []
        if slots == 0:
            return None
        a = int(np.sqrt(rem))
        while a > 0:
            rest = split(rem - a * a, slots - 1)
            if rest is not None:
                return [a] + rest
            a -= 1
        return None

    parts = split(target, 8)
    assert parts is not None
    return np.array(parts + [0] * (8 - len(parts)), dtype=np.float64) / 4.0


def ep_tie_rows(groups_per_row=3):
    """Rotated weights W~ [3, 48] (row scale 1 at step 1): every row is tie
    groups from the golden file, padded by one filler group so that the
    row's mean square is exactly 1 (s_r = 1, and X / step = W~ exactly).
    Returns (wt, positions) with positions[(row, group)] = golden row."""
    _, x, _ = lattice_ties()
    t = len(x)
    rows, pos = [], {}
    g_per = 5
    for r in range(3):
        picks = [(r * g_per + j) % t for j in range(g_per)]
        groups = [x[p] for p in picks]
        for j, p in enumerate(picks):
            pos[(r, j)] = p
        ss = float(sum(np.sum(g * g) for g in groups))
        groups.append(_filler(48.0 - ss))
        rows.append(np.concatenate(groups))
    wt = np.stack(rows)
    assert np.all(np.mean(wt * wt, axis=1) == 1.0)
    return wt, pos
