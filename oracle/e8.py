"""E8 lattice codebook: membership, shells, the stated order, nearest point.

[glq] "How it works", item 1: the codebook holds 65536 vectors taken from
the first 7 shells of the E8 lattice. The pages fix neither coordinates,
nor which 65536 points, nor their order. Readings:

R1  Standard coordinates: x is in E8 iff all x_i are integers or all are
    integers + 1/2, and sum(x) is even. Minimum squared norm 2. Points are
    held as y = 2x (int8), so membership is: all y_i even or all odd, and
    sum(y) = 0 mod 4.
R2  "7 shells" counts the origin as shell 0: squared norms 0,2,...,10 in
    full (56881 points) plus the first 8655 points of the norm-12 shell in
    the stated order.
R3  Stated order, ascending on the key
      (|x|^2, -orbit_size, max|x_i|, (|x_1|,...,|x_8|) lexicographic, j)
    where an orbit is the set of points sharing the vector of absolute
    values, orbit_size = 2^nnz for integer points and 128 for half-integer
    points (one sign is fixed by parity), and j is the sign counter:
      integer points: bit t of j = [t-th nonzero coordinate is negative]
      half points:    bit t of j = [x_{t+1} < 0] for t = 0, 1, 2 and
                      [x_{t+2} < 0] for t = 3..6; the sign of x4 is the one
                      the even-sum rule leaves
    Index i is the position in this order; the codebook is the first 65536.
    (Format 3. Format 2 fixed x8 by parity and counted x1..x7; x4 keeps the
    parity-fixed sign in the same half-vector as the two fastest sign bits.)
    Parity against the real glq package is unpinned (its order is not on
    the pages): the format is self-consistent, not checkpoint-compatible.
"""
from __future__ import annotations

import functools
import itertools

import numpy as np

CODEBOOK_SIZE = 65536


def is_e8(y: np.ndarray) -> np.ndarray:
    """Membership of points given in doubled coordinates y = 2x (R1)."""
    y = np.asarray(y, dtype=np.int64)
    par = y % 2
    all_even = np.all(par == 0, axis=-1)
    all_odd = np.all(par == 1, axis=-1)
    return (all_even | all_odd) & (y.sum(axis=-1) % 4 == 0)


def enumerate_shells(max_norm2: int) -> np.ndarray:
    """All E8 points with |x|^2 <= max_norm2, as y = 2x (int8), unordered.

    Brute force over the bounding box: |x_i| <= sqrt(max_norm2).
    """
    r = int(np.floor(np.sqrt(max_norm2)))
    ev = np.arange(-2 * r, 2 * r + 1, 2)
    od = np.arange(-(2 * r + 1), 2 * r + 2, 2)
    od = od[np.abs(od) <= 2 * np.sqrt(max_norm2)]
    pts = []
    for vals in (ev, od):
        g = np.array(list(itertools.product(vals, repeat=8)), dtype=np.int16)
        keep = is_e8(g) & ((g.astype(np.int32) ** 2).sum(1) <= 4 * max_norm2)
        pts.append(g[keep])
    return np.concatenate(pts).astype(np.int8)


def norm2(y: np.ndarray) -> np.ndarray:
    """|x|^2 for y = 2x, as an exact integer (sum y^2 / 4)."""
    s = (np.asarray(y, dtype=np.int64) ** 2).sum(axis=-1)
    return s // 4


def orbit_size(y: np.ndarray) -> np.ndarray:
    """Number of points sharing this vector of absolute values (R3)."""
    a = np.abs(np.asarray(y, dtype=np.int64))
    half = (a[..., 0] % 2) == 1
    nnz = (a != 0).sum(axis=-1)
    return np.where(half, 128, 2 ** nnz)


def sign_counter(y: np.ndarray) -> np.ndarray:
    """The sign counter j of R3."""
    y = np.asarray(y, dtype=np.int64)
    a = np.abs(y)
    neg = (y < 0).astype(np.int64)
    half = (a[:, 0] % 2) == 1
    j = np.zeros(len(y), dtype=np.int64)
    rank = np.cumsum(a != 0, axis=1) - 1           # rank among nonzeros
    half_pos = {0: 0, 1: 1, 2: 2, 4: 3, 5: 4, 6: 5, 7: 6}    # coordinate -> bit; x4 (c = 3) by parity
    for c in range(8):
        int_bit = np.where(a[:, c] != 0, neg[:, c] << np.maximum(rank[:, c], 0), 0)
        half_bit = (neg[:, c] << half_pos[c]) if c in half_pos else np.zeros(len(y), dtype=np.int64)
        j += np.where(half, half_bit, int_bit)
    return j


def order_key_sort(y: np.ndarray) -> np.ndarray:
    """Permutation sorting points by the R3 key."""
    y = np.asarray(y, dtype=np.int64)
    a = np.abs(y)
    keys = [sign_counter(y)]
    keys += [a[:, c] for c in range(7, -1, -1)]   # lexsort: last key is primary
    keys += [a.max(axis=1), -orbit_size(y), norm2(y)]
    return np.lexsort(keys)


@functools.lru_cache(maxsize=1)
def codebook() -> np.ndarray:
    """C as y = 2x, int8 [65536, 8], index = position in the stated order."""
    pts = enumerate_shells(12)
    pts = pts[order_key_sort(pts)]
    if len(pts) < CODEBOOK_SIZE:
        raise AssertionError("not enough points in the first 7 shells")
    cb = np.ascontiguousarray(pts[:CODEBOOK_SIZE])
    cb.setflags(write=False)
    return cb


def codebook_f64() -> np.ndarray:
    """C as float64 coordinates x = y / 2."""
    return codebook().astype(np.float64) / 2.0


def _pack_key(y: np.ndarray) -> np.ndarray:
    """Injective int64 key of a doubled-coordinate point (|y_i| <= 127)."""
    b = (np.asarray(y, dtype=np.int64) + 128) & 0xFF
    k = np.zeros(b.shape[:-1], dtype=np.int64)
    for c in range(8):
        k |= b[..., c] << (8 * c)
    return k


@functools.lru_cache(maxsize=4)
def _lookup(size: int):
    tab = codebook()[:size]
    keys = _pack_key(tab).astype(np.uint64)
    order = np.argsort(keys, kind="stable")
    return keys[order], order


def index_of(y: np.ndarray, size: int = CODEBOOK_SIZE) -> np.ndarray:
    """Index of each point in the first `size` codebook entries, or -1."""
    skeys, order = _lookup(size)
    k = _pack_key(y).astype(np.uint64)
    pos = np.searchsorted(skeys, k)
    pos_c = np.minimum(pos, len(skeys) - 1)
    hit = skeys[pos_c] == k
    return np.where(hit, order[pos_c], -1)


# --------------------------------------------------------------------------
# Closest lattice point (Conway & Sloane, "Sphere Packings, Lattices and
# Groups", chapter 20: decoders for D_n and E8 = D8 u (D8 + 1/2)), credited
# by [glq] "Acknowledgments". Used only as an exact prefilter: a point is
# returned as "certain" when it is the unique nearest lattice point with a
# margin, so that if it lies in the codebook it is also the unique nearest
# codebook point.
# --------------------------------------------------------------------------

_EPS = 1e-9


def _closest_dn(x: np.ndarray):
    """Nearest D8 point (integer coordinates, even sum) to each row of x.

    Round every coordinate; if the sum is odd, move the coordinate with the
    largest rounding error to its other neighbour. Returns (point, certain).
    """
    f = np.rint(x)
    d = x - f
    ad = np.abs(d)
    certain = np.all(np.abs(ad - 0.5) > _EPS, axis=1)          # no rounding tie
    odd = (f.sum(axis=1) % 2) != 0
    worst = np.argmax(ad, axis=1)
    srt = np.sort(ad, axis=1)
    uniq_worst = (srt[:, -1] - srt[:, -2]) > _EPS
    certain &= ~odd | uniq_worst
    rows = np.nonzero(odd)[0]
    c = worst[rows]
    step = np.where(d[rows, c] >= 0, 1.0, -1.0)
    g = f.copy()
    g[rows, c] += step
    return g, certain


def closest_e8(x: np.ndarray):
    """Nearest E8 point to each row of x (float64 [G, 8]).

    Returns (y = 2*point as int64, squared distance, certain).
    """
    x = np.asarray(x, dtype=np.float64)
    a, ca = _closest_dn(x)
    b, cb = _closest_dn(x - 0.5)
    b = b + 0.5
    da = ((x - a) ** 2).sum(axis=1)
    db = ((x - b) ** 2).sum(axis=1)
    use_b = db < da
    pt = np.where(use_b[:, None], b, a)
    dist = np.where(use_b, db, da)
    certain = np.where(use_b, cb, ca) & (np.abs(da - db) > _EPS)
    return np.rint(2.0 * pt).astype(np.int64), dist, certain
