"""Pins of the oracle's E8 codebook against facts independent of it:
the E8 definition (Conway & Sloane), the theta series closed form
240*sigma_3(m), hand-derived entries of the stated order, a pure-Python
re-sort of the inner shells, and brute force nearest neighbour."""
import itertools
import os

import numpy as np
import pytest

from oracle import e8, glq

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def sigma3(m):
    return sum(d ** 3 for d in range(1, m + 1) if m % d == 0)


def test_membership_examples():
    # doubled coordinates: (1,1,0..) member; (1,0,..) odd sum; (1/2)^8 member;
    # one -1/2 makes the sum 3 (odd); (-3/2,(1/2)^7) sum 2 member; mixed parity not.
    yes = [[2, 2, 0, 0, 0, 0, 0, 0], [1] * 8, [-3, 1, 1, 1, 1, 1, 1, 1], [2, -2, 0, 0, 0, 0, 0, 0]]
    no = [[2, 0, 0, 0, 0, 0, 0, 0], [1] * 7 + [-1], [3, 1, 1, 1, 1, 1, 1, 1], [1, 2, 0, 0, 0, 0, 0, 0]]
    assert e8.is_e8(np.array(yes)).all()
    assert not e8.is_e8(np.array(no)).any()


def test_theta_series_closed_form_and_golden():
    pts = e8.enumerate_shells(12)
    counts = np.bincount(e8.norm2(pts))
    gold = {int(a): int(b) for a, b in _golden("e8_theta.txt")}
    for m in range(0, 7):
        expect = 1 if m == 0 else 240 * sigma3(m)
        assert counts[2 * m] == expect == gold[2 * m]
    assert counts[1::2].sum() == 0          # E8 is even: no odd squared norms


def test_minimal_vectors_are_the_240_roots():
    pts = e8.enumerate_shells(2)
    roots = pts[e8.norm2(pts) == 2]
    assert len(roots) == 240
    # 112 of shape (+-1,+-1,0^6) and 128 of shape (+-1/2)^8 with an even number of minus signs
    integer = roots[(np.abs(roots) % 2 == 0).all(1)]
    half = roots[(np.abs(roots) % 2 == 1).all(1)]
    assert len(integer) == 112 and len(half) == 128
    assert ((half < 0).sum(1) % 2 == 0).all()


def test_codebook_basic_invariants():
    cb = e8.codebook()
    assert cb.shape == (65536, 8) and cb.dtype == np.int8
    assert e8.is_e8(cb).all()
    assert len(np.unique(e8._pack_key(cb))) == 65536          # distinct
    n2 = e8.norm2(cb)
    assert (np.diff(n2) >= 0).all()                           # shells in order
    assert np.array_equal(np.bincount(n2)[::2], [1, 240, 2160, 6720, 17520, 30240, 8655])
    assert np.abs(cb).max() == 6                              # |x_i| <= 3: 2x fits signed 4 bits
    # first 256 = origin + 240 roots + 15 points of squared norm 4
    assert np.array_equal(np.bincount(n2[:256])[::2], [1, 240, 15])


def test_codebook_hand_derived_entries():
    cb = e8.codebook()
    for row in _golden("codebook_first_entries.txt"):
        i = int(row[0])
        assert cb[i].tolist() == [int(v) for v in row[1:]], i


def _py_key(y):
    """Order key written out with plain Python, point by point."""
    a = [abs(v) for v in y]
    half = a[0] % 2 == 1
    nnz = sum(1 for v in a if v)
    size = 128 if half else 2 ** nnz
    j = 0
    if half:
        # bits 0..2: x1..x3; bits 3..6: x5..x8; x4 is fixed by the even sum
        for bit, c in enumerate((0, 1, 2, 4, 5, 6, 7)):
            if y[c] < 0:
                j |= 1 << bit
    else:
        r = 0
        for v in y:
            if v != 0:
                if v < 0:
                    j |= 1 << r
                r += 1
    return (sum(v * v for v in y), -size, max(a), tuple(a), j)


def test_order_matches_plain_python_sort_on_inner_shells():
    # all points with |x|^2 <= 4 (2401), listed by itertools and sorted by a
    # Python tuple key: must equal the codebook's first 2401 entries.
    pts = []
    for y in itertools.product(range(-4, 5), repeat=8):
        if sum(v * v for v in y) <= 16 and e8.is_e8(np.array(y)):
            pts.append(y)
    pts.sort(key=_py_key)
    assert len(pts) == 2401
    assert np.array_equal(np.array(pts), e8.codebook()[:2401])


def test_orbit_structure_of_stated_order():
    cb = e8.codebook().astype(np.int64)
    a = np.abs(cb)
    # orbit = run of equal abs vectors; sign counter counts up 0..size-1 in each
    key = e8._pack_key(a)
    starts = np.r_[0, np.nonzero(key[1:] != key[:-1])[0] + 1]
    assert len(starts) == 1439
    j = e8.sign_counter(cb)
    sizes = e8.orbit_size(cb)
    shell_start = {int(n): int(np.argmax(e8.norm2(cb) == n)) for n in range(0, 13, 2)}
    ends = np.r_[starts[1:], 65536]
    for s, e in zip(starts, ends):
        assert np.array_equal(j[s:e], np.arange(e - s))
        if e != 65536:
            assert e - s == sizes[s]                         # full orbits except the cut
        if s:
            off = s - shell_start[int(e8.norm2(cb[s:s + 1])[0])]
            assert off % sizes[s] == 0                        # aligned within its shell
    # the norm-12 points kept: all 56 orbits of (3/2^5, 1/2^3) and 1487 points
    # of (5/2, 3/2^2, 1/2^5) orbits
    sh = cb[e8.norm2(cb) == 12]
    pat = np.sort(np.abs(sh), axis=1)
    n1 = (pat == np.array([1, 1, 1, 3, 3, 3, 3, 3])).all(1).sum()
    n2 = (pat == np.array([1, 1, 1, 1, 1, 3, 3, 5])).all(1).sum()
    assert (n1, n2) == (7168, 1487)


def test_nearest_matches_bruteforce_random():
    # the fast search (Conway-Sloane prefilter, k-d tree candidates, margin
    # fallback) against the definition on 12,000 groups per run: typical
    # weights, points far outside the codebook, heavy tails; and the
    # 256-entry residual search on 4,000 more
    from oracle import cnative
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal((5000, 8)),
                        2.5 * rng.standard_normal((3000, 8)),        # many outside the codebook
                        rng.standard_t(3, (2000, 8)),
                        0.35 * rng.standard_normal((2000, 8))])     # near the origin's cell
    cb = e8.codebook_f64()
    assert np.array_equal(glq.nearest(x), cnative.nearest_bruteforce(x, cb))
    r = 1.2 * rng.standard_normal((4000, 8))
    assert np.array_equal(glq.nearest(r, size=256), cnative.nearest_bruteforce(r, cb[:256]))


def test_bruteforce_in_c_equals_numpy_definition():
    # the C loop and the numpy expression of the same definition agree,
    # exact ties included (midpoints between the origin and roots)
    from oracle import cnative
    rng = np.random.default_rng(8)
    cb = e8.codebook_f64()
    x = np.concatenate([rng.standard_normal((120, 8)), cb[1:31] / 2.0])
    assert np.array_equal(cnative.nearest_bruteforce(x, cb), glq.nearest_bruteforce(x))
    assert np.all(cnative.nearest_bruteforce(cb[1:31] / 2.0, cb) == 0)


def test_nearest_tie_rule_lowest_index():
    # midpoint of the origin and a root r: equidistant (|r|^2/4 = 1/2) from
    # index 0 and from r; the lowest index (0) must win.
    cb = e8.codebook_f64()
    for i in (1, 2, 100, 129, 200, 240):
        mid = cb[i] / 2.0
        assert glq.nearest_bruteforce(mid[None])[0] == 0
        assert glq.nearest(mid[None])[0] == 0
    # midpoint of two neighbouring codebook points away from the origin
    a, b = 241, 242
    mid = (cb[a] + cb[b]) / 2.0
    d = ((cb - mid) ** 2).sum(1)
    expect = int(np.nonzero(d == d.min())[0][0])
    assert glq.nearest(mid[None])[0] == expect == glq.nearest_bruteforce(mid[None])[0]


def test_round_trip_every_codebook_entry():
    cb = e8.codebook_f64()
    assert np.array_equal(glq.nearest(cb), np.arange(65536))
    # brute force on a sample (the definition, distance 0 is unique)
    sel = np.random.default_rng(3).choice(65536, 400, replace=False)
    assert np.array_equal(glq.nearest_bruteforce(cb[sel]), sel)


def test_conway_sloane_decoder_vs_bruteforce_and_covering_radius():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((2000, 8))
    y, dist, certain = e8.closest_e8(x)
    assert e8.is_e8(y).all()
    idx = e8.index_of(y)
    inside = certain & (idx >= 0)
    assert inside.mean() > 0.5
    bf = glq.nearest_bruteforce(x[inside])
    assert np.array_equal(bf, idx[inside])
    assert (dist <= 1.0 + 1e-12).all()          # covering radius of E8 is 1


def test_index_of_inverse_of_codebook():
    cb = e8.codebook()
    sel = np.arange(0, 65536, 97)
    assert np.array_equal(e8.index_of(cb[sel]), sel)
    assert e8.index_of(np.array([[2, 0, 0, 0, 0, 0, 0, 0]]))[0] == -1     # not in E8
    assert e8.index_of(np.array([[8, 0, 0, 0, 0, 0, 0, 0]]))[0] == -1     # beyond 7 shells
