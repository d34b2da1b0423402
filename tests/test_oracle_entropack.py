"""Pins of the oracle's entropy-coded E8 format (EntroPack news item).

Independent checks: the quantiser against E8's Voronoi-relevant vectors (the
240 roots and 2160 norm-4 vectors, Conway & Sloane ch. 21) and against the
lattice's normalised second moment 0.0716821 (Conway & Sloane, table 2.3);
the coder by lossless round trips and by the rANS length identity (bits out
+ log2 of the final states = ideal code length + a bounded per-symbol
excess); the frequency rule by a hand-worked example.
"""
import itertools

import numpy as np
import pytest

import workloads as wl
from oracle import e8, entropack as ep, rht


def _layer(n, k, dist="normal", seed=2000):
    spec = wl.LayerSpec("ep", n, k, 2, 1, dist, "f32", "f32", 0, seed)
    return wl.weights(spec), wl.sign_n(spec), wl.sign_k(spec)


def _relevant_vectors():
    """Doubled coordinates of the 240 + 2160 Voronoi-relevant vectors of E8,
    enumerated directly from the definition (norm^2 2 and 4)."""
    cand = np.concatenate([np.array(list(itertools.product((-4, -2, 0, 2, 4), repeat=8))),
                           np.array(list(itertools.product((-3, -1, 1, 3), repeat=8)))])
    keep = (cand.sum(axis=1) % 4 == 0) & np.isin((cand * cand).sum(axis=1), (8, 16))
    return cand[keep]


_RELEVANT = None


def _rel():
    global _RELEVANT
    if _RELEVANT is None:
        _RELEVANT = _relevant_vectors()
    return _RELEVANT


def test_relevant_vector_count():
    assert len(_rel()) == 240 + 2160


@pytest.mark.parametrize("step", [0.5, 0.13])
def test_quantiser_is_nearest_lattice_point(step):
    w, sn, sk = _layer(16, 128, "student_t")
    z, s = ep.quantise_lattice(w, sn, sk, step)
    wt = rht.rotate_weights(w, sn, sk)
    x = ((wt / s.astype(np.float64)[:, None]) / np.float64(np.float32(step))).reshape(-1, 8)
    z = z.reshape(-1, 8)
    # lattice membership (doubled): one parity, sum divisible by 4
    assert np.all((z % 2) == (z[:, :1] % 2))
    assert np.all(z.sum(axis=1) % 4 == 0)
    # no relevant vector brings a point closer: the Voronoi cell test
    d0 = ((x - z / 2.0) ** 2).sum(axis=1)
    rel = _rel() / 2.0
    for i in range(0, len(x), 64):
        xi = x[i:i + 64, None, :] - z[i:i + 64, None, :] / 2.0
        d = ((xi - rel[None]) ** 2).sum(axis=2)
        assert np.all(d.min(axis=1) >= d0[i:i + 64] - 1e-12)


def test_distortion_matches_e8_second_moment():
    # fine step: per-coordinate error variance -> G(E8) * step^2 with
    # G(E8) = 0.0716821 (unit-volume cell); D8 would give 0.0766, Z^8 0.0833
    w, sn, sk = _layer(128, 1024, "normal", seed=31)
    step = 0.1
    z, s = ep.quantise_lattice(w, sn, sk, step)
    wt = rht.rotate_weights(w, sn, sk)
    x = (wt / s.astype(np.float64)[:, None])
    err = np.mean((x - z.reshape(x.shape) / 2.0 * np.float64(np.float32(step))) ** 2)
    assert abs(err / (0.0716821 * step * step) - 1.0) < 0.02


def test_symbol_values_invert():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4000, 8)) * 3.0
    z, _, _ = e8.closest_e8(x)
    tabs, vals = ep.symbol_values(z)
    assert np.array_equal(ep.values_to_z(tabs, vals), z)
    b = z[:, 0] & 1
    assert np.all(tabs[:, 0] == 0)
    assert np.all(tabs[:, 1:7] == (1 + b)[:, None]) and np.all(tabs[:, 7] == 3 + b)


def test_normalise_counts_worked_example():
    # M = 2048. counts [3, 0, 1]: nz = 2, N = 4; 1 + floor(3*2046/4) = 1535,
    # 1 + floor(2046/4) = 512, one left over; remainders 2 and 2 tie, so
    # the smaller symbol takes it: [1536, 0, 512]
    assert ep.M == 2048
    assert list(ep.normalise_counts(np.array([3, 0, 1]))) == [1536, 0, 512]
    assert list(ep.normalise_counts(np.array([0, 9, 0]))) == [0, 2048, 0]


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_normalise_counts_properties(seed):
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 1000, 200) * (rng.random(200) < 0.7)
    c[rng.integers(0, 200, 5)] = 1
    f = ep.normalise_counts(c)
    assert f.sum() == ep.M
    assert np.all((f > 0) == (c > 0))
    # more counts never fewer slots (equal counts may differ by the one slot
    # the tie rule gives the smaller value: order ties larger value first)
    o = np.lexsort((-np.arange(len(c)), c))
    assert np.all(np.diff(f[o]) >= 0)


@pytest.mark.parametrize("n,k,step,lane_groups", [(8, 64, 0.4, 1), (13, 96, 0.25, 3), (32, 256, 0.15, 8),
                                                  (5, 8, 0.3, 2)])
def test_round_trip_lossless(n, k, step, lane_groups):
    w, sn, sk = _layer(n, k, "student_t", seed=n * k)
    st = ep.encode(w, sn, sk, step, lane_groups)
    z, s = ep.quantise_lattice(w, sn, sk, step)
    assert np.array_equal(ep.decode_z(st), z)
    assert np.array_equal(st.row_scale, s)
    assert st.nblocks == -(-(n * k // 8) // (64 * lane_groups))
    assert st.offsets[-1] == len(st.words)


def test_code_length_identity():
    """Each coding step multiplies the state by M / f_s up to a factor within
    1 + 2^(b-16) (b = precision bits; the state is at least f_s 2^(16-b) when
    coded), so 16 (words) + sum log2(final / 2^16) differs from the ideal
    length sum log2(M / f_s) by at most log2(1 + 2^(b-16)) per symbol."""
    w, sn, sk = _layer(64, 512, "student_t", seed=9)
    st = ep.encode(w, sn, sk, 0.2, lane_groups=16)
    z, _ = ep.quantise_lattice(w, sn, sk, 0.2)
    tabs, vals = ep.symbol_values(z)
    ideal = ep.code_length_bits(tabs, vals, st.model)
    used = 16.0 * len(st.words) + float(np.sum(np.log2(st.states.astype(np.float64)) - 16.0))
    nsym = vals.size
    slack = nsym * np.log2(1.0 + 2.0 ** (ep.M_BITS - 16))
    assert -slack <= used - ideal <= slack
    # and in practice far tighter than the bound
    assert abs(used - ideal) < 0.002 * ideal


@pytest.mark.parametrize("n,k,step,lane_groups", [(16, 128, 0.3, 2), (7, 264, 0.5, 1), (40, 64, 0.2, 4)])
def test_actual_bpp_is_the_serialised_length(n, k, step, lane_groups):
    # actual_bpp against the length of the coded layer actually written out
    # and read back: the buffer alone (plus the shape) decodes to the same
    # lattice points, and every byte of it is counted
    w, sn, sk = _layer(n, k, "student_t", seed=n + k)
    st = ep.encode(w, sn, sk, step, lane_groups=lane_groups)
    blob = ep.serialise_stream(st, sn, sk)
    assert ep.actual_bpp(st) == 8.0 * len(blob) / (n * k)
    back, bn, bk = ep.deserialise_stream(blob, n, k, lane_groups)
    assert np.array_equal(bn, sn) and np.array_equal(bk, sk)
    assert np.array_equal(ep.decode_z(back), ep.quantise_lattice(w, sn, sk, step)[0])
    assert np.array_equal(ep.weights_f32(ep.decode_z(back), back.row_scale, back.step),
                          ep.weights_f32(ep.decode_z(st), st.row_scale, st.step))
    with pytest.raises(ValueError):
        ep.deserialise_stream(blob + b"\0", n, k, lane_groups)


def test_too_fine_step_rejected():
    w, sn, sk = _layer(4, 64, "student_t")
    with pytest.raises(ValueError):
        ep.encode(w, sn, sk, 0.004)


# ------------------------------------------------------------- exact ties ----

def test_closest_point_exact_ties_follow_stated_rule():
    # hand-derived outcomes of the decoder's tie rules (tests/golden/
    # e8_lattice_ties.txt): half-to-even rounding, parity fixed on the first
    # largest error, integer coset on equal distance
    from tie_layers import lattice_ties
    names, x, z = lattice_ties()
    y, dist, _ = e8.closest_e8(x)
    for nm, a, b in zip(names, y, z):
        assert np.array_equal(a, b), nm
    # each is a genuine tie: another lattice point is exactly as far
    rel = _rel() / 2.0
    for xi, yi, di in zip(x, y, dist):
        d = ((xi[None] - (yi / 2.0)[None] - rel) ** 2).sum(axis=1)
        assert d.min() == di


def test_quantiser_exact_ties_through_the_layer():
    # the same ties reached through the whole quantiser: exact rotation,
    # row scale exactly 1, step 1
    from tie_layers import ep_tie_rows, exact_layer, lattice_ties
    _, _, zg = lattice_ties()
    wt, pos = ep_tie_rows()
    sn = np.array([1, -1, 1], dtype=np.int8)
    sk = np.where(np.arange(48) % 3 == 1, -1, 1).astype(np.int8)
    w = exact_layer(wt * 2.0 ** -6, sn, sk)
    z, s = ep.quantise_lattice(w, sn, sk, 1.0)
    assert np.all(s == np.float32(2.0 ** -6))
    for (r, j), p in pos.items():
        assert np.array_equal(z[r, j], zg[p])
    st = ep.encode(w.astype(np.float64), sn, sk, 1.0, lane_groups=1)
    assert np.array_equal(ep.decode_z(st), z)
