"""CPU model of the row transform's wave stages (no GPU): one wave holds a
1024-element Hadamard block, 16 registers a lane. It replays the kernel's
register butterflies, its four DPP lane stages (partners lane ^ 1, ^ 2, ^ 7 and
^ 8 over the relabelled lane l ^ 3 [bit 2 of l], the upper lane keeping the
negated difference) and its two lane-swap stages (the gfx950 permlane16 /
permlane32 swaps of a register pair), in both forms the kernels use: the
pair (p, p + 1) swapped back after the butterfly, and the pair (p, p + 8)
left in place, whose results land at the elements rb_elem_out names. Either
must give the orthonormal Sylvester transform H x / 32 once each value is
placed at its element and multiplied by its lane's sign factor."""
import numpy as np
from scipy.linalg import hadamard


def ell(l):
    return l ^ (((l >> 2) & 1) * 3)


def lane_sign(l):
    return -1.0 if bin(ell(l) & 15).count("1") & 1 else 1.0


def swap16(d, s):
    # odd 16-lane rows of d trade places with even rows of s
    nd, ns = d.copy(), s.copy()
    for l in range(64):
        if (l >> 4) & 1:
            nd[l] = s[l - 16]
        else:
            ns[l] = d[l + 16]
    return nd, ns


def swap32(d, s):
    # the upper 32 lanes of d trade places with the lower 32 of s
    nd, ns = d.copy(), s.copy()
    for l in range(64):
        if l >= 32:
            nd[l] = s[l - 32]
        else:
            ns[l] = d[l + 32]
    return nd, ns


def wave_transform(x, keep):
    v = np.zeros((16, 64))
    for l in range(64):
        for i in range(16):
            v[i, l] = x[8 * ell(l) + (i & 7) + 512 * (i >> 3)]
    for s in range(4):
        for i in range(16):
            if not i & (1 << s):
                a, b = v[i].copy(), v[i + (1 << s)].copy()
                v[i], v[i + (1 << s)] = a + b, a - b
    partners = [lambda l: l ^ 1, lambda l: l ^ 2, lambda l: (l & ~7) | (7 - (l & 7)),
                lambda l: (l & ~15) | ((l + 8) & 15)]
    for j, perm in enumerate(partners):
        s = np.array([-1.0 if (ell(l) >> j) & 1 else 1.0 for l in range(64)])
        v = v + s[None, :] * v[:, [perm(l) for l in range(64)]]
    for sw in (swap16, swap32):
        if keep:
            for p in range(8):
                a, b = sw(v[p], v[p + 8])
                v[p], v[p + 8] = a + b, a - b
        else:
            for p in range(0, 16, 2):
                a, b = sw(v[p], v[p + 1])
                v[p], v[p + 1] = sw(a + b, a - b)
    y = np.full(1024, np.nan)
    for l in range(64):
        for i in range(16):
            if keep:
                e = ((i & 7) | ((ell(l) & 15) << 3) | (((l >> 5) & 1) << 7) | (((i >> 3) & 1) << 8)
                     | (((l >> 4) & 1) << 9))
            else:
                q = 16 * l + i
                e = (q & 7) | (((q >> 3) & 1) << 9) | (ell((q >> 4) & 63) << 3)
            assert np.isnan(y[e])                   # every element exactly once
            y[e] = v[i, l] * lane_sign(l) / 32.0
    return y


def test_wave_stages_give_the_hadamard_transform():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(1024)
    ref = hadamard(1024) @ x / 32.0
    for keep in (False, True):
        assert np.allclose(wave_transform(x, keep), ref, rtol=0, atol=1e-12)


def test_kept_layout_stores_whole_16_byte_pieces():
    # registers 8 h .. 8 h + 7 of a lane are 8 consecutive elements, and the
    # 16 lanes of a row cover 128 consecutive elements for each register half
    for l in range(64):
        for h in range(2):
            e0 = ((ell(l) & 15) << 3) | (((l >> 5) & 1) << 7) | (h << 8) | (((l >> 4) & 1) << 9)
            assert e0 % 8 == 0
    for row in range(4):
        starts = sorted(((ell(l) & 15) << 3) | (((l >> 5) & 1) << 7) | (((l >> 4) & 1) << 9)
                        for l in range(16 * row, 16 * row + 16))
        assert starts == list(range(starts[0], starts[0] + 128, 8))

