"""Entropy-coded E8 lattice weights of the oracle (the EntroPack scheme).

TEST INFRASTRUCTURE ONLY: see the package header; the library never imports
this module.

[entropack] first and second paragraphs: rows are normalised, quantised to
the E8 lattice, and the lattice coordinates are entropy coded under a
conditional probability model; the coded coordinates are split into
independently decodable blocks; a GPU decodes the symbols and rebuilds the
weights in one fused step; the storage rate is set freely (non-integer)
and reported with metadata as actual_bpp. The page gives no formulas.
Readings of what the page leaves open:

R20 Quantiser: s_r per row as in R16, X = W~ / s_r, y = the nearest point
    of the whole (untruncated) E8 lattice to X / step (Conway & Sloane's
    decoder with the tie rules of oracle.e8.closest_e8), kept doubled:
    z = 2y in Z^8, all entries of one parity b, sum divisible by 4.
    Weight: w = fl32(e_r * (z / 2)) with e_r = fl32(step * s_r); bf16 =
    round-to-nearest-even of w. The step sets the rate.
R21 Conditional model, 8 symbols per group: z_1 itself (table 0, it fixes
    b = z_1 mod 2); (z_c - b) / 2 for c = 2..7 (table 1 + b); (z_8 - t) / 4
    for the last, with t = (-(z_1 + ... + z_7)) mod 4, the only residue
    the lattice allows (table 3 + b). Static per-layer frequencies of each
    table, normalised to M = 2^11: every symbol seen gets
    1 + floor(c_s (M - nz) / N), the remainder goes one each to the symbols
    with the largest c_s (M - nz) mod N (ties: smaller value first).
    Values span at most 256 per table.
R22 Coder: range asymmetric numeral systems (Duda, "Asymmetric numeral
    systems", 2013), 32-bit state in [2^16, 2^32), 16-bit words,
    precision 11 bits: encoding s from x emits the low 16 bits while
    x >= f_s 2^21, then x <- (x div f_s) 2^11 + (x mod f_s) + c_s; decoding
    takes slot = x mod 2^11, the s with c_s <= slot < c_s + f_s,
    x <- f_s (x >> 11) + slot - c_s, and reads one word if x < 2^16. (11
    bits cost about 0.1% of code length against 12 and halve the decoder's
    tables.)
R23 Blocks: groups in row-major order (row r, group q); blocks of 64 P
    consecutive groups (P groups per lane; the last block may be short).
    Group j of a block belongs to lane j mod 64 as its (j div 64)-th group.
    The 64 lanes decode in lockstep, symbol c of their p-th group at step
    8p + c; the words a step needs are taken from the block's one word
    stream in increasing lane order. Stored per block: the 64 start states
    (2^16 for a lane with no group) and the word offset of its stream.
R24 actual_bpp counts every stored byte: 2 per word, 4 per state, 4 per
    block offset (plus one), the model (5 x (4 + 4) header bytes and 2 per
    frequency entry), 4 per row scale, 4 for the step, and the two sign
    vectors at one bit per entry.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import e8, glq, rht

M_BITS = 11
M = 1 << M_BITS
L = 1 << 16
LANES = 64
NTAB = 5
MAX_SYMS = 256


# --------------------------------------------------------------------------
# quantiser (R20) and symbols (R21)
# --------------------------------------------------------------------------

def quantise_lattice(w: np.ndarray, sign_n: np.ndarray, sign_k: np.ndarray, step: float):
    """z [n, k/8, 8] int64 (doubled nearest E8 points) and s_r [n] float32."""
    wt = rht.rotate_weights(w, sign_n, sign_k)
    n, k = wt.shape
    if k % 8:
        raise ValueError("k must be a multiple of 8")
    s = glq.row_scales(wt)
    x = (wt / s.astype(np.float64)[:, None]) / np.float64(np.float32(step))
    z, _, _ = e8.closest_e8(x.reshape(-1, 8))
    return z.reshape(n, k // 8, 8), s


def weights_f32(z: np.ndarray, row_scale: np.ndarray, step: float) -> np.ndarray:
    """w = fl32(e_r * (z / 2)), e_r = fl32(step * s_r) (R20); [n, k] float32."""
    n, g, _ = z.shape
    e = np.float32(step) * np.asarray(row_scale, dtype=np.float32)
    half = (np.asarray(z, dtype=np.float64) / 2.0).astype(np.float32)      # exact
    return (e[:, None, None] * half).reshape(n, g * 8)


def symbol_values(z: np.ndarray):
    """Per group the 8 (table, value) pairs of R21: tabs, vals [G, 8]."""
    z = np.asarray(z, dtype=np.int64).reshape(-1, 8)
    b = z[:, 0] & 1
    vals = np.empty_like(z)
    tabs = np.empty_like(z)
    vals[:, 0] = z[:, 0]
    tabs[:, 0] = 0
    vals[:, 1:7] = (z[:, 1:7] - b[:, None]) // 2
    tabs[:, 1:7] = (1 + b)[:, None]
    t = (-z[:, :7].sum(axis=1)) % 4
    vals[:, 7] = (z[:, 7] - t) // 4
    tabs[:, 7] = 3 + b
    return tabs, vals


def values_to_z(tabs_unused, vals: np.ndarray) -> np.ndarray:
    """Inverse of symbol_values: rebuild z [G, 8] from the 8 values."""
    vals = np.asarray(vals, dtype=np.int64).reshape(-1, 8)
    z = np.empty_like(vals)
    z[:, 0] = vals[:, 0]
    b = z[:, 0] & 1
    z[:, 1:7] = 2 * vals[:, 1:7] + b[:, None]
    t = (-z[:, :7].sum(axis=1)) % 4
    z[:, 7] = 4 * vals[:, 7] + t
    return z


# --------------------------------------------------------------------------
# model (R21)
# --------------------------------------------------------------------------

def normalise_counts(counts: np.ndarray) -> np.ndarray:
    """Frequencies summing to M with every seen symbol >= 1 (R21)."""
    c = np.asarray(counts, dtype=np.int64)
    nz = int((c > 0).sum())
    f = np.zeros(len(c), dtype=np.int64)
    if nz == 0:
        return f
    tot = int(c.sum())
    seen = c > 0
    f[seen] = 1 + (c[seen] * (M - nz)) // tot
    rem = M - int(f.sum())
    frac = (c * (M - nz)) % tot
    order = sorted(np.nonzero(seen)[0], key=lambda s: (-int(frac[s]), int(s)))
    for s in order[:rem]:
        f[s] += 1
    assert f.sum() == M
    return f


@dataclass
class Model:
    vmin: np.ndarray      # int64 [5]
    freq: list            # 5 int64 arrays (length = table span, 0 for an empty table)

    def cum(self, t):
        return np.concatenate([[0], np.cumsum(self.freq[t])[:-1]]) if len(self.freq[t]) else np.zeros(0, np.int64)

    def stored_bytes(self) -> int:
        return NTAB * 8 + 2 * sum(len(f) for f in self.freq)


def build_model(tabs: np.ndarray, vals: np.ndarray) -> Model:
    vmin = np.zeros(NTAB, dtype=np.int64)
    freq = []
    for t in range(NTAB):
        v = vals[tabs == t]
        if v.size == 0:
            freq.append(np.zeros(0, dtype=np.int64))
            continue
        lo, hi = int(v.min()), int(v.max())
        if hi - lo + 1 > MAX_SYMS:
            raise ValueError("a symbol table spans more than 256 values: step too small for these weights")
        vmin[t] = lo
        freq.append(normalise_counts(np.bincount(v - lo, minlength=hi - lo + 1)))
    return Model(vmin, freq)


# --------------------------------------------------------------------------
# coder (R22) and blocks (R23)
# --------------------------------------------------------------------------

@dataclass
class Stream:
    n: int
    k: int
    lane_groups: int
    step: np.float32
    row_scale: np.ndarray     # float32 [n]
    model: Model
    states: np.ndarray        # uint32 [nblocks, 64]
    offsets: np.ndarray       # uint32 [nblocks + 1], in words
    words: np.ndarray         # uint16

    @property
    def nblocks(self) -> int:
        return len(self.offsets) - 1


def _lane_schedule(ng: int):
    """For a block of ng groups: per step (p, c) the lanes in lockstep order."""
    pmax = (ng + LANES - 1) // LANES
    for p in range(pmax):
        lanes = [l for l in range(LANES) if p * LANES + l < ng]
        for c in range(8):
            yield p, c, lanes


def encode_block(tabs: np.ndarray, vals: np.ndarray, model: Model):
    """rANS-encode one block (tabs/vals [ng, 8]). Returns (states [64], words)."""
    ng = len(vals)
    cums = [model.cum(t) for t in range(NTAB)]
    x = [L] * LANES
    out = []
    for p, c, lanes in reversed(list(_lane_schedule(ng))):
        for lane in reversed(lanes):
            j = p * LANES + lane
            t = int(tabs[j, c])
            s = int(vals[j, c] - model.vmin[t])
            f = int(model.freq[t][s])
            cs = int(cums[t][s])
            xs = x[lane]
            while xs >= f << (32 - M_BITS):
                out.append(xs & 0xFFFF)
                xs >>= 16
            x[lane] = ((xs // f) << M_BITS) + (xs % f) + cs
    return np.array(x, dtype=np.uint32), np.array(out[::-1], dtype=np.uint16)


def decode_block(ng: int, states: np.ndarray, words: np.ndarray, model: Model):
    """Decode one block of ng groups; returns vals [ng, 8] and the words used."""
    cums = [model.cum(t) for t in range(NTAB)]
    x = [int(v) for v in states]
    pos = 0
    vals = np.zeros((ng, 8), dtype=np.int64)
    for p, c, lanes in _lane_schedule(ng):
        for lane in lanes:
            j = p * LANES + lane
            if c == 0:
                t = 0
            else:
                b = int(vals[j, 0]) & 1
                t = (1 if c < 7 else 3) + b
            slot = x[lane] & (M - 1)
            cum = cums[t]
            s = int(np.searchsorted(cum, slot, side="right")) - 1
            f = int(model.freq[t][s])
            x[lane] = f * (x[lane] >> M_BITS) + slot - int(cum[s])
            vals[j, c] = s + int(model.vmin[t])
        for lane in lanes:          # renormalisation, in lane order
            if x[lane] < L:
                x[lane] = (x[lane] << 16) | int(words[pos])
                pos += 1
    if any(v != L for v in x):
        raise ValueError("stream does not end in the start state")
    return vals, pos


def encode(w: np.ndarray, sign_n: np.ndarray, sign_k: np.ndarray, step: float,
           lane_groups: int = 32) -> Stream:
    """Quantise (R20), model (R21) and code (R22, R23) a layer."""
    if lane_groups < 1:
        raise ValueError("lane_groups must be positive")
    z, s = quantise_lattice(w, sign_n, sign_k, step)
    n, g, _ = z.shape
    tabs, vals = symbol_values(z)
    model = build_model(tabs, vals)
    bg = LANES * lane_groups
    total = n * g
    nb = (total + bg - 1) // bg
    states = np.zeros((nb, LANES), dtype=np.uint32)
    offsets = np.zeros(nb + 1, dtype=np.uint32)
    chunks = []
    for b in range(nb):
        sl = slice(b * bg, min(total, (b + 1) * bg))
        st, wd = encode_block(tabs[sl], vals[sl], model)
        states[b] = st
        chunks.append(wd)
        offsets[b + 1] = offsets[b] + len(wd)
    words = np.concatenate(chunks) if chunks else np.zeros(0, np.uint16)
    return Stream(n, 8 * g, lane_groups, np.float32(step), s, model, states, offsets, words)


def decode_z(st: Stream) -> np.ndarray:
    """Lossless decode of every block: z [n, k/8, 8]."""
    g = st.k // 8
    total = st.n * g
    bg = LANES * st.lane_groups
    vals = np.zeros((total, 8), dtype=np.int64)
    for b in range(st.nblocks):
        lo, hi = b * bg, min(total, (b + 1) * bg)
        v, used = decode_block(hi - lo, st.states[b], st.words[st.offsets[b]:st.offsets[b + 1]], st.model)
        if used != st.offsets[b + 1] - st.offsets[b]:
            raise ValueError("block did not use its whole word stream")
        vals[lo:hi] = v
    return values_to_z(None, vals).reshape(st.n, g, 8)


def code_length_bits(tabs: np.ndarray, vals: np.ndarray, model: Model) -> float:
    """Ideal code length sum_s -log2(f_s / M) of the symbols under the model."""
    bits = 0.0
    for t in range(NTAB):
        v = vals[tabs == t]
        if v.size:
            f = model.freq[t][v - model.vmin[t]].astype(np.float64)
            bits += float(np.sum(M_BITS - np.log2(f)))
    return bits


def actual_bpp(st: Stream) -> float:
    """R24: every stored byte per weight, times 8."""
    b = (2 * len(st.words) + 4 * st.states.size + 4 * len(st.offsets) + st.model.stored_bytes()
         + 4 * st.n + 4 + (st.n + 7) // 8 + (st.k + 7) // 8)
    return 8.0 * b / (st.n * st.k)


def serialise_stream(st: Stream, sign_n: np.ndarray, sign_k: np.ndarray) -> bytes:
    """Every stored byte of a coded layer, in one buffer: start states
    (uint32), block offsets (uint32), the model (per table int32 vmin and
    int32 span, then the uint16 frequencies of every table), the float32
    row scales and step, the sign vectors at one bit per entry (bit set =
    -1), then the words (uint16); all little-endian. The shape (n, k) and
    the groups per lane travel beside the buffer, as a tensor header would
    carry them."""
    spans = [len(f) for f in st.model.freq]
    hdr = np.empty(2 * NTAB, dtype="<i4")
    hdr[0::2] = st.model.vmin
    hdr[1::2] = spans
    parts = [np.ascontiguousarray(st.states, dtype="<u4").tobytes(),
             np.ascontiguousarray(st.offsets, dtype="<u4").tobytes(),
             hdr.tobytes()]
    parts += [np.asarray(f, dtype="<u2").tobytes() for f in st.model.freq]
    parts.append(np.asarray(st.row_scale, dtype="<f4").tobytes())
    parts.append(np.asarray([st.step], dtype="<f4").tobytes())
    for sg in (sign_n, sign_k):
        parts.append(np.packbits(np.asarray(sg) < 0, bitorder="little").tobytes())
    parts.append(np.ascontiguousarray(st.words, dtype="<u2").tobytes())
    return b"".join(parts)


def deserialise_stream(blob: bytes, n: int, k: int, lane_groups: int):
    """Inverse of serialise_stream: (Stream, sign_n, sign_k). Raises
    ValueError when the buffer is not exactly one coded layer long."""
    pos = 0

    def take(count, dtype):
        nonlocal pos
        size = count * np.dtype(dtype).itemsize
        if pos + size > len(blob):
            raise ValueError("buffer too short")
        a = np.frombuffer(blob, dtype=dtype, count=count, offset=pos)
        pos += size
        return a

    total = n * (k // 8)
    nb = -(-total // (LANES * lane_groups))
    states = take(nb * LANES, "<u4").astype(np.uint32).reshape(nb, LANES)
    offsets = take(nb + 1, "<u4").astype(np.uint32)
    hdr = take(2 * NTAB, "<i4").astype(np.int64)
    freq = [take(int(hdr[2 * t + 1]), "<u2").astype(np.int64) for t in range(NTAB)]
    model = Model(hdr[0::2].copy(), freq)
    row_scale = take(n, "<f4").astype(np.float32)
    step = np.float32(take(1, "<f4")[0])
    signs = []
    for length in (n, k):
        bits = np.unpackbits(take((length + 7) // 8, np.uint8), bitorder="little")[:length]
        signs.append(np.where(bits == 1, -1, 1).astype(np.int8))
    words = take(int(offsets[-1]), "<u2").astype(np.uint16)
    if pos != len(blob):
        raise ValueError("trailing bytes")
    return Stream(n, k, lane_groups, step, row_scale, model, states, offsets, words), signs[0], signs[1]
