"""Encode, decode and the layer reference of the oracle.

[glq] "How it works" (item 1: 16-bit E8 index per 8-weight group; 3/4 bpw
add a second-stage residual codebook of 8 or 16 bits), "Bit widths" (global
scale only, no group size), "Results" (sizes equal the nominal rate).
Readings of what the pages leave open:

R7  Global scale s = fp32(sqrt(mean(W~^2))), computed in float64 and rounded
    once; s = 1 when W~ is identically zero.
R8  Groups are 8 consecutive weights along the input axis of W~ [n, k]:
    group (r, g) = W~[r, 8g:8g+8]; k must be a multiple of 8. X = W~ / s.
R9  Stage-1 index i1 = argmin_i |X - C[i]|^2 in float64; lowest index on
    exact ties.
R10 Residual (3/4 bpw): greedy second stage R = X - C[i1],
    i2 = argmin_j |R - 2^-k C_r[j]|^2, with C_r = the first 2^bits entries
    of the same ordered codebook (bits = 8 or 16) and k = 1 (8-bit) or
    k = 2 (16-bit). One stored scale remains: 2^-k is fixed by bpw.
R11 Decode: v = C[i1] + 2^-k C_r[i2] (exact in float32), then one IEEE
    float32 multiply w32 = fl32(s * v), and bf16 = round-to-nearest-even of
    w32. Output [n, k] row-major in the rotated basis.
R12 Layer reference in float64: y = U^T (W32 (V x)) with W32 the float32
    decoded weights (exact in float64) and x as given.
R16 Per-row scales ("EntroPack", first paragraph: per-row normalized E8
    quantization; no formula given): s_r = fp32(sqrt(mean_j W~[r, j]^2)) per
    output row, X[r] = W~[r] / s_r, the same index search; a row's weights
    decode as fl32(s_r' * v) with s_r' = fl32(scale * s_r) when a global
    scale multiplies too.
"""
from __future__ import annotations

import numpy as np
import scipy.spatial

from . import e8, rht

RESID_BITS = {3: 8, 4: 16}
RESID_SHIFT = {3: 1, 4: 2}


# --------------------------------------------------------------------------
# scale and grouping
# --------------------------------------------------------------------------

def global_scale(wt: np.ndarray) -> np.float32:
    """R7: s = fp32(sqrt(mean(W~^2)))."""
    wt = np.asarray(wt, dtype=np.float64)
    if not np.all(np.isfinite(wt)):
        raise ValueError("non-finite weights")
    ms = np.mean(wt * wt)
    if ms == 0.0:
        return np.float32(1.0)
    return np.float32(np.sqrt(ms))


def row_scales(wt: np.ndarray) -> np.ndarray:
    """Per-row normalisation (EntroPack page, first paragraph: "per-row
    normalized E8"; the page gives no formula, reading R16): s_r =
    fp32(sqrt(mean_j W~[r, j]^2)) for each output row r, 1 for a zero row."""
    wt = np.asarray(wt, dtype=np.float64)
    if not np.all(np.isfinite(wt)):
        raise ValueError("non-finite weights")
    ms = np.mean(wt * wt, axis=1)
    out = np.sqrt(ms).astype(np.float32)
    out[ms == 0.0] = np.float32(1.0)
    return out


def groups(wt: np.ndarray) -> np.ndarray:
    """R8: view W~ [n, k] as groups [n, k/8, 8]."""
    n, k = wt.shape
    if k % 8:
        raise ValueError("k must be a multiple of 8")
    return np.asarray(wt, dtype=np.float64).reshape(n, k // 8, 8)


# --------------------------------------------------------------------------
# nearest neighbour (R9)
# --------------------------------------------------------------------------

def nearest_bruteforce(x: np.ndarray, size: int = e8.CODEBOOK_SIZE) -> np.ndarray:
    """argmin_i sum_c (x_c - C[i]_c)^2 over the first `size` entries, float64,
    lowest index on exact ties. The definition itself; use on small inputs."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, 8)
    cb = e8.codebook_f64()[:size]
    out = np.empty(len(x), dtype=np.int64)
    step = max(1, (1 << 22) // size)
    for s in range(0, len(x), step):
        d = ((x[s:s + step, None, :] - cb[None, :, :]) ** 2).sum(axis=2)
        out[s:s + step] = np.argmin(d, axis=1)       # first minimum = lowest index
    return out


_TREES = {}


def _tree(size: int):
    t = _TREES.get(size)
    if t is None:
        t = scipy.spatial.cKDTree(e8.codebook_f64()[:size])
        _TREES[size] = t
    return t


def nearest(x: np.ndarray, size: int = e8.CODEBOOK_SIZE, workers: int = -1) -> np.ndarray:
    """Same result as nearest_bruteforce, faster.

    1. Conway-Sloane closest lattice point; if it is certain (unique with a
       margin) and lies in the first `size` entries, it is the answer.
    2. Otherwise a k-d tree proposes the 8 nearest entries; their exact
       squared distances are recomputed as in the definition and the lowest
       index among the minima is taken, provided the 8th candidate is
       farther by a margin; if not, the definition is evaluated in full.
    """
    x = np.asarray(x, dtype=np.float64).reshape(-1, 8)
    out = np.full(len(x), -1, dtype=np.int64)
    y, _, certain = e8.closest_e8(x)
    idx = e8.index_of(y, size)
    ok = certain & (idx >= 0)
    out[ok] = idx[ok]
    rest = np.nonzero(~ok)[0]
    if len(rest):
        kk = min(8, size)
        _, cand = _tree(size).query(x[rest], k=kk, workers=workers)
        cand = np.asarray(cand).reshape(len(rest), kk)
        cb = e8.codebook_f64()
        d = ((x[rest, None, :] - cb[cand]) ** 2).sum(axis=2)
        dmin = d.min(axis=1)
        is_min = d == dmin[:, None]
        best = np.where(is_min, cand, np.iinfo(np.int64).max).min(axis=1)
        safe = (d.max(axis=1) - dmin > 1e-9) if kk < size else np.ones(len(rest), bool)
        out[rest] = best
        unsafe = rest[~safe]
        if len(unsafe):
            out[unsafe] = nearest_bruteforce(x[unsafe], size)
    return out


# --------------------------------------------------------------------------
# encode / decode
# --------------------------------------------------------------------------

def encode(w: np.ndarray, bpw: int, sign_n: np.ndarray, sign_k: np.ndarray,
           scale: float | None = None, search=nearest, per_row: bool = False):
    """Quantise W [n, k] (original basis). Returns (idx1 u16, idx2 | None, s).

    W~ = U W V^T (R6); s per R7 unless given; X = W~/s grouped per R8;
    stage 1 per R9; for 3/4 bpw the residual stage per R10. per_row: s is the
    float32 vector of row scales (R16) and row r is divided by s[r].
    """
    if bpw not in (2, 3, 4):
        raise ValueError("bpw must be 2, 3 or 4")
    wt = rht.rotate_weights(w, sign_n, sign_k)
    if per_row:
        s = row_scales(wt)
        x = groups(wt) / s.astype(np.float64)[:, None, None]
    else:
        s = global_scale(wt) if scale is None else np.float32(scale)
        x = groups(wt) / np.float64(s)
    n, g, _ = x.shape
    i1, i2, _ = quantise(x.reshape(-1, 8), bpw, search)
    idx2 = None if i2 is None else i2.reshape(n, g).astype(np.uint8 if bpw == 3 else np.uint16)
    return i1.reshape(n, g).astype(np.uint16), idx2, (s if per_row else np.float32(s))


def quantise(flat: np.ndarray, bpw: int, search=nearest):
    """The quantiser Q of one 8-vector per row of flat [G, 8] (already divided
    by the scale): stage 1 per R9, the residual stage per R10 for 3/4 bpw.
    Returns (i1 int64 [G], i2 int64 [G] | None, v float64 [G, 8]) with
    v = C[i1] + 2^-k C_r[i2], the exact decoded vector."""
    flat = np.asarray(flat, dtype=np.float64).reshape(-1, 8)
    cb = e8.codebook_f64()
    i1 = search(flat)
    v = cb[i1]
    i2 = None
    if bpw > 2:
        k = RESID_SHIFT[bpw]
        size = 1 << RESID_BITS[bpw]
        r = flat - v
        # |R - 2^-k c|^2 = 4^-k |2^k R - c|^2 : the same argmin, exactly.
        i2 = search(r * np.float64(1 << k), size=size)
        v = v + cb[i2] * (2.0 ** -k)
    return i1, i2, v


def decode_values(idx1: np.ndarray, idx2, bpw: int) -> np.ndarray:
    """v = C[i1] + 2^-k C_r[i2] (R11), float64 [n, k] (exact)."""
    cb = e8.codebook_f64()
    idx1 = np.asarray(idx1)
    n, g = idx1.shape
    v = cb[idx1.astype(np.int64)]
    if bpw > 2:
        size = 1 << RESID_BITS[bpw]
        i2 = np.asarray(idx2).astype(np.int64)
        if i2.max(initial=0) >= size:
            raise ValueError("residual index out of range")
        v = v + cb[i2] * (2.0 ** -RESID_SHIFT[bpw])
    return v.reshape(n, g * 8)


def effective_scale(scale, row_scale=None):
    """Scale of each row: the global scale, or fl32(scale * row_scale[r]) (R16)."""
    if row_scale is None:
        return np.float32(scale)
    return np.float32(scale) * np.asarray(row_scale, dtype=np.float32)


def decode_f32(idx1, idx2, bpw: int, scale) -> np.ndarray:
    """w32 = fl32(s * v): one IEEE float32 multiply per weight (R11); scale is
    one float32 or a float32 vector with one scale per row (R16)."""
    v = decode_values(idx1, idx2, bpw).astype(np.float32)   # exact
    if np.ndim(scale) == 0:
        return np.float32(scale) * v
    return np.asarray(scale, dtype=np.float32)[:, None] * v


def f32_to_bf16_bits(w32: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit pattern (uint16).
    Inputs are finite (NaN/Inf cannot arise from a finite scale)."""
    u = np.ascontiguousarray(w32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def decode_bf16_bits(idx1, idx2, bpw: int, scale) -> np.ndarray:
    return f32_to_bf16_bits(decode_f32(idx1, idx2, bpw, scale))


# --------------------------------------------------------------------------
# layer reference (R12) and size accounting
# --------------------------------------------------------------------------

def layer_reference(x: np.ndarray, idx1, idx2, bpw: int, scale,
                    sign_n: np.ndarray, sign_k: np.ndarray,
                    input_rht: bool = True, output_rht: bool = True) -> np.ndarray:
    """y = U^T (W32 (V x)) in float64 for x [m, k]; returns [m, n].

    input_rht / output_rht off give the rotated-basis forms (x already
    rotated; output left as z).
    """
    w32 = decode_f32(idx1, idx2, bpw, scale).astype(np.float64)
    x = np.asarray(x, dtype=np.float64)
    xt = rht.rht_forward(x, sign_k) if input_rht else x
    z = xt @ w32.T
    return rht.rht_transpose(z, sign_n) if output_rht else z


def compressed_bytes(n: int, k: int, bpw: int) -> int:
    """Index-plane bytes: 2 (stage 1) + 0/1/2 (residual) per 8 weights.
    [glq] "Bit widths": 16 / 16+8 / 16+16 bits per 8 weights."""
    per_group = {2: 2, 3: 3, 4: 4}[bpw]
    return (n * k // 8) * per_group


def actual_bpw(n: int, k: int, bpw: int) -> float:
    """Bits per weight including metadata: the index planes, the fp32 scale
    and the sign vectors packed one bit per entry ([entropack]: actual_bpp
    counts metadata)."""
    meta = 4 + (n + 7) // 8 + (k + 7) // 8
    return 8.0 * (compressed_bytes(n, k, bpw) + meta) / (n * k)


def serialise_layer(idx1, idx2, scale, sign_n, sign_k) -> bytes:
    """Every stored byte of a compressed layer, in one buffer: the index
    planes (little-endian uint16, then uint8 / uint16 residuals), the float32
    scale and the two sign vectors at one bit per entry (bit set = -1, bits
    little-endian within a byte). The shape and the bit width travel beside
    the buffer, as a tensor header would carry them."""
    parts = [np.ascontiguousarray(idx1, dtype="<u2").tobytes()]
    if idx2 is not None:
        i2 = np.asarray(idx2)
        parts.append(np.ascontiguousarray(i2, dtype="<u1" if i2.dtype == np.uint8 else "<u2").tobytes())
    parts.append(np.asarray([scale], dtype="<f4").tobytes())
    for sg in (sign_n, sign_k):
        parts.append(np.packbits(np.asarray(sg) < 0, bitorder="little").tobytes())
    return b"".join(parts)


def deserialise_layer(blob: bytes, n: int, k: int, bpw: int):
    """Inverse of serialise_layer: (idx1, idx2 | None, scale, sign_n, sign_k).
    Raises ValueError when the buffer is not exactly one layer long."""
    g = n * (k // 8)
    pos = 0

    def take(count, dtype):
        nonlocal pos
        size = count * np.dtype(dtype).itemsize
        if pos + size > len(blob):
            raise ValueError("buffer too short")
        a = np.frombuffer(blob, dtype=dtype, count=count, offset=pos)
        pos += size
        return a

    idx1 = take(g, "<u2").astype(np.uint16).reshape(n, k // 8)
    idx2 = None
    if bpw == 3:
        idx2 = take(g, "<u1").astype(np.uint8).reshape(n, k // 8)
    elif bpw == 4:
        idx2 = take(g, "<u2").astype(np.uint16).reshape(n, k // 8)
    scale = np.float32(take(1, "<f4")[0])
    signs = []
    for length in (n, k):
        bits = np.unpackbits(take((length + 7) // 8, np.uint8), bitorder="little")[:length]
        signs.append(np.where(bits == 1, -1, 1).astype(np.int8))
    if pos != len(blob):
        raise ValueError("trailing bytes")
    return idx1, idx2, scale, signs[0], signs[1]


def row_relative_error(y: np.ndarray, y_ref: np.ndarray) -> float:
    """The row-normalised maximum: max over output rows r of
    max|y_r - y_ref_r| / max|y_ref_r| (a row of zeros in y_ref contributes its
    absolute error). Reported beside relative_error, which a few large rows
    can dominate."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    y_ref = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
    num = np.max(np.abs(y - y_ref), axis=-1)
    den = np.max(np.abs(y_ref), axis=-1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1.0), num)))


def relative_error(y: np.ndarray, y_ref: np.ndarray) -> float:
    """max|y - y_ref| / max|y_ref| over the whole output (the tolerance
    measure for layer outputs)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.max(np.abs(y_ref))
    num = np.max(np.abs(y - y_ref))
    return float(num / den) if den > 0 else float(num)
