"""ctypes binding of libglq.so (include/glq.h). Argument marshalling only.

Every computation happens in the library: the GPU entry points take device
pointers from torch tensors and the current HIP stream; the CPU entry points
(codebook tables, reference encoder) take numpy arrays. There is no fallback:
if the library is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GLQ_LIBRARY") or os.path.join(_PKG, "lib", "libglq.so")   # override: another build

GLQ_OK, GLQ_ERR_ARG, GLQ_ERR_UNSUPPORTED, GLQ_ERR_HIP, GLQ_ERR_WORKSPACE = 0, -1, -2, -3, -4
GLQ_F32, GLQ_BF16 = 0, 1
GLQ_CB_INT8_2X, GLQ_CB_DEVICE = 0, 1
FLAG_NO_INPUT_RHT, FLAG_NO_OUTPUT_RHT = 1, 2

EXPORTS = ("glq_build_codebook", "glq_encode_ref", "glq_encode_ldlq", "glq_rht_apply", "glq_decode_weights",
           "glq_fused_linear_workspace", "glq_fused_linear", "glq_fused_linear_noalloc", "glq_status_string",
           "glq_last_error",
           "glq_version", "glq_ep_encode", "glq_ep_build_lut", "glq_ep_decode_weights",
           "glq_ep_fused_linear_workspace", "glq_ep_fused_linear")
EP_LANES, EP_TABLES, EP_MAX_SYMS = 64, 5, 256
EP_LUT_BYTES = 64 + EP_TABLES * 2048 * 4

# torch's wheel bundles its own HIP runtime (libamdhip64.so, same soname as
# /opt/rocm's). Load torch first so libglq.so binds to that one runtime:
# loaded the other way round the process ends up with two HIP/HSA runtimes
# and neither sees the device.
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libglq.so not built at {LIB_PATH}: run python -m dequant_e8_codebook_amd.build")
_lib = ctypes.CDLL(LIB_PATH)

_vp, _i64, _i32, _u32, _f32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t)


class GlqLayerStruct(ctypes.Structure):
    _fields_ = [("n", _i64), ("k", _i64), ("bpw", _i32), ("resid_shift", _i32), ("scale", _f32),
                ("idx1", _vp), ("idx2", _vp), ("sign_k", _vp), ("sign_n", _vp), ("cb", _vp),
                ("row_scale", _vp)]


class EpModel(ctypes.Structure):
    _fields_ = [("vmin", ctypes.c_int32 * EP_TABLES), ("nsym", ctypes.c_int32 * EP_TABLES),
                ("freq", (ctypes.c_uint16 * EP_MAX_SYMS) * EP_TABLES)]


class EpLayerStruct(ctypes.Structure):
    _fields_ = [("n", _i64), ("k", _i64), ("lane_groups", _i32), ("step", _f32), ("row_scale", _vp),
                ("states", _vp), ("offsets", _vp), ("words", _vp), ("nwords", _i64), ("lut", _vp),
                ("sign_k", _vp), ("sign_n", _vp)]


_lib.glq_build_codebook.argtypes = [_i32, _vp, _sz, ctypes.POINTER(_sz)]
_lib.glq_encode_ref.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp, _f32, ctypes.POINTER(_f32), _vp, _vp, _i32, _vp]
_lib.glq_encode_ldlq.argtypes = [_vp, _i64, _i64, _i32, _vp, _vp, _vp, ctypes.c_double, _f32,
                                 ctypes.POINTER(_f32), _vp, _vp, _i32, _vp]
_lib.glq_rht_apply.argtypes = [_vp, _i32, _vp, _i32, _i64, _i64, _vp, _i32, _vp]
_lib.glq_decode_weights.argtypes = [ctypes.POINTER(GlqLayerStruct), _vp, _i32, _vp]
_lib.glq_fused_linear_workspace.argtypes = [ctypes.POINTER(GlqLayerStruct), _i64]
_lib.glq_fused_linear_workspace.restype = _sz
_lib.glq_fused_linear.argtypes = [ctypes.POINTER(GlqLayerStruct), _vp, _i32, _i64, _vp, _i32, _vp, _sz,
                                  _u32, _vp]
_lib.glq_fused_linear_noalloc.argtypes = [ctypes.POINTER(GlqLayerStruct), _vp, _i32, _i64, _vp, _i32, _u32, _vp]
STATIC_WS_BYTES = 32 << 20
_lib.glq_ep_encode.argtypes = [_vp, _i64, _i64, _vp, _vp, _f32, _i32, _i32, _vp, ctypes.POINTER(EpModel), _vp, _vp,
                               _vp, _i64, ctypes.POINTER(_i64)]
_lib.glq_ep_build_lut.argtypes = [ctypes.POINTER(EpModel), _vp, _sz]
_lib.glq_ep_decode_weights.argtypes = [ctypes.POINTER(EpLayerStruct), _vp, _i32, _vp]
_lib.glq_ep_fused_linear_workspace.argtypes = [ctypes.POINTER(EpLayerStruct), _i64]
_lib.glq_ep_fused_linear_workspace.restype = _sz
_lib.glq_ep_fused_linear.argtypes = [ctypes.POINTER(EpLayerStruct), _vp, _i32, _i64, _vp, _i32, _vp, _sz, _u32, _vp]
_lib.glq_status_string.argtypes = [_i32]
_lib.glq_status_string.restype = ctypes.c_char_p
_lib.glq_version.restype = _u32
_lib.glq_last_error.restype = ctypes.c_char_p
for _name in ("glq_build_codebook", "glq_encode_ref", "glq_encode_ldlq", "glq_rht_apply", "glq_decode_weights",
              "glq_fused_linear", "glq_ep_encode", "glq_ep_build_lut", "glq_ep_decode_weights",
              "glq_ep_fused_linear"):
    getattr(_lib, _name).restype = ctypes.c_int


class GlqError(RuntimeError):
    def __init__(self, status: int, what: str):
        detail = _lib.glq_last_error().decode() if status == GLQ_ERR_HIP else ""
        super().__init__(f"{what}: {status_string(status)} ({status}) {detail}".rstrip())
        self.status = status


def _check(rc: int, what: str):
    if rc != GLQ_OK:
        raise GlqError(rc, what)


def raw():
    """The ctypes library object (for tests of the C ABI itself)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.glq_status_string(status).decode()


def version() -> int:
    return int(_lib.glq_version())


# ------------------------------------------------------------------ CPU calls

def build_codebook(form: int) -> bytes:
    need = _sz(0)
    _check(_lib.glq_build_codebook(form, None, 0, ctypes.byref(need)), "glq_build_codebook")
    buf = ctypes.create_string_buffer(need.value)
    _check(_lib.glq_build_codebook(form, buf, need.value, None), "glq_build_codebook")
    return buf.raw


def codebook_doubled() -> np.ndarray:
    """int8 [65536, 8] doubled coordinates 2*C[i]."""
    return np.frombuffer(build_codebook(GLQ_CB_INT8_2X), dtype=np.int8).reshape(65536, 8).copy()


def encode_ref(w: np.ndarray, bpw: int, sign_n: np.ndarray, sign_k: np.ndarray,
               scale: float = 0.0, nthreads: int = 0, per_row: bool = False):
    """CPU encoder: returns (idx1 uint16 [n, k/8], idx2 or None, scale); with
    per_row the scale returned is the float32 vector of row scales."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    sn = np.ascontiguousarray(sign_n, dtype=np.int8)
    sk = np.ascontiguousarray(sign_k, dtype=np.int8)
    i1 = np.empty((n, max(k // 8, 0)), dtype=np.uint16)
    i2 = None
    if bpw in (3, 4):
        i2 = np.empty((n, k // 8), dtype=np.uint8 if bpw == 3 else np.uint16)
    s = _f32(0.0)
    rs = np.empty(n, dtype=np.float32) if per_row else None
    rc = _lib.glq_encode_ref(w.ctypes.data, n, k, bpw, sn.ctypes.data, sk.ctypes.data, float(scale),
                             ctypes.byref(s), i1.ctypes.data, None if i2 is None else i2.ctypes.data,
                             nthreads, None if rs is None else rs.ctypes.data)
    _check(rc, "glq_encode_ref")
    return i1, i2, (rs if per_row else np.float32(s.value))


def encode_ldlq(w: np.ndarray, bpw: int, sign_n: np.ndarray, sign_k: np.ndarray, hessian: np.ndarray,
                damp: float = 0.01, scale: float = 0.0, nthreads: int = 0, per_row: bool = False):
    """CPU encoder with LDLQ error feedback (glq_encode_ldlq); hessian is the
    float64 [k, k] Hessian over the input features. Returns what encode_ref
    returns."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    h = np.ascontiguousarray(hessian, dtype=np.float64)
    if h.shape != (k, k):
        raise ValueError(f"hessian must be [{k}, {k}]")
    sn = np.ascontiguousarray(sign_n, dtype=np.int8)
    sk = np.ascontiguousarray(sign_k, dtype=np.int8)
    i1 = np.empty((n, max(k // 8, 0)), dtype=np.uint16)
    i2 = None
    if bpw in (3, 4):
        i2 = np.empty((n, k // 8), dtype=np.uint8 if bpw == 3 else np.uint16)
    s = _f32(0.0)
    rs = np.empty(n, dtype=np.float32) if per_row else None
    rc = _lib.glq_encode_ldlq(w.ctypes.data, n, k, bpw, sn.ctypes.data, sk.ctypes.data, h.ctypes.data,
                              float(damp), float(scale), ctypes.byref(s), i1.ctypes.data,
                              None if i2 is None else i2.ctypes.data, nthreads,
                              None if rs is None else rs.ctypes.data)
    _check(rc, "glq_encode_ldlq")
    return i1, i2, (rs if per_row else np.float32(s.value))


@dataclass
class EpHost:
    """An entropy-coded layer on the host (glq_ep_encode's outputs)."""
    n: int
    k: int
    lane_groups: int
    step: float
    row_scale: np.ndarray      # float32 [n]
    model: EpModel
    states: np.ndarray         # uint32 [nblocks, 64]
    offsets: np.ndarray        # uint32 [nblocks + 1]
    words: np.ndarray          # uint16 [nwords]

    @property
    def nblocks(self) -> int:
        return len(self.offsets) - 1


def ep_encode(w: np.ndarray, sign_n: np.ndarray, sign_k: np.ndarray, step: float, lane_groups: int = 32,
              nthreads: int = 0) -> EpHost:
    """CPU encoder of the entropy-coded E8 lattice format (glq_ep_encode)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    sn = np.ascontiguousarray(sign_n, dtype=np.int8)
    sk = np.ascontiguousarray(sign_k, dtype=np.int8)
    total = n * (k // 8)
    nb = max(0, -(-total // (EP_LANES * lane_groups))) if lane_groups > 0 else 0
    rs = np.empty(n, dtype=np.float32)
    model = EpModel()
    states = np.empty((max(nb, 1), EP_LANES), dtype=np.uint32)
    offsets = np.empty(nb + 1, dtype=np.uint32)
    cap = n * k
    words = np.empty(max(cap, 1), dtype=np.uint16)
    nw = _i64(0)
    rc = _lib.glq_ep_encode(w.ctypes.data, n, k, sn.ctypes.data, sk.ctypes.data, float(step), lane_groups,
                            nthreads, rs.ctypes.data, ctypes.byref(model), states.ctypes.data, offsets.ctypes.data,
                            words.ctypes.data, cap, ctypes.byref(nw))
    _check(rc, "glq_ep_encode")
    return EpHost(n, k, lane_groups, float(np.float32(step)), rs, model, states[:nb].copy(), offsets,
                  words[:nw.value].copy())


def ep_build_lut(model: EpModel) -> np.ndarray:
    """Decode tables of a model (glq_ep_build_lut), uint8 [EP_LUT_BYTES]."""
    out = np.zeros(EP_LUT_BYTES, dtype=np.uint8)
    _check(_lib.glq_ep_build_lut(ctypes.byref(model), out.ctypes.data, out.size), "glq_ep_build_lut")
    return out


# ------------------------------------------------------------------ GPU calls

def _torch():
    import torch
    return torch


def _stream_ptr(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return GLQ_F32
    if t.dtype == torch.bfloat16:
        return GLQ_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


# ------------------------------------------------ argument checks (no launch)
# The C entry points check pointers, sizes and enums; only the caller knows
# how large each buffer is. These checks run before every GPU call so a
# wrong shape, a strided view or a host tensor raises ValueError instead of
# reaching a kernel.

def _dev_tensor(t, name, device=None, shape=None, numel=None, min_numel=None, dtypes=None):
    if t is None:
        raise ValueError(f"{name}: missing")
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name}: must be a device (cuda) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected at least {min_numel}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {dtypes}")
    return t


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check_layer(layer, need_sign_k=True, need_sign_n=True):
    torch = _torch()
    dev = layer.idx1.device if getattr(layer.idx1, "is_cuda", False) else None
    if dev is None:
        raise ValueError("idx1: must be a device (cuda) tensor")
    g = layer.k // 8
    if layer.bpw not in (2, 3, 4) or layer.k % 8 or layer.n < 1 or layer.k < 8:
        raise ValueError("layer: bad n, k or bpw")
    _dev_tensor(layer.idx1, "idx1", dev, shape=(layer.n, g), dtypes=(torch.int16,))
    if layer.bpw == 2:
        if layer.idx2 is not None:
            raise ValueError("idx2: must be None at 2 bpw")
    else:
        _dev_tensor(layer.idx2, "idx2", dev, shape=(layer.n, g),
                    dtypes=((torch.uint8,) if layer.bpw == 3 else (torch.int16,)))
    _dev_tensor(layer.cb, "cb", dev, min_numel=_codebook_bytes(), dtypes=(torch.uint8,))
    if need_sign_k:
        _dev_tensor(layer.sign_k, "sign_k", dev, numel=layer.k, dtypes=(torch.int8,))
    if need_sign_n:
        _dev_tensor(layer.sign_n, "sign_n", dev, numel=layer.n, dtypes=(torch.int8,))
    if layer.row_scale is not None:
        _dev_tensor(layer.row_scale, "row_scale", dev, numel=layer.n, dtypes=(torch.float32,))
    return dev


def _check_ep_layer(layer, need_sign_k=False, need_sign_n=False):
    torch = _torch()
    dev = layer.words.device if getattr(layer.words, "is_cuda", False) else None
    if dev is None:
        raise ValueError("words: must be a device (cuda) tensor")
    total = layer.n * (layer.k // 8)
    if layer.k % 8 or layer.n < 1 or layer.k < 8 or layer.lane_groups < 1:
        raise ValueError("layer: bad n, k or lane_groups")
    nb = -(-total // (EP_LANES * layer.lane_groups))
    _dev_tensor(layer.row_scale, "row_scale", dev, numel=layer.n, dtypes=(torch.float32,))
    _dev_tensor(layer.states, "states", dev, numel=nb * EP_LANES, dtypes=(torch.int32,))
    _dev_tensor(layer.offsets, "offsets", dev, numel=nb + 1, dtypes=(torch.int32,))
    _dev_tensor(layer.words, "words", dev, min_numel=max(8, (layer.nwords + 7) // 8 * 8), dtypes=(torch.int16,))
    _dev_tensor(layer.lut, "lut", dev, numel=EP_LUT_BYTES, dtypes=(torch.uint8,))
    if layer.words.numel() % 8 or layer.words.data_ptr() % 16:
        raise ValueError("words: must hold a multiple of 8 entries and be 16-byte aligned")
    if need_sign_k:
        _dev_tensor(layer.sign_k, "sign_k", dev, numel=layer.k, dtypes=(torch.int8,))
    if need_sign_n:
        _dev_tensor(layer.sign_n, "sign_n", dev, numel=layer.n, dtypes=(torch.int8,))
    return dev


def _check_linear_io(dev, n, k, x, y, workspace, flags):
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != k:
        raise ValueError(f"x: shape {tuple(x.shape)}, expected (m, {k})")
    m = x.shape[0]
    _dev_tensor(x, "x", dev, dtypes=(torch.float32, torch.bfloat16))
    _dev_tensor(y, "y", dev, shape=(m, n), dtypes=(torch.float32, torch.bfloat16))
    _dev_tensor(workspace, "workspace", dev)
    if workspace.data_ptr() % 256:
        raise ValueError("workspace: must be 256-byte aligned")
    if flags & ~(FLAG_NO_INPUT_RHT | FLAG_NO_OUTPUT_RHT):
        raise ValueError("flags: unknown bits")
    for t, nm in ((x, "x"), (y, "y")):
        a0, a1 = t.data_ptr(), t.data_ptr() + _nbytes(t)
        b0, b1 = workspace.data_ptr(), workspace.data_ptr() + _nbytes(workspace)
        if _nbytes(t) and a0 < b1 and b0 < a1:
            raise ValueError(f"{nm}: overlaps the workspace")
    return m


_CB_BYTES = None


def _codebook_bytes() -> int:
    global _CB_BYTES
    if _CB_BYTES is None:
        need = _sz(0)
        _check(_lib.glq_build_codebook(GLQ_CB_DEVICE, None, 0, ctypes.byref(need)), "glq_build_codebook")
        _CB_BYTES = int(need.value)
    return _CB_BYTES


def device_codebook(device="cuda"):
    """The GLQ_CB_DEVICE tables copied into a device uint8 tensor."""
    torch = _torch()
    blob = np.frombuffer(build_codebook(GLQ_CB_DEVICE), dtype=np.uint8).copy()
    return torch.from_numpy(blob).to(device)


@dataclass
class Layer:
    """Device tensors of one compressed layer, and its glq_layer struct."""
    n: int
    k: int
    bpw: int
    scale: float
    idx1: object                # torch uint16-compatible tensor [n, k/8] (stored as int16)
    idx2: object                # torch [n, k/8] uint8 / int16, or None
    sign_k: object              # torch int8 [k]
    sign_n: object              # torch int8 [n]
    cb: object                  # torch uint8 device tables
    row_scale: object = None    # torch float32 [n] per-row scales, or None

    def struct(self) -> GlqLayerStruct:
        st = self.__dict__.get("_st")
        if st is None:
            st = self._make_struct()
            self.__dict__["_st"] = st
        return st

    def _make_struct(self) -> GlqLayerStruct:
        return GlqLayerStruct(
            self.n, self.k, self.bpw, {2: 0, 3: 1, 4: 2}[self.bpw], float(self.scale),
            self.idx1.data_ptr(), 0 if self.idx2 is None else self.idx2.data_ptr(),
            0 if self.sign_k is None else self.sign_k.data_ptr(),
            0 if self.sign_n is None else self.sign_n.data_ptr(), self.cb.data_ptr(),
            0 if self.row_scale is None else self.row_scale.data_ptr())

    @staticmethod
    def from_numpy(idx1, idx2, scale, sign_n, sign_k, cb, device="cuda", row_scale=None) -> "Layer":
        """scale: one float, or a float32 vector of per-row scales (then the
        global scale is 1, unless row_scale is given separately)."""
        torch = _torch()
        if np.ndim(scale) == 1:
            scale, row_scale = 1.0, scale
        rs = None if row_scale is None else torch.from_numpy(np.ascontiguousarray(row_scale, np.float32)).to(device)
        idx1 = np.ascontiguousarray(idx1, dtype=np.uint16)
        n, g = idx1.shape
        bpw = 2 if idx2 is None else (3 if np.asarray(idx2).dtype == np.uint8 else 4)
        t1 = torch.from_numpy(idx1.view(np.int16)).to(device)
        t2 = None
        if idx2 is not None:
            a2 = np.ascontiguousarray(idx2)
            t2 = torch.from_numpy(a2 if bpw == 3 else a2.astype(np.uint16).view(np.int16)).to(device)
        sk = None if sign_k is None else torch.from_numpy(np.ascontiguousarray(sign_k, np.int8)).to(device)
        sn = None if sign_n is None else torch.from_numpy(np.ascontiguousarray(sign_n, np.int8)).to(device)
        return Layer(n, 8 * g, bpw, float(scale), t1, t2, sk, sn, cb, rs)


@dataclass
class EpLayer:
    """Device tensors of one entropy-coded layer, and its glq_ep_layer struct."""
    n: int
    k: int
    lane_groups: int
    step: float
    row_scale: object           # torch float32 [n]
    states: object              # torch int32 [nblocks, 64] (uint32 bits)
    offsets: object             # torch int32 [nblocks + 1] (uint32 bits)
    words: object               # torch int16, nwords rounded up to 8 (>= 8), 16-byte aligned (uint16 bits)
    nwords: int
    lut: object                 # torch uint8 [EP_LUT_BYTES]
    sign_k: object = None       # torch int8 [k] (the layer product only)
    sign_n: object = None       # torch int8 [n]

    def struct(self) -> EpLayerStruct:
        st = self.__dict__.get("_st")
        if st is None:
            st = EpLayerStruct(self.n, self.k, self.lane_groups, float(self.step), self.row_scale.data_ptr(),
                               self.states.data_ptr(), self.offsets.data_ptr(), self.words.data_ptr(), self.nwords,
                               self.lut.data_ptr(), 0 if self.sign_k is None else self.sign_k.data_ptr(),
                               0 if self.sign_n is None else self.sign_n.data_ptr())
            self.__dict__["_st"] = st
        return st

    @staticmethod
    def from_host(h: EpHost, device="cuda", sign_k=None, sign_n=None) -> "EpLayer":
        torch = _torch()

        def dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device)
        words = np.zeros(max(8, (len(h.words) + 7) // 8 * 8), np.uint16)    # 16-byte reads
        words[:len(h.words)] = h.words
        return EpLayer(h.n, h.k, h.lane_groups, h.step, dev(h.row_scale.astype(np.float32)),
                       dev(h.states.view(np.int32)), dev(h.offsets.view(np.int32)), dev(words.view(np.int16)),
                       len(h.words), dev(ep_build_lut(h.model)),
                       None if sign_k is None else dev(np.asarray(sign_k, np.int8)),
                       None if sign_n is None else dev(np.asarray(sign_n, np.int8)))


def fused_linear_noalloc(layer: Layer, x, y, flags: int = 0, stream=None):
    """glq_fused_linear_noalloc: the layer with the library's static per-GPU
    scratch instead of a caller workspace (no allocation in the call)."""
    dev = _check_layer(layer, not (flags & FLAG_NO_INPUT_RHT), not (flags & FLAG_NO_OUTPUT_RHT))
    torch = _torch()
    if x.dim() != 2 or x.shape[1] != layer.k:
        raise ValueError(f"x: shape {tuple(x.shape)}, expected (m, {layer.k})")
    _dev_tensor(x, "x", dev, dtypes=(torch.float32, torch.bfloat16))
    _dev_tensor(y, "y", dev, shape=(x.shape[0], layer.n), dtypes=(torch.float32, torch.bfloat16))
    if flags & ~(FLAG_NO_INPUT_RHT | FLAG_NO_OUTPUT_RHT):
        raise ValueError("flags: unknown bits")
    st = layer.struct()
    rc = _lib.glq_fused_linear_noalloc(ctypes.byref(st), x.data_ptr(), _dtype_code(x), x.shape[0], y.data_ptr(),
                                       _dtype_code(y), flags, _stream_ptr(stream))
    _check(rc, "glq_fused_linear_noalloc")
    return y


def ep_decode_weights(layer: EpLayer, out, stream=None):
    """Fused symbol decode + weight reconstruction (glq_ep_decode_weights)."""
    torch = _torch()
    dev = _check_ep_layer(layer)
    _dev_tensor(out, "out", dev, shape=(layer.n, layer.k), dtypes=(torch.float32, torch.bfloat16))
    if out.data_ptr() % 16:
        raise ValueError("out: must be 16-byte aligned")
    st = layer.struct()
    _check(_lib.glq_ep_decode_weights(ctypes.byref(st), out.data_ptr(), _dtype_code(out), _stream_ptr(stream)),
           "glq_ep_decode_weights")
    return out


def ep_workspace_bytes(layer: EpLayer, m: int) -> int:
    st = layer.struct()
    return int(_lib.glq_ep_fused_linear_workspace(ctypes.byref(st), m))


def ep_fused_linear(layer: EpLayer, x, y, workspace, flags: int = 0, stream=None):
    """y = U^T W^ (V x) on an entropy-coded layer (glq_ep_fused_linear)."""
    dev = _check_ep_layer(layer, not (flags & FLAG_NO_INPUT_RHT), not (flags & FLAG_NO_OUTPUT_RHT))
    m = _check_linear_io(dev, layer.n, layer.k, x, y, workspace, flags)
    st = layer.struct()
    rc = _lib.glq_ep_fused_linear(ctypes.byref(st), x.data_ptr(), _dtype_code(x), m, y.data_ptr(),
                                  _dtype_code(y), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                  flags, _stream_ptr(stream))
    _check(rc, "glq_ep_fused_linear")
    return y


def rht_apply(inp, out, signs, transpose: bool, stream=None):
    """out = RHT(inp) along the last axis (glq_rht_apply)."""
    torch = _torch()
    if inp.dim() < 1 or inp.shape[-1] < 1:
        raise ValueError("inp: needs a last axis of length >= 1")
    n = inp.shape[-1]
    rows = inp.numel() // n
    dev = _dev_tensor(inp, "inp", dtypes=(torch.float32, torch.bfloat16)).device
    _dev_tensor(out, "out", dev, shape=tuple(inp.shape), dtypes=(torch.float32, torch.bfloat16))
    _dev_tensor(signs, "signs", dev, numel=n, dtypes=(torch.int8,))
    if out.data_ptr() != inp.data_ptr() and _nbytes(inp) and _nbytes(out):
        a0, a1 = inp.data_ptr(), inp.data_ptr() + _nbytes(inp)
        b0, b1 = out.data_ptr(), out.data_ptr() + _nbytes(out)
        if a0 < b1 and b0 < a1:
            raise ValueError("out: partly overlaps inp (only the same buffer is allowed)")
    if out.data_ptr() == inp.data_ptr() and out.dtype != inp.dtype:
        raise ValueError("out: in place needs the same dtype")
    rc = _lib.glq_rht_apply(inp.data_ptr(), _dtype_code(inp), out.data_ptr(), _dtype_code(out), rows, n,
                            signs.data_ptr(), int(bool(transpose)), _stream_ptr(stream))
    _check(rc, "glq_rht_apply")
    return out


def decode_weights(layer: Layer, out, stream=None):
    """W^ [n, k] in the rotated basis (glq_decode_weights)."""
    torch = _torch()
    dev = _check_layer(layer, False, False)
    _dev_tensor(out, "out", dev, shape=(layer.n, layer.k), dtypes=(torch.float32, torch.bfloat16))
    st = layer.struct()
    _check(_lib.glq_decode_weights(ctypes.byref(st), out.data_ptr(), _dtype_code(out), _stream_ptr(stream)),
           "glq_decode_weights")
    return out


def workspace_bytes(layer: Layer, m: int) -> int:
    st = layer.struct()
    return int(_lib.glq_fused_linear_workspace(ctypes.byref(st), m))


def fused_linear(layer: Layer, x, y, workspace, flags: int = 0, stream=None):
    """y = U^T (s W^) (V x) (glq_fused_linear); x [m, k], y [m, n]."""
    dev = _check_layer(layer, not (flags & FLAG_NO_INPUT_RHT), not (flags & FLAG_NO_OUTPUT_RHT))
    m = _check_linear_io(dev, layer.n, layer.k, x, y, workspace, flags)
    st = layer.struct()
    rc = _lib.glq_fused_linear(ctypes.byref(st), x.data_ptr(), _dtype_code(x), m, y.data_ptr(),
                               _dtype_code(y), workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                               flags, _stream_ptr(stream))
    _check(rc, "glq_fused_linear")
    return y
