"""Loader of the oracle's C part (nearest_bf.c): compiled with gcc into
oracle/_build/ on first use (or by the package's build step), loaded with
ctypes. TEST INFRASTRUCTURE ONLY, like the rest of the oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "nearest_bf.c")
BUILD_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(BUILD_DIR, "liboracle_bf.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile nearest_bf.c (gcc -O2, OpenMP) unless an up-to-date build exists."""
    if not force and os.path.exists(LIB) and os.path.getmtime(LIB) >= os.path.getmtime(SRC):
        return LIB
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = LIB + f".tmp{os.getpid()}"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-o", tmp, SRC], check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.oracle_nearest_bf.restype = None
        lib.oracle_nearest_bf.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int64, ctypes.c_void_p]
        _lib = lib
    return _lib


def nearest_bruteforce(x: np.ndarray, table: np.ndarray) -> np.ndarray:
    """argmin over the rows of table [size, 8] (float64) for every row of x,
    lowest index on exact ties: the definition, evaluated in C."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64).reshape(-1, 8))
    table = np.ascontiguousarray(table, dtype=np.float64)
    out = np.empty(len(x), dtype=np.int64)
    if len(x):
        _load().oracle_nearest_bf(x.ctypes.data, len(x), table.ctypes.data, len(table), out.ctypes.data)
    return out
