"""CPU oracle for the VBM stencil pipeline -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP path never calls it and shares no
code with it.  ``oracle.cpp`` states, function by function, what the pipeline
computes and which passage of the pages each step follows.

This module compiles ``oracle.cpp`` with g++ (single-threaded, -O2,
-ffp-contract=off, no fast-math) and wraps it with ctypes over numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB = os.path.join(_HERE, "_build", "liboracle.so")
CXXFLAGS = ["-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
            "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/_build/liboracle.so and return its path."""
    if not force and os.path.exists(_LIB):
        return _LIB
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    tmp = _LIB + ".tmp%d" % os.getpid()
    subprocess.run(["g++", *CXXFLAGS, _SRC, "-o", tmp], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I32 = ctypes.c_int
    lib.oracle_create.restype = P
    lib.oracle_create.argtypes = [P, I64]
    lib.oracle_destroy.argtypes = [P]
    lib.oracle_n_active.restype = I64
    lib.oracle_n_active.argtypes = [P]
    lib.oracle_n_leaves.restype = I64
    lib.oracle_n_leaves.argtypes = [P]
    lib.oracle_n_blocks.restype = I64
    lib.oracle_n_blocks.argtypes = [P, I32]
    lib.oracle_voxels.argtypes = [P, P]
    lib.oracle_leaves.argtypes = [P, P, P, P, P]
    lib.oracle_blocks.argtypes = [P, I32, P, P]
    lib.oracle_decode.argtypes = [P, I32, P, P]
    lib.oracle_taps_rows.restype = I32
    lib.oracle_taps_rows.argtypes = [P, I32, P, I64, P]
    lib.oracle_box_rows.argtypes = [P, P, I32, P, I64, P]
    lib.oracle_cross_rows.restype = I32
    lib.oracle_cross_rows.argtypes = [P, P, I32, I32, P, I64, P]
    lib.oracle_box_filter.argtypes = [P, P, I32, P]
    lib.oracle_cross_filter.restype = I32
    lib.oracle_cross_filter.argtypes = [P, P, I32, I32, P]
    lib.oracle_axis_rows.argtypes = [P, P, I32, P, I64, P]
    lib.oracle_axis_filter.argtypes = [P, P, I32, P]
    lib.oracle_weno_rows.argtypes = [P, P, I32, P, I64, P]
    lib.oracle_weno_filter.argtypes = [P, P, I32, P]
    lib.oracle_weno5.restype = ctypes.c_float
    lib.oracle_weno5.argtypes = [ctypes.c_float] * 5
    _lib = lib
    return lib


def weno5(a: float, b: float, c: float, d: float, e: float) -> float:
    """The oracle's fifth-order WENO derivative from five differences (fp32)."""
    return float(_load().oracle_weno5(a, b, c, d, e))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class OracleGrid:
    """The oracle's index grid over a set of integer coordinates."""

    def __init__(self, coords: np.ndarray):
        lib = _load()
        c = np.ascontiguousarray(coords, dtype=np.int32).reshape(-1, 3)
        self._h = lib.oracle_create(_ptr(c), c.shape[0])
        if not self._h:
            raise ValueError("coordinate out of the oracle's range (|c| < 2^20 - 1)")
        self._lib = lib
        self.n_active = int(lib.oracle_n_active(self._h))
        self.n_leaves = int(lib.oracle_n_leaves(self._h))

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.oracle_destroy(h)
            self._h = None

    def n_blocks(self, log2w: int) -> int:
        return int(self._lib.oracle_n_blocks(self._h, log2w))

    def voxels(self) -> np.ndarray:
        out = np.empty((self.n_active, 3), np.int32)
        self._lib.oracle_voxels(self._h, _ptr(out))
        return out

    def leaves(self):
        L = self.n_leaves
        origin = np.empty((L, 3), np.int32)
        mask = np.empty((L, 8), np.uint64)
        first = np.empty(L, np.uint64)
        prefix = np.empty(L, np.uint64)
        self._lib.oracle_leaves(self._h, _ptr(origin), _ptr(mask), _ptr(first), _ptr(prefix))
        return dict(origin=origin, mask=mask, first=first, prefix=prefix)

    def blocks(self, log2w: int):
        nb = self.n_blocks(log2w)
        first_leaf = np.empty(nb, np.uint32)
        jump = np.empty((nb, (1 << log2w) // 64), np.uint64)
        self._lib.oracle_blocks(self._h, log2w, _ptr(first_leaf), _ptr(jump))
        return dict(first_leaf=first_leaf, jump=jump)

    def decode(self, log2w: int):
        total = self.n_blocks(log2w) << log2w
        leaf = np.empty(total, np.uint32)
        off = np.empty(total, np.uint16)
        self._lib.oracle_decode(self._h, log2w, _ptr(leaf), _ptr(off))
        return leaf, off

    def taps(self, shape: int, idx: np.ndarray | None = None) -> np.ndarray:
        """Rows of raw tap indices (uint64) for the given indices (default 1..N)."""
        if idx is None:
            idx = np.arange(1, self.n_active + 1, dtype=np.uint64)
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        out = np.empty((idx.size, shape), np.uint64)
        if self._lib.oracle_taps_rows(self._h, shape, _ptr(idx), idx.size, _ptr(out)) != 0:
            raise ValueError("shape must be 27, 7 or 19")
        return out

    def box(self, sidecar: np.ndarray, idx: np.ndarray | None = None) -> np.ndarray:
        sc = np.ascontiguousarray(sidecar, dtype=np.float32)
        C = sc.shape[1]
        assert sc.shape[0] == self.n_active + 1
        if idx is None:
            out = np.empty((self.n_active + 1, C), np.float32)
            self._lib.oracle_box_filter(self._h, _ptr(sc), C, _ptr(out))
            return out
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        out = np.empty((idx.size, C), np.float32)
        self._lib.oracle_box_rows(self._h, _ptr(sc), C, _ptr(idx), idx.size, _ptr(out))
        return out

    def cross(self, sidecar: np.ndarray, op: str = "sum", idx: np.ndarray | None = None) -> np.ndarray:
        code = {"sum": 0, "laplacian": 1}[op]
        sc = np.ascontiguousarray(sidecar, dtype=np.float32)
        C = sc.shape[1]
        assert sc.shape[0] == self.n_active + 1
        if idx is None:
            out = np.empty((self.n_active + 1, C), np.float32)
            self._lib.oracle_cross_filter(self._h, _ptr(sc), C, code, _ptr(out))
            return out
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        out = np.empty((idx.size, C), np.float32)
        self._lib.oracle_cross_rows(self._h, _ptr(sc), C, code, _ptr(idx), idx.size, _ptr(out))
        return out

    def axis(self, sidecar: np.ndarray, idx: np.ndarray | None = None) -> np.ndarray:
        """19-tap axis stencil (centre and +-1..+-3 along each axis): fp32 sum in tap order."""
        sc = np.ascontiguousarray(sidecar, dtype=np.float32)
        C = sc.shape[1]
        assert sc.shape[0] == self.n_active + 1
        if idx is None:
            out = np.empty((self.n_active + 1, C), np.float32)
            self._lib.oracle_axis_filter(self._h, _ptr(sc), C, _ptr(out))
            return out
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        out = np.empty((idx.size, C), np.float32)
        self._lib.oracle_axis_rows(self._h, _ptr(sc), C, _ptr(idx), idx.size, _ptr(out))
        return out

    def weno(self, sidecar: np.ndarray, idx: np.ndarray | None = None) -> np.ndarray:
        """WENO consumer on the 19 axis taps: per channel the squared norm of the
        Godunov upwind gradient from fifth-order WENO one-sided derivatives (fp32).
        Inactive taps read sidecar row 0."""
        sc = np.ascontiguousarray(sidecar, dtype=np.float32)
        C = sc.shape[1]
        assert sc.shape[0] == self.n_active + 1
        if idx is None:
            out = np.empty((self.n_active + 1, C), np.float32)
            self._lib.oracle_weno_filter(self._h, _ptr(sc), C, _ptr(out))
            return out
        idx = np.ascontiguousarray(idx, dtype=np.uint64)
        out = np.empty((idx.size, C), np.float32)
        self._lib.oracle_weno_rows(self._h, _ptr(sc), C, _ptr(idx), idx.size, _ptr(out))
        return out
