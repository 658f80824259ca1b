"""CPU oracle for SwiGLU / GeGLU (forward and backward).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The arithmetic lives in ``glu_oracle.c``
(plain C, double precision); this module marshals numpy arrays through ctypes.
That file's header lists the page it follows and the readings taken where the
page is silent.

``GluOracle(path)`` wraps one build of the C file (the mutation tests load
deliberately broken builds made on the CPU); the module-level functions use the
default build, ``oracle/libglu_oracle.so``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

KINDS = {"swiglu": 0, "geglu": 1, "geglu_tanh": 2}
DTYPES = {"f32": 0, "bf16": 1, "f16": 2}


def _rows_view(x: np.ndarray, dtype: str):
    """(array, row stride in elements) of a 2-D [rows, cols] view whose columns are
    contiguous: float32 for f32, raw 16-bit words for bf16 / f16."""
    want = np.float32 if dtype == "f32" else np.uint16
    if x.dtype == np.int16 and dtype != "f32":
        x = x.view(np.uint16)
    if x.dtype != want:
        raise TypeError(f"{dtype} inputs are passed as {np.dtype(want).name} arrays")
    if x.ndim != 2:
        raise ValueError("expected a 2-D [rows, cols] array")
    rows, cols = x.shape
    if cols > 1 and x.strides[1] != x.itemsize:
        raise ValueError("columns must be contiguous")
    stride = x.strides[0] // x.itemsize if rows > 1 else cols
    if rows > 1 and (x.strides[0] % x.itemsize or stride < cols):
        raise ValueError("rows must be at least cols elements apart")
    return x, stride


class GluOracle:
    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i32, i64, dbl, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        lib.oracle_glu_act.argtypes = [i32, dbl]
        lib.oracle_glu_act.restype = dbl
        lib.oracle_glu_grad.argtypes = [i32, dbl]
        lib.oracle_glu_grad.restype = dbl
        lib.oracle_glu_fwd.argtypes = [i32, i32, vp, vp, vp, i64, i64, i64, i32]
        lib.oracle_glu_fwd.restype = i32
        lib.oracle_glu_bwd.argtypes = [i32, i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32]
        lib.oracle_glu_bwd.restype = i32
        lib.oracle_glu_round.argtypes = [i32, vp, vp, i64]
        lib.oracle_glu_round.restype = None
        lib.oracle_glu_seconds.argtypes = [i32, i32, vp, vp, vp, vp, vp, vp, i64, i64, i32]
        lib.oracle_glu_seconds.restype = dbl
        self.lib = lib
        self.path = path

    def act(self, kind: str, e) -> np.ndarray:
        """act(e) per element, e as float64 values."""
        k = KINDS[kind]
        flat = np.asarray(e, dtype=np.float64).ravel()
        out = np.array([self.lib.oracle_glu_act(k, float(v)) for v in flat])
        return out.reshape(np.shape(e))

    def grad(self, kind: str, e) -> np.ndarray:
        """act'(e) per element, e as float64 values."""
        k = KINDS[kind]
        flat = np.asarray(e, dtype=np.float64).ravel()
        out = np.array([self.lib.oracle_glu_grad(k, float(v)) for v in flat])
        return out.reshape(np.shape(e))

    def fwd(self, kind: str, e: np.ndarray, g: np.ndarray, dtype: str,
            nthreads: int = 1) -> np.ndarray:
        """h = act(e) * g as dense float64 [rows, cols]; e and g are [rows, cols]
        views sharing one row stride."""
        e, se = _rows_view(e, dtype)
        g, sg = _rows_view(g, dtype)
        if e.shape != g.shape or se != sg:
            raise ValueError("e and g must share shape and row stride")
        rows, cols = e.shape
        h = np.empty((rows, cols), dtype=np.float64)
        rc = self.lib.oracle_glu_fwd(KINDS[kind], DTYPES[dtype], e.ctypes.data, g.ctypes.data,
                                     h.ctypes.data, rows, cols, se, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_glu_fwd rejected its arguments")
        return h

    def bwd(self, kind: str, dh: np.ndarray, e: np.ndarray, g: np.ndarray, dtype: str,
            nthreads: int = 1):
        """(de, dg) as dense float64 [rows, cols]."""
        e, se = _rows_view(e, dtype)
        g, sg = _rows_view(g, dtype)
        dh, sh = _rows_view(dh, dtype)
        if e.shape != g.shape or e.shape != dh.shape or se != sg:
            raise ValueError("dh, e and g must share a shape; e and g one row stride")
        rows, cols = e.shape
        de = np.empty((rows, cols), dtype=np.float64)
        dg = np.empty((rows, cols), dtype=np.float64)
        rc = self.lib.oracle_glu_bwd(KINDS[kind], DTYPES[dtype], dh.ctypes.data, e.ctypes.data,
                                     g.ctypes.data, de.ctypes.data, dg.ctypes.data, rows, cols,
                                     se, sh, int(nthreads))
        if rc != 0:
            raise ValueError("oracle_glu_bwd rejected its arguments")
        return de, dg

    def round(self, dtype: str, x: np.ndarray) -> np.ndarray:
        """One rounding (to nearest, ties to even) from float64 to the storage
        format: float32 values, or uint16 words for bf16 / f16."""
        xs = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(xs.shape, dtype=np.float32 if dtype == "f32" else np.uint16)
        self.lib.oracle_glu_round(DTYPES[dtype], xs.ctypes.data, out.ctypes.data, xs.size)
        return out

    def seconds(self, kind: str, e, g, dh, dtype: str, nthreads: int = 1) -> float:
        """Wall time of one forward plus one backward over dense [rows, cols] inputs."""
        e, _ = _rows_view(np.ascontiguousarray(e), dtype)
        g, _ = _rows_view(np.ascontiguousarray(g), dtype)
        dh, _ = _rows_view(np.ascontiguousarray(dh), dtype)
        rows, cols = e.shape
        outs = [np.empty((rows, cols), dtype=np.float64) for _ in range(3)]
        sec = self.lib.oracle_glu_seconds(KINDS[kind], DTYPES[dtype], e.ctypes.data,
                                          g.ctypes.data, dh.ctypes.data,
                                          *(o.ctypes.data for o in outs), rows, cols,
                                          int(nthreads))
        if sec < 0:
            raise ValueError("oracle rejected its arguments")
        return sec


_default: GluOracle | None = None


def default() -> GluOracle:
    global _default
    if _default is None:
        if not os.path.exists(_build.GLU_LIB_PATH):
            _build.build(_build.GLU_SRC, _build.GLU_LIB_PATH)
        _default = GluOracle(_build.GLU_LIB_PATH)
    return _default


def act(kind, e):
    return default().act(kind, e)


def grad(kind, e):
    return default().grad(kind, e)


def fwd(kind, e, g, dtype, nthreads=1):
    return default().fwd(kind, e, g, dtype, nthreads)


def bwd(kind, dh, e, g, dtype, nthreads=1):
    return default().bwd(kind, dh, e, g, dtype, nthreads)


def round_to(dtype, x):
    return default().round(dtype, x)


def seconds(kind, e, g, dh, dtype, nthreads=1):
    return default().seconds(kind, e, g, dh, dtype, nthreads)
