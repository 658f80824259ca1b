"""CPU oracle for packed variable-length QK rotary position embedding.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers. The product path (the HIP library and
its Python binding) never imports this package.

The arithmetic lives in ``rope_oracle.c`` (plain C, fp64/long double); this
module only marshals numpy arrays through ctypes. See that file's header for
the pages each function follows and the readings taken where they are silent.

``Oracle(path)`` wraps one build of the C file (the mutation tests load
deliberately broken builds made on the CPU); the module-level functions use
the default build, ``oracle/librope_oracle.so``.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, F16 = 0, 1, 2
_DTYPES = {"f32": F32, "bf16": BF16, "f16": F16}


def _ptr(a):
    return None if a is None else a.ctypes.data


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Element storage for the C side: float32 for f32, raw 16-bit words otherwise."""
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if x.dtype not in (np.uint16, np.int16):
        raise TypeError("bf16/f16 inputs are passed as their raw 16-bit words")
    return np.ascontiguousarray(x).view(np.uint16)


class Oracle:
    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        vp = ctypes.c_void_p
        lib.oracle_inv_freq.argtypes = [dbl, i32, vp]
        lib.oracle_inv_freq.restype = None
        lib.oracle_cos_sin.argtypes = [vp, i64, i32, dbl, vp, vp]
        lib.oracle_cos_sin.restype = None
        lib.oracle_positions.argtypes = [vp, i32, vp, i64, vp, vp]
        lib.oracle_positions.restype = None
        lib.oracle_rope.argtypes = [i32, vp, vp, i64, i32, i32, vp, i32, vp, dbl, i32, i32]
        lib.oracle_rope.restype = i32
        lib.oracle_rope_rows.argtypes = [i32, vp, vp, vp, i64, i32, i32, vp, i32, vp, dbl, i32,
                                         i32]
        lib.oracle_rope_rows.restype = i32
        lib.oracle_rope_table.argtypes = [i32, vp, vp, i64, i32, i32, vp, i32, vp, vp, vp, vp, vp,
                                          i64, i32]
        lib.oracle_rope_table.restype = i32
        lib.oracle_round_bf16.argtypes = [vp, vp, i64]
        lib.oracle_round_bf16.restype = None
        lib.oracle_fwd_bwd_seconds.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32,
                                               i32, vp, i32, vp, dbl, i32]
        lib.oracle_fwd_bwd_seconds.restype = dbl
        lib.oracle_cos_sin_ex.argtypes = [vp, i64, i32, dbl, dbl, vp, vp]
        lib.oracle_cos_sin_ex.restype = None
        lib.oracle_positions_ex.argtypes = [vp, i32, vp, vp, vp, i64, vp, vp]
        lib.oracle_positions_ex.restype = None
        lib.oracle_rope_ex.argtypes = [i32, vp, vp, i64, i32, i32, vp, i32, vp, vp, vp, dbl, dbl,
                                       i32, i32]
        lib.oracle_rope_ex.restype = i32
        lib.oracle_rope_rows_ex.argtypes = [i32, vp, vp, vp, i64, i32, i32, vp, i32, vp, vp, vp,
                                            dbl, dbl, i32, i32]
        lib.oracle_rope_rows_ex.restype = i32
        lib.oracle_rows_fwd_bwd_seconds.argtypes = [i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64,
                                                    i32, i32, i32, vp, i32, vp, dbl, i32]
        lib.oracle_rows_fwd_bwd_seconds.restype = dbl
        self.lib = lib
        self.path = path

    def inv_freq(self, theta: float, D: int) -> np.ndarray:
        out = np.empty(D // 2, dtype=np.float32)
        self.lib.oracle_inv_freq(float(theta), int(D), _ptr(out))
        return out

    def cos_sin(self, positions, D: int, theta: float, pos_scale: float = 1.0):
        pos = _i32(np.atleast_1d(positions))
        c = np.empty((pos.size, D // 2), dtype=np.float32)
        s = np.empty_like(c)
        self.lib.oracle_cos_sin_ex(_ptr(pos), pos.size, int(D), float(theta), float(pos_scale),
                                   _ptr(c), _ptr(s))
        return c, s

    def positions(self, cu_seqlens, T: int, seqused=None, seq_offsets=None, position_ids=None):
        cu, su, so, pid = (_i32(a) for a in (cu_seqlens, seqused, seq_offsets, position_ids))
        pos = np.empty(int(T), dtype=np.int32)
        seq = np.empty(int(T), dtype=np.int32)
        num_seqs = 0 if cu is None else cu.size - 1
        self.lib.oracle_positions_ex(_ptr(cu), num_seqs, _ptr(su), _ptr(so), _ptr(pid), int(T),
                                     _ptr(pos), _ptr(seq))
        return pos, seq

    def rope(self, x: np.ndarray, cu_seqlens, theta: float, direction: int = 1,
             dtype: str = "f32", seqused=None, nthreads: int = 1, seq_offsets=None,
             position_ids=None, pos_scale: float = 1.0) -> np.ndarray:
        """Rotate a packed tensor x[T, H, D]; returns the fp32 result, same shape."""
        xs = _storage(x, dtype)
        T, H, D = xs.shape
        cu, su, so, pid = (_i32(a) for a in (cu_seqlens, seqused, seq_offsets, position_ids))
        num_seqs = 0 if cu is None else cu.size - 1
        y = np.empty((T, H, D), dtype=np.float32)
        rc = self.lib.oracle_rope_ex(_DTYPES[dtype], _ptr(xs), _ptr(y), T, H, D, _ptr(cu),
                                     num_seqs, _ptr(su), _ptr(so), _ptr(pid), float(theta),
                                     float(pos_scale), int(direction), int(nthreads))
        if rc != 0:
            raise ValueError("oracle_rope_ex rejected its arguments")
        return y

    def rope_table(self, x: np.ndarray, cu_seqlens, cos_tab, sin_tab, direction: int = 1,
                   dtype: str = "f32", seqused=None, seq_offsets=None,
                   position_ids=None) -> np.ndarray:
        """Rotate x[T, H, D] with cos/sin from tables [rows, D/2] (row p = position p);
        positions without a row are untouched. Returns the fp32 result."""
        xs = _storage(x, dtype)
        T, H, D = xs.shape
        ct = np.ascontiguousarray(cos_tab, dtype=np.float32)
        st = np.ascontiguousarray(sin_tab, dtype=np.float32)
        if ct.shape != st.shape or ct.ndim != 2 or ct.shape[1] != D // 2:
            raise ValueError("cos_tab and sin_tab must both be [rows, D/2]")
        cu, su, so, pid = (_i32(a) for a in (cu_seqlens, seqused, seq_offsets, position_ids))
        num_seqs = 0 if cu is None else cu.size - 1
        y = np.empty((T, H, D), dtype=np.float32)
        rc = self.lib.oracle_rope_table(_DTYPES[dtype], _ptr(xs), _ptr(y), T, H, D, _ptr(cu),
                                        num_seqs, _ptr(su), _ptr(so), _ptr(pid), _ptr(ct),
                                        _ptr(st), ct.shape[0], int(direction))
        if rc != 0:
            raise ValueError("oracle_rope_table rejected its arguments")
        return y

    def rope_rows(self, x_rows: np.ndarray, tokens, cu_seqlens, theta: float, direction: int = 1,
                  dtype: str = "f32", seqused=None, nthreads: int = 1, seq_offsets=None,
                  position_ids=None, pos_scale: float = 1.0) -> np.ndarray:
        """Outputs for the listed tokens only; x_rows[n, H, D] are their input rows."""
        xs = _storage(x_rows, dtype)
        n, H, D = xs.shape
        tok = np.ascontiguousarray(tokens, dtype=np.int64)
        if tok.size != n:
            raise ValueError("one token index per input row")
        cu, su, so, pid = (_i32(a) for a in (cu_seqlens, seqused, seq_offsets, position_ids))
        num_seqs = 0 if cu is None else cu.size - 1
        y = np.empty((n, H, D), dtype=np.float32)
        rc = self.lib.oracle_rope_rows_ex(_DTYPES[dtype], _ptr(xs), _ptr(y), _ptr(tok), n, H, D,
                                          _ptr(cu), num_seqs, _ptr(su), _ptr(so), _ptr(pid),
                                          float(theta), float(pos_scale), int(direction),
                                          int(nthreads))
        if rc != 0:
            raise ValueError("oracle_rope_rows_ex rejected its arguments")
        return y

    def round_bf16(self, y: np.ndarray) -> np.ndarray:
        """fp32 -> bf16 bits (uint16), round to nearest even."""
        ys = np.ascontiguousarray(y, dtype=np.float32)
        out = np.empty(ys.shape, dtype=np.uint16)
        self.lib.oracle_round_bf16(_ptr(ys), _ptr(out), ys.size)
        return out

    def fwd_bwd_seconds(self, q, k, dq, dk, cu_seqlens, theta: float, dtype: str, seqused=None,
                        nthreads: int = 1) -> float:
        """Wall time of the oracle's forward on (q, k) plus backward on (dq, dk)."""
        qs, ks, dqs, dks = (_storage(a, dtype) for a in (q, k, dq, dk))
        T, Hq, D = qs.shape
        Hkv = ks.shape[1]
        outs = [np.empty(a.shape, dtype=np.float32) for a in (qs, ks, dqs, dks)]
        cu, su = _i32(cu_seqlens), _i32(seqused)
        sec = self.lib.oracle_fwd_bwd_seconds(_DTYPES[dtype], _ptr(qs), _ptr(ks), _ptr(dqs),
                                              _ptr(dks), *(_ptr(o) for o in outs), T, Hq, Hkv, D,
                                              _ptr(cu), cu.size - 1, _ptr(su), float(theta),
                                              int(nthreads))
        if sec < 0:
            raise ValueError("oracle rejected its arguments")
        return sec


    def rows_fwd_bwd_timer(self, q_rows, k_rows, dq_rows, dk_rows, tokens, cu_seqlens,
                           theta: float, dtype: str, seqused=None):
        """A callable(nthreads) -> seconds: the oracle's forward on the gathered rows
        of q and k plus its backward on those of dq and dk (rows[n, H, D] of the
        listed tokens), timed inside the C library; outputs are allocated once."""
        ins = [_storage(a, dtype) for a in (q_rows, k_rows, dq_rows, dk_rows)]
        outs = [np.empty(a.shape, dtype=np.float32) for a in ins]
        tok = np.ascontiguousarray(tokens, dtype=np.int64)
        n, Hq, D = ins[0].shape
        Hkv = ins[1].shape[1]
        cu, su = _i32(cu_seqlens), _i32(seqused)

        def run(nthreads: int) -> float:
            sec = self.lib.oracle_rows_fwd_bwd_seconds(
                _DTYPES[dtype], *(_ptr(a) for a in ins), *(_ptr(o) for o in outs), _ptr(tok), n,
                Hq, Hkv, D, _ptr(cu), cu.size - 1, _ptr(su), float(theta), int(nthreads))
            if sec < 0:
                raise ValueError("oracle rejected its arguments")
            return sec
        return run


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB_PATH):
            _build.build()
        _default = Oracle(_build.LIB_PATH)
    return _default


def inv_freq(theta, D):
    return default().inv_freq(theta, D)


def cos_sin(positions, D, theta, pos_scale=1.0):
    return default().cos_sin(positions, D, theta, pos_scale)


def positions(cu_seqlens, T, seqused=None, seq_offsets=None, position_ids=None):
    return default().positions(cu_seqlens, T, seqused, seq_offsets, position_ids)


def rope(x, cu_seqlens, theta, direction=1, dtype="f32", seqused=None, nthreads=1,
         seq_offsets=None, position_ids=None, pos_scale=1.0):
    return default().rope(x, cu_seqlens, theta, direction, dtype, seqused, nthreads, seq_offsets,
                          position_ids, pos_scale)


def rope_rows(x_rows, tokens, cu_seqlens, theta, direction=1, dtype="f32", seqused=None,
              nthreads=1, seq_offsets=None, position_ids=None, pos_scale=1.0):
    return default().rope_rows(x_rows, tokens, cu_seqlens, theta, direction, dtype, seqused,
                               nthreads, seq_offsets, position_ids, pos_scale)


def rope_table(x, cu_seqlens, cos_tab, sin_tab, direction=1, dtype="f32", seqused=None,
               seq_offsets=None, position_ids=None):
    return default().rope_table(x, cu_seqlens, cos_tab, sin_tab, direction, dtype, seqused,
                                seq_offsets, position_ids)


def round_bf16(y):
    return default().round_bf16(y)


def fwd_bwd_seconds(q, k, dq, dk, cu_seqlens, theta, dtype, seqused=None, nthreads=1):
    return default().fwd_bwd_seconds(q, k, dq, dk, cu_seqlens, theta, dtype, seqused, nthreads)


def rows_fwd_bwd_timer(q_rows, k_rows, dq_rows, dk_rows, tokens, cu_seqlens, theta, dtype,
                       seqused=None):
    return default().rows_fwd_bwd_timer(q_rows, k_rows, dq_rows, dk_rows, tokens, cu_seqlens,
                                        theta, dtype, seqused)
