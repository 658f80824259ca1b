"""Fused, in-place, packed variable-length QK rotary position embedding (RoPE),
and the SwiGLU / GeGLU MLP activations, for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``include/rope_qk.h`` and ``include/glu.h``
(librope_qk.so, built from ``csrc/rope_qk.hip`` and ``csrc/glu.hip``). This module
only checks tensor metadata and marshals pointers, sizes and the current HIP
stream; every step of the computation runs in the library's HIP kernels. There is
no CPU fallback: if the library is missing, importing this package raises.
Differentiable wrappers live in ``packed_varlen_rotary_rope_amd.functional``.

The operations follow the Unsloth page "Entrainement des LLM 3 fois plus rapide
avec les noyaux Unsloth + le packing" (section "Kernel Triton QK RoPE fusionne
avec packing": one in-place kernel for Q and K, rotate_half form, backward =
sin negated; section "Packing non contamine": positions restart per sample;
section "Indexage int64 pour les kernels Triton": SwiGLU / GeGLU kernels with a
64-bit offset specialization).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "RopeError", "qk_fwd_", "qk_bwd_", "qk_apply_", "qk_apply_ex_", "qk_apply_table_",
    "qk_apply_padded_", "valid_prefix", "qk_fwd_pos_", "qk_bwd_pos_",
    "positions", "cos_sin", "cos_sin_table", "inv_freq", "abi_version", "LIB_PATH", "INDEX_AUTO", "INDEX_32",
    "INDEX_64", "glu_fwd", "glu_bwd", "GLU_KINDS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librope_qk.so")

F32, BF16, F16 = 0, 1, 2
INDEX_AUTO, INDEX_32, INDEX_64 = 0, 1, 2
_DTYPE_CODE = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}


class RopeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_lib.rope_status_str(status).decode()} ({status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python packed_varlen_rotary_rope_amd/build.py` "
            "(hipcc, gfx950). There is no fallback implementation.")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, dbl, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    qk = [vp, vp, i64, i32, i32, i32, vp, i32, vp, dbl, i32]
    lib.rope_qk_fwd.argtypes = qk + [vp]
    lib.rope_qk_bwd.argtypes = qk + [vp]
    lib.rope_qk_apply.argtypes = qk + [i32, i32, i32, vp]
    lib.rope_qk_apply_ex.argtypes = [vp, vp, i64, i32, i32, i32, i64, i64, vp, i32, vp, vp, vp,
                                     dbl, dbl, i32, i32, i32, i32, vp]
    lib.rope_qk_apply_table.argtypes = [vp, vp, i64, i32, i32, i32, i64, i64, vp, i32, vp, vp, vp,
                                        vp, vp, i32, i32, i32, i32, i32, vp]
    lib.rope_qk_fwd_pos.argtypes = [vp, vp, i64, i32, i32, i32, vp, dbl, i32, vp]
    lib.rope_qk_bwd_pos.argtypes = [vp, vp, i64, i32, i32, i32, vp, dbl, i32, vp]
    lib.rope_qk_apply_padded.argtypes = [vp, vp, i64, i32, i32, i32, i64, i64, vp, i32, vp, vp,
                                         i64, vp, dbl, dbl, i32, i32, i32, vp]
    lib.rope_valid_prefix.argtypes = [vp, i32, vp, vp, vp]
    lib.rope_positions.argtypes = [vp, i32, vp, i64, vp, vp, vp]
    lib.rope_positions_ex.argtypes = [vp, i32, vp, vp, vp, i64, vp, vp, vp]
    lib.rope_cos_sin.argtypes = [i32, i32, dbl, vp, vp, vp]
    lib.rope_cos_sin_at.argtypes = [vp, i64, i32, dbl, dbl, vp, vp, vp]
    lib.rope_inv_freq.argtypes = [dbl, i32, vp]
    lib.glu_fwd.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp]
    lib.glu_bwd.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, i32, vp]
    for name in ("rope_qk_fwd", "rope_qk_bwd", "rope_qk_apply", "rope_qk_apply_ex", "rope_qk_apply_table",
                 "rope_qk_apply_padded", "rope_valid_prefix",
                 "rope_qk_fwd_pos", "rope_qk_bwd_pos", "rope_positions", "rope_positions_ex",
                 "rope_cos_sin", "rope_cos_sin_at", "rope_inv_freq", "rope_abi_version",
                 "glu_fwd", "glu_bwd"):
        getattr(lib, name).restype = i32
    lib.rope_status_str.argtypes = [i32]
    lib.rope_status_str.restype = ctypes.c_char_p
    lib.rope_abi_version.argtypes = []
    return lib


_lib = _load()


def abi_version() -> int:
    return int(_lib.rope_abi_version())


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, what: str) -> None:
    if status != 0:
        raise RopeError(status, what)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _index_tensor(t, name: str, device: torch.device):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.device != device or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor on {device}")
    return t


def _qk_tensors(q, k, strided: bool = False):
    if q.device.type != "cuda" or k.device != q.device:
        raise TypeError("q and k must be on the same GPU")
    if q.dtype != k.dtype or q.dtype not in _DTYPE_CODE:
        raise TypeError("q and k must share one dtype: float32, bfloat16 or float16")
    if q.dim() != 3 or k.dim() != 3 or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("expected q[T, Hq, D] and k[T, Hkv, D]")
    if not strided and not (q.is_contiguous() and k.is_contiguous()):
        raise ValueError("q and k must be contiguous (rotation is in place)")
    T, Hq, D = q.shape
    return T, Hq, k.shape[1], D


def _token_stride(x, name: str) -> int:
    """Token stride of a [T, H, D] view whose heads are contiguous within a token
    (0 when the view is contiguous, meaning H * D)."""
    T, H, D = x.shape
    if x.is_contiguous() or x.numel() == 0:
        return 0
    if (D > 1 and x.stride(2) != 1) or (H > 1 and x.stride(1) != D):
        raise ValueError(f"{name}: the heads of a token must be contiguous "
                         "(stride(2) == 1 and stride(1) == D)")
    return 0 if T == 1 else x.stride(0)


def _qk_args(q, k, cu_seqlens, seqused):
    T, Hq, Hkv, D = _qk_tensors(q, k)
    if cu_seqlens is None:
        raise ValueError("cu_seqlens is required")
    cu = _index_tensor(cu_seqlens, "cu_seqlens", q.device)
    su = _index_tensor(seqused, "seqused", q.device)
    num_seqs = cu.numel() - 1
    if su is not None and su.numel() != num_seqs:
        raise ValueError("seqused must have one entry per sequence")
    return T, Hq, Hkv, D, cu, num_seqs, su


def qk_apply_(q, k, cu_seqlens, theta: float, direction: int = 1, seqused=None,
              index_mode: int = INDEX_AUTO, tokens_per_wave: int = 0):
    """Rotate q[T, Hq, D] and k[T, Hkv, D] in place (direction +1: forward, -1:
    backward), one kernel launch on the current stream. Returns (q, k)."""
    T, Hq, Hkv, D, cu, num_seqs, su = _qk_args(q, k, cu_seqlens, seqused)
    st = _lib.rope_qk_apply(_ptr(q), _ptr(k), T, Hq, Hkv, D, _ptr(cu), num_seqs, _ptr(su),
                            float(theta), _DTYPE_CODE[q.dtype], int(direction), int(index_mode),
                            int(tokens_per_wave), _stream(q.device))
    _check(st, "rope_qk_apply")
    return q, k


def qk_apply_ex_(q, k, theta: float, direction: int = 1, cu_seqlens=None, seqused=None,
                 seq_offsets=None, position_ids=None, pos_scale: float = 1.0,
                 index_mode: int = INDEX_AUTO, tokens_per_wave: int = 0):
    """The general form: positions from `position_ids` (int32[T], negative = untouched)
    or from `cu_seqlens` (+ optional `seqused`, `seq_offsets`), angles with linear
    position interpolation by `pos_scale` (>= 1). In place; returns (q, k).

    q and k may be strided views, e.g. slices of a fused QKV projection output
    [T, (Hq + 2 Hkv) * D] viewed as [T, H, D], as long as the heads of each token
    are contiguous; they must not overlap."""
    T, Hq, Hkv, D = _qk_tensors(q, k, strided=True)
    qs, ks = _token_stride(q, "q"), _token_stride(k, "k")
    cu, num_seqs, su, so, pid = _position_args(q, T, cu_seqlens, seqused, seq_offsets, position_ids)
    st = _lib.rope_qk_apply_ex(_ptr(q), _ptr(k), T, Hq, Hkv, D, qs, ks, _ptr(cu), num_seqs,
                               _ptr(su), _ptr(so), _ptr(pid), float(theta), float(pos_scale),
                               _DTYPE_CODE[q.dtype], int(direction), int(index_mode),
                               int(tokens_per_wave), _stream(q.device))
    _check(st, "rope_qk_apply_ex")
    return q, k


def qk_apply_padded_(q, k, theta: float, direction: int, cu_seqlens, seqused, cu_valid,
                     valid_tokens: int, seq_offsets=None, pos_scale: float = 1.0,
                     index_mode: int = INDEX_AUTO):
    """qk_apply_ex_ on a padded layout whose rotated tokens are counted up front:
    `cu_valid` (int32[B+1] on the GPU, from valid_prefix, once per batch) holds the
    running count of rotated tokens per sequence and `valid_tokens` (a host int)
    their total, so the launch covers only those tokens. Same results as
    qk_apply_ex_ with the same cu_seqlens, seqused and seq_offsets. In place;
    returns (q, k)."""
    T, Hq, Hkv, D = _qk_tensors(q, k, strided=True)
    qs, ks = _token_stride(q, "q"), _token_stride(k, "k")
    if cu_seqlens is None:
        raise ValueError("cu_seqlens is required")
    cu, num_seqs, su, so, _ = _position_args(q, T, cu_seqlens, seqused, seq_offsets, None)
    cv = _index_tensor(cu_valid, "cu_valid", q.device)
    if cv is None or cv.numel() != num_seqs + 1:
        raise ValueError("cu_valid must have num_seqs + 1 entries")
    st = _lib.rope_qk_apply_padded(_ptr(q), _ptr(k), T, Hq, Hkv, D, qs, ks, _ptr(cu), num_seqs,
                                   _ptr(su), _ptr(cv), int(valid_tokens), _ptr(so), float(theta),
                                   float(pos_scale), _DTYPE_CODE[q.dtype], int(direction),
                                   int(index_mode), _stream(q.device))
    _check(st, "rope_qk_apply_padded")
    return q, k


def valid_prefix(cu_seqlens, seqused=None, out=None):
    """int32[B+1] on cu_seqlens' GPU: the running count of the tokens each sequence
    rotates (min(seqused[s], its length)), the cu_valid of qk_apply_padded_; written
    to `out` (int32[B+1]) when given."""
    dev = cu_seqlens.device
    cu = _index_tensor(cu_seqlens, "cu_seqlens", dev)
    su = _index_tensor(seqused, "seqused", dev)
    num_seqs = cu.numel() - 1
    if num_seqs < 0 or (su is not None and su.numel() != num_seqs):
        raise ValueError("cu_seqlens needs >= 1 entry and seqused one entry per sequence")
    if out is None:
        out = torch.empty(num_seqs + 1, dtype=torch.int32, device=dev)
    elif _index_tensor(out, "out", dev).numel() != num_seqs + 1:
        raise ValueError("out must have num_seqs + 1 entries")
    _check(_lib.rope_valid_prefix(_ptr(cu), num_seqs, _ptr(su), _ptr(out), _stream(dev)),
           "rope_valid_prefix")
    return out


def _position_args(q, T, cu_seqlens, seqused, seq_offsets, position_ids):
    cu = _index_tensor(cu_seqlens, "cu_seqlens", q.device)
    su = _index_tensor(seqused, "seqused", q.device)
    so = _index_tensor(seq_offsets, "seq_offsets", q.device)
    pid = _index_tensor(position_ids, "position_ids", q.device)
    if pid is None and cu is None:
        raise ValueError("give cu_seqlens or position_ids")
    if pid is not None and pid.numel() != T:
        raise ValueError("position_ids must have one entry per token")
    num_seqs = 0 if cu is None else cu.numel() - 1
    for name, t in (("seqused", su), ("seq_offsets", so)):
        if t is not None and t.numel() != num_seqs:
            raise ValueError(f"{name} must have one entry per sequence")
    return cu, num_seqs, su, so, pid


def qk_apply_table_(q, k, cos_tab, sin_tab, direction: int = 1, cu_seqlens=None, seqused=None,
                    seq_offsets=None, position_ids=None, index_mode: int = INDEX_AUTO,
                    tokens_per_wave: int = 0):
    """qk_apply_ex_ with caller-supplied cos/sin tables: `cos_tab` and `sin_tab` are
    float32 [rows, D/2] device tensors whose row p holds the cos / sin of position p
    (as `cos_sin(torch.arange(rows), D, theta)` returns them). Tokens whose position
    has no row are left untouched. In place; returns (q, k)."""
    T, Hq, Hkv, D = _qk_tensors(q, k, strided=True)
    qs, ks = _token_stride(q, "q"), _token_stride(k, "k")
    for name, t in (("cos_tab", cos_tab), ("sin_tab", sin_tab)):
        if (t.dtype != torch.float32 or t.device != q.device or not t.is_contiguous()
                or t.dim() != 2 or t.shape[1] != D // 2):
            raise ValueError(f"{name} must be a contiguous float32 [rows, D/2] tensor on "
                             f"{q.device}")
    if cos_tab.shape != sin_tab.shape or cos_tab.shape[0] < 1 or cos_tab.shape[0] > 2 ** 31 - 1:
        raise ValueError("cos_tab and sin_tab must have the same 1 .. 2^31-1 rows")
    cu, num_seqs, su, so, pid = _position_args(q, T, cu_seqlens, seqused, seq_offsets, position_ids)
    st = _lib.rope_qk_apply_table(_ptr(q), _ptr(k), T, Hq, Hkv, D, qs, ks, _ptr(cu), num_seqs,
                                  _ptr(su), _ptr(so), _ptr(pid), _ptr(cos_tab), _ptr(sin_tab),
                                  int(cos_tab.shape[0]), _DTYPE_CODE[q.dtype], int(direction),
                                  int(index_mode), int(tokens_per_wave), _stream(q.device))
    _check(st, "rope_qk_apply_table")
    return q, k


def qk_fwd_pos_(q, k, position_ids, theta: float):
    """Forward RoPE in place with explicit positions (int32[T]; negative = untouched)."""
    T, Hq, Hkv, D = _qk_tensors(q, k)
    pid = _index_tensor(position_ids, "position_ids", q.device)
    if pid.numel() != T:
        raise ValueError("position_ids must have one entry per token")
    st = _lib.rope_qk_fwd_pos(_ptr(q), _ptr(k), T, Hq, Hkv, D, _ptr(pid), float(theta),
                              _DTYPE_CODE[q.dtype], _stream(q.device))
    _check(st, "rope_qk_fwd_pos")
    return q, k


def qk_bwd_pos_(dq, dk, position_ids, theta: float):
    """Backward RoPE in place with explicit positions (int32[T]; negative = untouched)."""
    T, Hq, Hkv, D = _qk_tensors(dq, dk)
    pid = _index_tensor(position_ids, "position_ids", dq.device)
    if pid.numel() != T:
        raise ValueError("position_ids must have one entry per token")
    st = _lib.rope_qk_bwd_pos(_ptr(dq), _ptr(dk), T, Hq, Hkv, D, _ptr(pid), float(theta),
                              _DTYPE_CODE[dq.dtype], _stream(dq.device))
    _check(st, "rope_qk_bwd_pos")
    return dq, dk


def qk_fwd_(q, k, cu_seqlens, theta: float, seqused=None):
    """Forward RoPE on q and k in place (one launch; a long pass several, over
    consecutive token ranges). Returns (q, k)."""
    T, Hq, Hkv, D, cu, num_seqs, su = _qk_args(q, k, cu_seqlens, seqused)
    st = _lib.rope_qk_fwd(_ptr(q), _ptr(k), T, Hq, Hkv, D, _ptr(cu), num_seqs, _ptr(su),
                          float(theta), _DTYPE_CODE[q.dtype], _stream(q.device))
    _check(st, "rope_qk_fwd")
    return q, k


def qk_bwd_(dq, dk, cu_seqlens, theta: float, seqused=None):
    """Backward RoPE (sin negated) on the gradients dq and dk in place. Returns (dq, dk)."""
    T, Hq, Hkv, D, cu, num_seqs, su = _qk_args(dq, dk, cu_seqlens, seqused)
    st = _lib.rope_qk_bwd(_ptr(dq), _ptr(dk), T, Hq, Hkv, D, _ptr(cu), num_seqs, _ptr(su),
                          float(theta), _DTYPE_CODE[dq.dtype], _stream(dq.device))
    _check(st, "rope_qk_bwd")
    return dq, dk


def positions(cu_seqlens, T: int, seqused=None, seq_offsets=None, position_ids=None):
    """(pos, seq) int32[T] on the GPU as the kernels compute them; -1 = untouched."""
    ref = cu_seqlens if cu_seqlens is not None else position_ids
    device = ref.device
    cu = _index_tensor(cu_seqlens, "cu_seqlens", device)
    su = _index_tensor(seqused, "seqused", device)
    so = _index_tensor(seq_offsets, "seq_offsets", device)
    pid = _index_tensor(position_ids, "position_ids", device)
    pos = torch.empty(int(T), dtype=torch.int32, device=device)
    seq = torch.empty(int(T), dtype=torch.int32, device=device)
    num_seqs = 0 if cu is None else cu.numel() - 1
    st = _lib.rope_positions_ex(_ptr(cu), num_seqs, _ptr(su), _ptr(so), _ptr(pid), int(T),
                                _ptr(pos), _ptr(seq), _stream(device))
    _check(st, "rope_positions_ex")
    return pos, seq


def cos_sin(pos, D: int, theta: float, pos_scale: float = 1.0):
    """fp32 (cos, sin) [n, D/2] for the int32 positions `pos` (on the GPU)."""
    p = _index_tensor(pos, "pos", pos.device)
    c = torch.empty((p.numel(), D // 2), dtype=torch.float32, device=p.device)
    s = torch.empty_like(c)
    st = _lib.rope_cos_sin_at(_ptr(p), p.numel(), int(D), float(theta), float(pos_scale), _ptr(c),
                              _ptr(s), _stream(p.device))
    _check(st, "rope_cos_sin_at")
    return c, s


def cos_sin_table(max_pos: int, D: int, theta: float, device=None):
    """fp32 (cos, sin) [max_pos, D/2] for positions 0 .. max_pos-1 on `device`
    (default: the current GPU): the tables qk_apply_table_ takes."""
    device = torch.device(device) if device is not None else torch.device(
        "cuda", torch.cuda.current_device())
    c = torch.empty((int(max_pos), D // 2), dtype=torch.float32, device=device)
    s = torch.empty_like(c)
    _check(_lib.rope_cos_sin(int(max_pos), int(D), float(theta), _ptr(c), _ptr(s),
                             _stream(device)), "rope_cos_sin")
    return c, s


def inv_freq(theta: float, D: int) -> torch.Tensor:
    """Host-computed fp32 inverse frequencies theta^(-2j/D) (a CPU tensor)."""
    out = torch.empty(D // 2, dtype=torch.float32)
    _check(_lib.rope_inv_freq(float(theta), int(D), out.data_ptr()), "rope_inv_freq")
    return out


# ---------------------------------------------------------------- SwiGLU / GeGLU

GLU_KINDS = {"swiglu": 0, "geglu": 1, "geglu_tanh": 2}


def _rows(x, name: str):
    """(rows, cols, row stride) of a 2-D CUDA tensor with contiguous columns."""
    if x.device.type != "cuda" or x.dtype not in _DTYPE_CODE:
        raise TypeError(f"{name}: expected a float32, bfloat16 or float16 CUDA tensor")
    if x.dim() != 2:
        raise ValueError(f"{name}: expected a 2-D [rows, cols] tensor")
    rows, cols = x.shape
    if cols > 1 and x.stride(1) != 1:
        raise ValueError(f"{name}: columns must be contiguous")
    return rows, cols, (x.stride(0) if rows > 1 else cols)


def _glu_group(tensors, names):
    """Shape and one shared row stride for tensors that the C ABI lays out alike."""
    dims = [_rows(t, n) for t, n in zip(tensors, names)]
    rows, cols, stride = dims[0]
    for (r, c, st), n in zip(dims[1:], names[1:]):
        if (r, c) != (rows, cols):
            raise ValueError(f"{n}: shape differs from {names[0]}")
        if st != stride and rows > 1:
            raise ValueError(f"{n}: row stride differs from {names[0]}")
    dtype = tensors[0].dtype
    if any(t.dtype != dtype or t.device != tensors[0].device for t in tensors):
        raise TypeError("all tensors must share one dtype and device")
    return rows, cols, stride


def glu_fwd(kind: str, e, g, out=None, index_mode: int = INDEX_AUTO):
    """h = act(e) * g for act = silu ("swiglu"), exact gelu ("geglu") or tanh gelu
    ("geglu_tanh"), on the current stream (one launch; a long call several, one after
    another over consecutive element ranges). e and g: [rows, cols] with
    contiguous columns and one row stride (two dense tensors, or the two halves of
    a fused gate/up output). out: a [rows, cols] tensor (new and dense if None; it
    may be e or g itself). Returns out."""
    rows, cols, in_stride = _glu_group([e, g], ["e", "g"])
    if out is None:
        out = torch.empty((rows, cols), dtype=e.dtype, device=e.device)
    orows, ocols, out_stride = _rows(out, "out")
    if (orows, ocols) != (rows, cols) or out.dtype != e.dtype or out.device != e.device:
        raise ValueError("out: shape, dtype or device differs from e")
    st = _lib.glu_fwd(GLU_KINDS[kind], _ptr(e), _ptr(g), _ptr(out), rows, cols, in_stride,
                      out_stride, _DTYPE_CODE[e.dtype], int(index_mode), _stream(e.device))
    _check(st, "glu_fwd")
    return out


def glu_bwd(kind: str, dh, e, g, de=None, dg=None, index_mode: int = INDEX_AUTO):
    """de = dh * g * act'(e), dg = dh * act(e), launched like glu_fwd. de and dg take the
    layout of e and g (new tensors with e's strides if None; pass de=e, dg=g to
    update the inputs in place). Returns (de, dg)."""
    rows, cols, in_stride = _glu_group([e, g], ["e", "g"])
    hrows, hcols, out_stride = _rows(dh, "dh")
    if (hrows, hcols) != (rows, cols) or dh.dtype != e.dtype or dh.device != e.device:
        raise ValueError("dh: shape, dtype or device differs from e")
    if de is None and dg is None and in_stride == 2 * cols and \
            g.data_ptr() == e.data_ptr() + cols * e.element_size():
        # e and g are the halves of one fused gate/up output: so are de and dg
        buf = torch.empty((rows, 2 * cols), dtype=e.dtype, device=e.device)
        de, dg = buf[:, :cols], buf[:, cols:]
    if de is None:
        de = torch.empty_strided((rows, cols), (in_stride, 1), dtype=e.dtype, device=e.device)
    if dg is None:
        dg = torch.empty_strided((rows, cols), (in_stride, 1), dtype=e.dtype, device=e.device)
    _glu_group([e, g, de, dg], ["e", "g", "de", "dg"])
    st = _lib.glu_bwd(GLU_KINDS[kind], _ptr(dh), _ptr(e), _ptr(g), _ptr(de), _ptr(dg), rows, cols,
                      in_stride, out_stride, _DTYPE_CODE[e.dtype], int(index_mode),
                      _stream(e.device))
    _check(st, "glu_bwd")
    return de, dg
