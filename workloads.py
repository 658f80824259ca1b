"""Seeded synthetic workloads for packed variable-length QK-RoPE.

Shared by the tests, the smoke check and the benchmark, and by both sides of
every parity check (the HIP path and the CPU oracle). It holds only input
recipes -- sequence-length draws, cu_seqlens, N(0,1) tensors -- and none of
the rotation's arithmetic.

The shapes stand in for the pages' workloads (Unsloth "3x faster training +
packing": packed batches of short and long samples, an 80% short / 20% long
mix in the padding arithmetic, 1K-32K tokens per batch, 500K-token contexts;
TRL long-context guide: rope_theta = 1e6 for Qwen3). Head counts and head
size follow the Qwen3 family shapes: 4B/8B are 32 query heads and 8 KV heads,
32B is 64 and 8, all with head size 128.

Seeds: lengths 1000+k, Q 2000+k, K 3000+k, dQ 4000+k, dK 5000+k for workload
number k. Lengths use numpy's PCG64 (``default_rng``); tensors are drawn with
``torch.randn`` in fp32 from a seeded generator and then rounded to the storage
dtype, so the GPU and the oracle see the same bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "make_tensor", "names", "GluWorkload",
           "GLU_WORKLOADS", "glu_get", "glu_names"]


@dataclass(frozen=True)
class Workload:
    name: str
    number: int  # 1..5, the order the workloads are listed in
    T: int  # rows of the packed tensors
    Hq: int
    Hkv: int
    D: int
    dtype: str  # "f32" | "bf16" | "f16"
    theta: float
    cu_seqlens: np.ndarray = field(repr=False)  # int32[num_seqs + 1]
    seqused: np.ndarray | None = field(default=None, repr=False)  # int32[num_seqs] or None
    description: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.size - 1)

    @property
    def lengths(self) -> np.ndarray:
        spans = np.diff(self.cu_seqlens.astype(np.int64))
        if self.seqused is not None:
            spans = np.minimum(spans, self.seqused.astype(np.int64))
        return spans

    @property
    def valid_tokens(self) -> int:
        return int(self.lengths.sum())

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def seed(self, what: str) -> int:
        base = {"lengths": 1000, "q": 2000, "k": 3000, "dq": 4000, "dk": 5000}[what]
        return base + self.number

    def shape(self, what: str) -> tuple:
        heads = self.Hq if what in ("q", "dq") else self.Hkv
        return (self.T, heads, self.D)


def _cu(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def _fill_to(T: int, draw) -> list:
    """Append draws until the total reaches T; the last one is cut to hit T exactly."""
    lengths, total = [], 0
    while total < T:
        n = int(draw())
        n = min(n, T - total)
        lengths.append(n)
        total += n
    return lengths


def tiny_packed() -> Workload:
    lengths = [5, 17, 3, 39]
    return Workload("tiny_packed", 1, 64, 4, 2, 16, "f32", 1e4, _cu(lengths),
                    description="4 sequences {5,17,3,39}, T=64, Hq=4, Hkv=2, D=16, fp32")


def qwen3_4b_packed() -> Workload:
    rng = np.random.default_rng(1002)

    def draw():
        if rng.random() < 0.8:
            return rng.integers(32, 512, endpoint=True)
        return rng.integers(1024, 4096, endpoint=True)

    lengths = _fill_to(16384, draw)
    return Workload("qwen3_4b_packed", 2, 16384, 32, 8, 128, "bf16", 1e6, _cu(lengths),
                    description="T=16384 packed from 80% U{32..512} / 20% U{1024..4096}, "
                                "Hq=32, Hkv=8, D=128, bf16")


def _qwen3_8b_lengths() -> np.ndarray:
    rng = np.random.default_rng(1003)
    return rng.integers(256, 2048, size=8, endpoint=True)


def qwen3_8b_packed() -> Workload:
    lengths = _qwen3_8b_lengths()
    return Workload("qwen3_8b_packed", 3, int(lengths.sum()), 32, 8, 128, "bf16", 1e6,
                    _cu(lengths),
                    description="8 sequences U{256..2048} packed, Hq=32, Hkv=8, D=128, bf16")


def qwen3_8b_padded() -> Workload:
    lengths = _qwen3_8b_lengths()
    cu = (np.arange(9, dtype=np.int64) * 2048).astype(np.int32)
    return Workload("qwen3_8b_padded", 3, 8 * 2048, 32, 8, 128, "bf16", 1e6, cu,
                    seqused=lengths.astype(np.int32),
                    description="same 8 sequences padded to 8x2048 rows, padded rows skipped")


def qwen3_32b_packed() -> Workload:
    rng = np.random.default_rng(1004)
    lengths = _fill_to(32768, lambda: np.clip(rng.geometric(1.0 / 300.0), 8, 8192))
    return Workload("qwen3_32b_packed", 4, 32768, 64, 8, 128, "bf16", 1e6, _cu(lengths),
                    description="T=32768 packed from geometric(mean 300) clipped to [8,8192], "
                                "Hq=64, Hkv=8, D=128, bf16")


def long_ctx_512k() -> Workload:
    return Workload("long_ctx_512k", 5, 524288, 32, 8, 128, "bf16", 1e6, _cu([524288]),
                    description="one sequence of 524288 tokens, Hq=32, Hkv=8, D=128, bf16 "
                                "(Q has 2^31 elements)")


WORKLOADS = {
    "tiny_packed": tiny_packed,
    "qwen3_4b_packed": qwen3_4b_packed,
    "qwen3_8b_packed": qwen3_8b_packed,
    "qwen3_8b_padded": qwen3_8b_padded,
    "qwen3_32b_packed": qwen3_32b_packed,
    "long_ctx_512k": long_ctx_512k,
}


def names() -> list:
    return list(WORKLOADS)


def get(name: str) -> Workload:
    return WORKLOADS[name]()


# ---------------------------------------------------------------- SwiGLU / GeGLU inputs
#
# The gated MLP activation runs on [tokens, intermediate] tensors: e (gate
# projection), g (up projection) and, in the backward, dh (upstream gradient),
# each N(0, 1) from its own seed: e 6000+k, g 7000+k, dh 8000+k. Token counts are
# those of the packed RoPE batches; the intermediate sizes are the published
# Qwen3 model configurations (4B: 9728, 8B: 12288). The 524288-token case is the
# pages' 500K-context run, where 2^31-element offsets are exceeded.

@dataclass(frozen=True)
class GluWorkload:
    name: str
    number: int
    rows: int  # tokens
    cols: int  # intermediate size
    dtype: str
    description: str = ""

    @property
    def elements(self) -> int:
        return self.rows * self.cols

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def seed(self, what: str) -> int:
        return {"e": 6000, "g": 7000, "dh": 8000}[what] + self.number


GLU_WORKLOADS = {
    "glu_tiny": GluWorkload("glu_tiny", 11, 37, 40, "f32",
                            "37 rows x 40 columns, fp32 (oracle in milliseconds)"),
    "glu_qwen3_4b": GluWorkload("glu_qwen3_4b", 12, 16384, 9728, "bf16",
                                "16384 tokens x 9728 (Qwen3-4B MLP), bf16"),
    "glu_qwen3_8b": GluWorkload("glu_qwen3_8b", 13, 8554, 12288, "bf16",
                                "8554 tokens x 12288 (Qwen3-8B MLP), bf16"),
    "glu_long_512k": GluWorkload("glu_long_512k", 14, 524288, 9728, "bf16",
                                 "524288 tokens x 9728, bf16: 5.1e9 elements, 64-bit offsets"),
}


def glu_names() -> list:
    return list(GLU_WORKLOADS)


def glu_get(name: str) -> GluWorkload:
    return GLU_WORKLOADS[name]


_TORCH_DTYPES = {"f32": "float32", "bf16": "bfloat16", "f16": "float16"}


def torch_dtype(dtype: str):
    import torch

    return getattr(torch, _TORCH_DTYPES[dtype])


def make_tensor(shape, seed: int, dtype: str, device="cpu", chunk_rows: int | None = None):
    """N(0,1) tensor of ``shape`` drawn in fp32 from a generator seeded with ``seed``
    on ``device``, rounded to ``dtype``. With ``chunk_rows`` the first dimension is
    drawn in chunks of that many rows (bounded fp32 scratch for the largest
    workloads); the values then depend on the chunk size, which callers fix."""
    import torch

    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(seed))
    tdt = torch_dtype(dtype)
    if chunk_rows is None:
        return torch.randn(shape, generator=gen, dtype=torch.float32, device=dev).to(tdt)
    out = torch.empty(shape, dtype=tdt, device=dev)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen,
                                 dtype=torch.float32, device=dev).to(tdt)
    return out


def host_bits(t) -> np.ndarray:
    """A CPU tensor's storage as numpy: float32 values, or raw uint16 words."""
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)
