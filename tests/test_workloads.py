"""The seeded input recipes: shapes, length mixes and determinism."""
import numpy as np
import pytest
import torch

import workloads


@pytest.mark.parametrize("name", workloads.names())
def test_cu_seqlens_well_formed(name):
    w = workloads.get(name)
    cu = w.cu_seqlens.astype(np.int64)
    assert cu.dtype == np.int64 and cu[0] == 0 and np.all(np.diff(cu) >= 0) and cu[-1] <= w.T
    assert w.valid_tokens <= w.T
    assert w.D % 2 == 0


def test_length_mixes():
    w = workloads.get("qwen3_4b_packed")
    L = w.lengths
    assert w.T == 16384 and L.sum() == 16384
    body = L[:-1]  # the last draw is cut to hit T exactly
    assert np.all(((body >= 32) & (body <= 512)) | ((body >= 1024) & (body <= 4096)))
    w = workloads.get("qwen3_32b_packed")
    L = w.lengths
    assert w.T == 32768 and L.sum() == 32768 and np.all((L[:-1] >= 8) & (L[:-1] <= 8192))
    assert 150 < L[:-1].mean() < 450  # geometric with mean 300, clipped below at 8
    a, b = workloads.get("qwen3_8b_packed"), workloads.get("qwen3_8b_padded")
    assert np.array_equal(a.lengths, b.lengths) and a.num_seqs == 8
    assert np.all((a.lengths >= 256) & (a.lengths <= 2048))
    assert b.T == 8 * 2048 and b.valid_tokens == a.T
    w = workloads.get("long_ctx_512k")
    assert w.T * w.Hq * w.D == 2 ** 31  # Q alone has 2^31 elements
    assert w.T * (w.Hq + w.Hkv) * w.D >= 2 ** 31


def test_tensors_seeded():
    w = workloads.get("tiny_packed")
    a = workloads.make_tensor(w.shape("q"), w.seed("q"), "bf16")
    b = workloads.make_tensor(w.shape("q"), w.seed("q"), "bf16")
    c = workloads.make_tensor(w.shape("q"), w.seed("k"), "bf16")
    assert a.dtype == torch.bfloat16 and torch.equal(a, b) and not torch.equal(a, c)
    d = workloads.make_tensor((10, 3, 4), 5, "f32", chunk_rows=3)
    e = workloads.make_tensor((10, 3, 4), 5, "f32", chunk_rows=3)
    assert torch.equal(d, e)
    assert len({w.seed(k) for k in ("lengths", "q", "k", "dq", "dk")}) == 5
