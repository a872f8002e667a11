"""The Python binding rejects bad device arguments before calling the library.

The C ABI takes bare pointers: it cannot see a buffer's dtype, size or device.
The binding therefore checks each of them, and these CPU-only tests show that
every check raises before anything reaches the library (no GPU is needed: the
device check comes last, so CPU tensors exercise all the others).
"""
import numpy as np
import pytest
import torch

import synth
import ternary_hybrid_bit_amd as wal
from ternary_hybrid_bit_amd import workloads


@pytest.fixture(scope="module")
def blob():
    m = synth.make_matrix(91, 0, 64, 256, k=8, n_paths=1, rank=16)
    b, info = wal.pack_matrix(m)
    return torch.from_numpy(b), info


def _x(n, dt=torch.bfloat16):
    return torch.zeros(n, dtype=dt)


def test_gemv_checks(blob):
    W, info = blob
    out, inp = info.d.out, info.d.in_
    y = torch.zeros(out, dtype=torch.float32)
    with pytest.raises(TypeError):       # numpy weights (a host pointer)
        wal.wal_gemv(info, W.numpy(), _x(inp), y)
    with pytest.raises(ValueError):      # short weights
        wal.wal_gemv(info, W[:-1], _x(inp), y)
    with pytest.raises(TypeError):       # fp16 activations
        wal.wal_gemv(info, W, _x(inp, torch.float16), y)
    with pytest.raises(ValueError):      # short activations
        wal.wal_gemv(info, W, _x(inp - 1), y)
    with pytest.raises(ValueError):      # strided activations
        wal.wal_gemv(info, W, _x(2 * inp)[::2], y)
    with pytest.raises(TypeError):       # bf16 output
        wal.wal_gemv(info, W, _x(inp), y.to(torch.bfloat16))
    with pytest.raises(ValueError):      # short output
        wal.wal_gemv(info, W, _x(inp), y[:-1])
    with pytest.raises(TypeError):       # workspace not a tensor
        wal.wal_gemv(info, W, _x(inp), y, ws=np.zeros(64, np.float32))
    with pytest.raises(ValueError, match="GPU"):   # everything right, but on the CPU
        wal.wal_gemv(info, W, _x(inp), y)


def test_gemm_checks(blob):
    W, info = blob
    out, inp = info.d.out, info.d.in_
    X = torch.zeros((4, inp), dtype=torch.bfloat16)
    Y = torch.zeros((4, out), dtype=torch.float32)
    for fn in (wal.wal_gemm_small, wal.wal_gemm_prefill):
        with pytest.raises(ValueError):      # 1-D X
            fn(info, W, X[0], Y)
        with pytest.raises(ValueError):      # too few columns
            fn(info, W, X[:, :inp - 128], Y)
        with pytest.raises(ValueError):      # too few output rows
            fn(info, W, X, Y[:3])
        with pytest.raises(TypeError):       # int8 X
            fn(info, W, X.to(torch.int8), Y)
        with pytest.raises(TypeError):       # bf16 Y
            fn(info, W, X, Y.to(torch.bfloat16))
        with pytest.raises(ValueError):      # short weights
            fn(info, W[:100], X, Y)
        with pytest.raises(ValueError, match="GPU"):
            fn(info, W, X, Y)
    with pytest.raises(ValueError):          # batch above the small-batch limit
        wal.wal_gemm_small(info, W, torch.zeros((wal.WAL_MAX_BATCH + 1, inp), dtype=torch.bfloat16),
                           torch.zeros((wal.WAL_MAX_BATCH + 1, out), dtype=torch.float32))


def test_grouped_checks(blob):
    W, info = blob
    out, inp = info.d.out, info.d.in_
    x, y = _x(inp), torch.zeros(out, dtype=torch.float32)
    with pytest.raises(ValueError):          # lengths differ
        wal.wal_grouped_plan([info], [W, W], [x], [y], None, wal.WAL_X_BF16, grid=4)
    with pytest.raises(TypeError):           # fp32 x for a bf16 plan
        wal.wal_grouped_plan([info], [W], [x.float()], [y], None, wal.WAL_X_BF16, grid=4)
    with pytest.raises(ValueError):          # short output
        wal.wal_grouped_plan([info], [W], [x], [y[:5]], None, wal.WAL_X_BF16, grid=4)
    with pytest.raises(ValueError, match="GPU"):
        wal.wal_grouped_plan([info], [W], [x], [y], None, wal.WAL_X_BF16, grid=4)
    g = wal.wal_grouped_info()
    g.plan_bytes = 4096
    with pytest.raises(ValueError):          # plan shorter than its size
        wal.wal_gemv_grouped(g, torch.zeros(1024, dtype=torch.uint8))
    with pytest.raises(ValueError):
        wal.wal_gemv_grouped_seq([(g, torch.zeros(1024, dtype=torch.uint8))])


def test_head_embed_rotate_checks():
    V, inp = 8, 256
    x, y = _x(inp), torch.zeros(V, dtype=torch.float32)
    for fn, size in ((wal.wal_int4_gemv, wal.wal_int4_size), (wal.wal_int5_gemv, wal.wal_int5_size)):
        W = torch.zeros(size(V, inp), dtype=torch.uint8)
        with pytest.raises(ValueError):      # short matrix
            fn(W[:-1], V, inp, x, y)
        with pytest.raises(ValueError):      # short x
            fn(W, V, inp, x[:-1], y)
        with pytest.raises(ValueError):      # short y
            fn(W, V, inp, x, y[:-1])
        with pytest.raises(TypeError):       # fp16 x
            fn(W, V, inp, x.half(), y)
        with pytest.raises(ValueError, match="GPU"):
            fn(W, V, inp, x, y)
    E = torch.zeros(wal.wal_int3_size(V, inp), dtype=torch.uint8)
    ids = torch.zeros(3, dtype=torch.int32)
    out = torch.zeros((3, inp), dtype=torch.bfloat16)
    with pytest.raises(TypeError):           # int64 ids
        wal.wal_embed_rows(E, 3, V, inp, ids.long(), out)
    with pytest.raises(ValueError):          # too few output rows
        wal.wal_embed_rows(E, 3, V, inp, ids, out[:2])
    with pytest.raises(ValueError):          # narrow output
        wal.wal_embed_rows(E, 3, V, inp, ids, out[:, :128])
    with pytest.raises(ValueError):          # INT4 table size for an INT3 buffer
        wal.wal_embed_rows(E, 4, V, inp, ids, out)
    with pytest.raises(ValueError):
        wal.wal_embed_rows(E, 5, V, inp, ids, out)
    with pytest.raises(ValueError, match="GPU"):
        wal.wal_embed_rows(E, 3, V, inp, ids, out)
    X = torch.zeros((2, inp), dtype=torch.float32)
    with pytest.raises(TypeError):
        wal.wal_rotate_h128(X.half(), X)
    with pytest.raises(ValueError):          # fewer output rows
        wal.wal_rotate_h128(X, X[:1])
    with pytest.raises(ValueError, match="GPU"):
        wal.wal_rotate_h128(X, X)


def test_pack_workers_rule(monkeypatch):
    """Parent + packing workers stay within 16 processes, and a profiled
    process packs in-process (the profiler would follow every child)."""
    for k in [k for k in list(__import__("os").environ) if k.startswith("ROCPROF")]:
        monkeypatch.delenv(k)
    monkeypatch.delenv("WAL_PACK_WORKERS", raising=False)
    monkeypatch.setenv("LD_PRELOAD", "")
    assert 1 <= workloads.default_workers() <= workloads.MAX_WORKERS <= 15
    monkeypatch.setenv("WAL_PACK_WORKERS", "64")
    assert workloads.default_workers() == workloads.MAX_WORKERS
    monkeypatch.setenv("WAL_PACK_WORKERS", "1")
    assert workloads.default_workers() == 1
    monkeypatch.delenv("WAL_PACK_WORKERS")
    monkeypatch.setenv("ROCPROF_KERNEL_TRACE", "1")
    assert workloads.under_profiler() and workloads.default_workers() == 1


def test_sweep_cache_roundtrip(tmp_path):
    items = workloads.packed_config(2, [1, 2], workers=1)
    path = str(tmp_path / "c.npz")
    workloads._save(path, items)
    back = workloads._load(path)
    assert len(back) == len(items)
    for (b0, i0, x0), (b1, i1, x1) in zip(items, back):
        assert np.array_equal(b0, b1) and np.array_equal(x0, x1)
        assert i0.total_bytes == i1.total_bytes and i0.algorithmic_bytes == i1.algorithmic_bytes
