"""GPU parity of the INT4/g128 GEMV (wal_int4_gemv, the LM head format)
against the CPU oracle (oracle/int4.py), through the C ABI.

Tolerance: relative L2 1e-3 (bf16 x).  x = e_j must give column j of W
bit-exactly (codes and scales are exact, and the kernel's 136-offset
baseline is formed by the same instruction sequence as the codes' sum, so it
cancels exactly); all-zero codes give exact zeros.
"""
import numpy as np
import pytest

import synth
from oracle import int4 as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_TOL = 1e-3


@pytest.fixture(scope="module")
def wal():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import ternary_hybrid_bit_amd as w
    return w


def dev():
    return torch.device("cuda:0")


def make(seed, V, inp):
    """Codes ~ uniform on [-8, 7]; scales ~ |N(0, 1)| / 64 rounded to fp16."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 50, seed]))
    q = rng.integers(-8, 8, size=(V, inp)).astype(np.int8)
    s = (np.abs(rng.standard_normal((V, inp // 128))) / 64).astype(np.float16).astype(np.float32)
    return q, s


def run(wal, blob, V, inp, xbits):
    W = torch.from_numpy(blob).to(dev())
    X = torch.from_numpy(np.ascontiguousarray(xbits).view(np.int16)).to(dev()).view(torch.bfloat16)
    y = torch.full((V,), float("nan"), dtype=torch.float32, device=dev())
    wal.wal_int4_gemv(W, V, inp, X, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("V,inp", [(1, 128), (7, 384), (1000, 4224), (4099, 4096), (300, 12288), (65, 5120), (9000, 4224),
                                   (37, 3072), (29, 2176), (17, 8320), (9, 12416)])
def test_shapes(wal, V, inp):
    q, s = make(V + inp, V, inp)
    blob = wal.wal_int4_pack(q, s)
    x, bits = synth.make_x(350, V, inp)
    print(f"int4 {V}x{inp}", flush=True)
    y = run(wal, blob, V, inp, bits[0])
    ref = I.gemv(blob, V, inp, x[0])
    err = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    print(f"  rel_l2 {err:.2e}", flush=True)
    assert err <= BF16_TOL


def test_columns_exact_and_zero(wal):
    V, inp = 300, 4224
    q, s = make(1, V, inp)
    blob = wal.wal_int4_pack(q, s)
    for j in (0, 1, 3, 4, 7, 63, 64, 127, 128, 2047, 2048, 2049, 4095, 4096, 4223):
        e = np.zeros(inp, np.float32)
        e[j] = 1.0
        y = run(wal, blob, V, inp, synth.round_bf16_bits(e))
        assert np.array_equal(y, (s[:, j // 128].astype(np.float64) * q[:, j])), j
    z = wal.wal_int4_pack(np.zeros((V, inp), np.int8), s)
    x, bits = synth.make_x(351, 0, inp)
    assert not run(wal, z, V, inp, bits[0]).any()



def test_columns_exact_partial_pass(wal):
    """A width between 2048 and 4096 (one partial pass: lanes past the width
    read zeros through out-of-range offsets): exact columns around 2048."""
    V, inp = 45, 3072
    q, s = make(4, V, inp)
    blob = wal.wal_int4_pack(q, s)
    for j in (0, 2047, 2048, 2049, 3071):
        e = np.zeros(inp, np.float32)
        e[j] = 1.0
        y = run(wal, blob, V, inp, synth.round_bf16_bits(e))
        assert np.array_equal(y, (s[:, j // 128].astype(np.float64) * q[:, j])), j

def test_qwen3_8b_head_sampled(wal):
    """The 151936 x 4096 head at full size; sampled rows against the oracle."""
    V, inp = 151936, 4096
    q, s = make(2, V, inp)
    blob = wal.wal_int4_pack(q, s)
    x, bits = synth.make_x(352, 0, inp)
    print("int4 head 151936x4096", flush=True)
    y = run(wal, blob, V, inp, bits[0])
    assert np.isfinite(y).all()
    rows = np.unique(np.concatenate([[0, 1, 2, 3, V - 1], np.random.default_rng(3).integers(0, V, 200)]))
    ref = I.gemv_rows(blob, V, inp, x[0], rows)
    err = np.linalg.norm(y[rows] - ref) / np.linalg.norm(ref)
    print(f"  sampled rel_l2 {err:.2e}", flush=True)
    assert err <= BF16_TOL
