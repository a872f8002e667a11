"""GPU parity of the INT5/g128 GEMV (wal_int5_gemv, the RC1 card's packed
INT5 LM head) against the CPU oracle (oracle/int5.py), through the C ABI.

Tolerance: relative L2 1e-3 (bf16 x).  x = e_j must give column j of W
bit-exactly (codes and scales are exact, and the kernel's 144-offset
baseline is formed by the same instruction sequence as the codes' sum, so it
cancels exactly); all-zero codes give exact zeros.
"""
import numpy as np
import pytest

import synth
from oracle import int5 as I

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
    """Codes uniform on [-16, 15]; scales |N(0, 1)| / 64 rounded to fp16."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 55, seed]))
    q = rng.integers(-16, 16, size=(V, inp), dtype=np.int8)
    s = (np.abs(rng.standard_normal((V, inp // 128))) / 64).astype(np.float16).astype(np.float32)
    return q, s


def run(wal, blob, V, inp, xbits):
    W = torch.from_numpy(blob).to(dev())
    X = torch.from_numpy(np.ascontiguousarray(xbits).view(np.int16)).to(dev()).view(torch.bfloat16)
    y = torch.full((V,), float("nan"), dtype=torch.float32, device=dev())
    wal.wal_int5_gemv(W, V, inp, X, y)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("V,inp", [(1, 128), (7, 384), (1000, 4224), (4099, 4096), (300, 12288), (65, 5120), (9000, 4224),
                                   (33, 8192), (37, 3072), (29, 2176), (17, 8320), (9, 12416)])
def test_shapes(wal, V, inp):
    q, s = make(V + inp, V, inp)
    blob = wal.wal_int5_pack(q, s)
    x, bits = synth.make_x(355, V, inp)
    print(f"int5 {V}x{inp}", flush=True)
    y = run(wal, blob, V, inp, bits[0])
    ref = I.gemv(blob, V, inp, x[0])
    err = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    print(f"  rel_l2 {err:.2e}", flush=True)
    assert err <= BF16_TOL


def test_columns_exact_and_zero(wal):
    V, inp = 300, 4224
    q, s = make(1, V, inp)
    q[:, :8] = np.array([-16, 15, -1, 0, 1, -8, 7, 8])   # the range's ends in the first pairs
    blob = wal.wal_int5_pack(q, s)
    for j in (0, 1, 2, 3, 5, 6, 7, 12, 13, 63, 64, 127, 128, 2047, 2048, 2049, 4095, 4096, 4223):
        e = np.zeros(inp, np.float32)
        e[j] = 1.0
        y = run(wal, blob, V, inp, synth.round_bf16_bits(e))
        assert np.array_equal(y, (s[:, j // 128].astype(np.float64) * q[:, j])), j
    z = wal.wal_int5_pack(np.zeros((V, inp), np.int8), s)
    x, bits = synth.make_x(356, 0, inp)
    assert not run(wal, z, V, inp, bits[0]).any()



def test_columns_exact_partial_pass(wal):
    """A width between 2048 and 4096 (one partial pass: lanes past the width
    read zeros through out-of-range offsets): exact columns around 2048."""
    V, inp = 45, 3072
    q, s = make(4, V, inp)
    blob = wal.wal_int5_pack(q, s)
    for j in (0, 2047, 2048, 2049, 3071):
        e = np.zeros(inp, np.float32)
        e[j] = 1.0
        y = run(wal, blob, V, inp, synth.round_bf16_bits(e))
        assert np.array_equal(y, (s[:, j // 128].astype(np.float64) * q[:, j])), j

def test_every_column_of_a_group(wal):
    """All 128 columns of one scale group (every bit offset of the 5-bit
    stream inside a lane's window) on a small matrix, exactly."""
    V, inp = 17, 256
    q, s = make(3, V, inp)
    blob = wal.wal_int5_pack(q, s)
    for j in range(128, 256):
        e = np.zeros(inp, np.float32)
        e[j] = 1.0
        y = run(wal, blob, V, inp, synth.round_bf16_bits(e))
        assert np.array_equal(y, (s[:, 1].astype(np.float64) * q[:, j])), j


def test_27b_head_sampled(wal):
    """A 248320 x 5120 head (the 27B model's vocabulary and width) at full
    size; sampled rows against the oracle."""
    V, inp = 248320, 5120
    q, s = make(2, V, inp)
    blob = wal.wal_int5_pack(q, s)
    del q
    x, bits = synth.make_x(357, 0, inp)
    print("int5 head 248320x5120", flush=True)
    y = run(wal, blob, V, inp, bits[0])
    assert np.isfinite(y).all()
    rows = np.unique(np.concatenate([[0, 1, 2, 3, V - 1], np.random.default_rng(4).integers(0, V, 200)]))
    ref = I.gemv_rows(blob, V, inp, x[0], rows)
    err = np.linalg.norm(y[rows] - ref) / np.linalg.norm(ref)
    print(f"  sampled rel_l2 {err:.2e}", flush=True)
    assert err <= BF16_TOL
