"""GPU parity of the small-batch product Y = X W^T (wal_gemm_small) against the
CPU oracle, for both kernels (batched GEMV on the vector ALUs, MFMA) and the
automatic choice.

Tolerance: relative L2 per batch row against the float64 oracle, 1e-3 with
bf16 activations and 1e-5 with fp32 ones.  Rows X[n] = e_j must give column j
of W bit-exactly (decoded values are exact in bf16 and every product and
partial sum is exact in fp32), and the all-zero blob gives exact zeros.
"""
import ctypes
import numpy as np
import pytest

import synth
from oracle import dense as D
from oracle import format as F

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_TOL = 1e-3
F32_TOL = 1e-5


@pytest.fixture(scope="module")
def wal():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import ternary_hybrid_bit_amd as w
    return w


def dev():
    return torch.device("cuda:0")


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def run_gemm(wal, blob, info, x_f32, x_bits, mode, ldx=None, ldy=None):
    """Y [B][out] from the GPU; X and Y may be padded to ldx / ldy columns."""
    B, inp = x_f32.shape
    out = info.d.out
    ldx = ldx or inp
    ldy = ldy or out
    W = to_dev(blob)
    if x_bits is None:
        Xh = np.zeros((B, ldx), np.float32)
        Xh[:, :inp] = x_f32
        X = to_dev(Xh)
    else:
        Xh = np.zeros((B, ldx), np.uint16)
        Xh[:, :inp] = x_bits
        X = to_dev(Xh.view(np.int16)).view(torch.bfloat16)
    Y = torch.full((B, ldy), float("nan"), dtype=torch.float32, device=dev())
    nws = wal.wal_workspace_size(info, B)
    ws = torch.zeros(max(nws, 4) // 4, dtype=torch.float32, device=dev())
    wal.wal_gemm_small(info, W, X, Y, mode, ws)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy().astype(np.float64)
    if ldy > out:
        assert np.isnan(Yh[:, out:]).all(), "padding of Y was written"
    return Yh[:, :out]


def modes(wal):
    return {"valu": wal.WAL_GEMM_VALU, "mfma": wal.WAL_GEMM_MFMA, "auto": wal.WAL_GEMM_AUTO}


@pytest.fixture(scope="module")
def config3(wal):
    m = synth.config_matrix(3)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.config_x(3, batch=32)
    print("config 3: oracle for 4096x12288, batch 32", flush=True)
    ref = D.gemm(F.pack(F.from_synth(m)), x)
    return blob, info, x, bits, ref


@pytest.mark.parametrize("B", [1, 2, 3, 4, 16, 32])
@pytest.mark.parametrize("mode", ["valu", "mfma", "auto"])
def test_config3(wal, config3, B, mode):
    blob, info, x, bits, ref = config3
    print(f"config 3: B={B} mode={mode}", flush=True)
    Y = run_gemm(wal, blob, info, x[:B], bits[:B], modes(wal)[mode])
    errs = [D.rel_l2(Y[n], ref[n]) for n in range(B)]
    print(f"config 3 B={B} {mode}: worst rel_l2 = {max(errs):.3e}", flush=True)
    assert max(errs) <= BF16_TOL


@pytest.mark.parametrize("out,inp,k,P,r,sf,B", [
    (1, 128, 2, 0, 0, 0, 3),           # one row, one group, one K slice
    (129, 4224, 8, 1, 16, 1, 5),       # ragged rows, second pass of one group, fp24
    (300, 384, 4, 2, 7, 0, 17),        # two n-tiles of the MFMA kernel, odd rank
    (65, 8320, 0, 4, 64, 1, 32),       # 256 low-rank terms, no sites
    (1000, 4096, 8, 1, 16, 0, 2),
    (4099, 12288, 8, 1, 16, 0, 7),     # down_proj width, ragged rows
])
@pytest.mark.parametrize("mode", ["valu", "mfma"])
def test_shapes(wal, out, inp, k, P, r, sf, B, mode):
    m = synth.make_matrix(310, out * 3 + inp + k, out, inp, k=k, n_paths=P, rank=r, scale_fmt=sf)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(310, out + inp, inp, B)
    print(f"gemm {out}x{inp} k={k} P={P} r={r} sf={sf} B={B} {mode}", flush=True)
    Y = run_gemm(wal, blob, info, x, bits, modes(wal)[mode], ldx=inp + 64, ldy=out + 3)
    ref = D.gemm(F.pack(F.from_synth(m)), x)
    for n in range(B):
        assert D.rel_l2(Y[n], ref[n]) <= BF16_TOL, n


def test_fp32_batch_runs_per_column(wal):
    m = synth.make_matrix(311, 0, 65, 1024, k=8, n_paths=3, rank=7, scale_fmt=1)
    blob, info = wal.pack_matrix(m)
    x, _ = synth.make_x(311, 0, 1024, 3, bf16=False)
    print("gemm fp32 activations B=3", flush=True)
    ref = D.gemm(F.pack(F.from_synth(m)), x)
    for mode in ("valu", "auto"):
        Y = run_gemm(wal, blob, info, x, None, modes(wal)[mode], ldx=1028)
        for n in range(3):
            assert D.rel_l2(Y[n], ref[n]) <= F32_TOL
    with pytest.raises(wal.WalError) as ei:
        run_gemm(wal, blob, info, x, None, wal.WAL_GEMM_MFMA)
    assert ei.value.status == -9


def test_base3_batch(wal):
    m = synth.make_matrix(312, 0, 200, 5120, k=4, n_paths=2, rank=16, trit_fmt=synth.TRIT_BASE3,
                          scale_fmt=1)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(312, 0, 5120, 4)
    print("gemm base-3 B=4", flush=True)
    ref = D.gemm(F.pack(F.from_synth(m)), x)
    Y = run_gemm(wal, blob, info, x, bits, wal.WAL_GEMM_AUTO)
    for n in range(4):
        assert D.rel_l2(Y[n], ref[n]) <= BF16_TOL
    with pytest.raises(wal.WalError) as ei:
        run_gemm(wal, blob, info, x, bits, wal.WAL_GEMM_MFMA)
    assert ei.value.status == -9


@pytest.mark.parametrize("sf,P,k", [(0, 1, 8), (1, 2, 2), (0, 0, 4)])
@pytest.mark.parametrize("mode", ["valu", "mfma"])
def test_columns_bit_exact(wal, sf, P, k, mode):
    inp = 4224
    m = synth.make_matrix(313, sf * 8 + k, 200, inp, k=k, n_paths=P, rank=16, scale_fmt=sf)
    blob, info = wal.pack_matrix(m)
    W = D.dense_W(F.from_synth(m))
    cols = [0, 1, 7, 8, 15, 16, 31, 32, 63, 64, 77, 95, 96, 127, 128, 4095, 4096, 4223]
    E = np.zeros((len(cols), inp), np.float32)
    E[np.arange(len(cols)), cols] = 1.0
    bits = synth.round_bf16_bits(E)
    print(f"gemm columns sf={sf} P={P} k={k} {mode}", flush=True)
    Y = run_gemm(wal, blob, info, E, bits, modes(wal)[mode])
    for n, j in enumerate(cols):
        assert np.array_equal(Y[n], W[:, j].astype(np.float32).astype(np.float64)), j


@pytest.mark.parametrize("mode", ["valu", "mfma"])
def test_zero_case_and_determinism(wal, mode):
    m = synth.make_matrix(314, 0, 300, 4096, k=8, n_paths=1, rank=16, zero_T=True)
    m.beta[:] = 0
    m.s[:] = 0
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(314, 0, 4096, 20)
    Y = run_gemm(wal, blob, info, x, bits, modes(wal)[mode])
    assert not Y.any()
    m = synth.make_matrix(314, 1, 2048, 4096, k=8, n_paths=1, rank=16)
    blob, info = wal.pack_matrix(m)
    Y1 = run_gemm(wal, blob, info, x, bits, modes(wal)[mode])
    Y2 = run_gemm(wal, blob, info, x, bits, modes(wal)[mode])
    assert np.array_equal(Y1, Y2)


def test_rejects_bad_leading_dimensions(wal):
    m = synth.make_matrix(315, 0, 64, 256, k=8, n_paths=0)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(315, 0, 256, 2)
    W = to_dev(blob)
    X = to_dev(bits.view(np.int16)).view(torch.bfloat16)
    Y = torch.zeros((2, 64), dtype=torch.float32, device=dev())
    ws = torch.zeros(wal.wal_workspace_size(info, 2) // 4 + 1, dtype=torch.float32, device=dev())
    with pytest.raises(ValueError):   # ldx < in: the binding refuses it
        wal.wal_gemm_small(info, W, X[:, :128].contiguous(), Y, wal.WAL_GEMM_VALU, ws)
    Xn = X[:, :128].contiguous()      # and so does the library, called directly
    st = wal._lib.wal_gemm_small(ctypes.byref(info), W.data_ptr(), Xn.data_ptr(), wal.WAL_X_BF16, 2, 128,
                                 Y.data_ptr(), 64, wal.WAL_GEMM_VALU, ws.data_ptr(), ws.numel() * 4, None)
    assert st == -1
    Xp = torch.zeros((2, 260), dtype=torch.bfloat16, device=dev())
    with pytest.raises(wal.WalError) as ei:   # row pitch not a multiple of 16 bytes
        wal.wal_gemm_small(info, W, Xp, Y, wal.WAL_GEMM_VALU, ws)
    assert ei.value.status == -6
