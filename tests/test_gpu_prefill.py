"""GPU parity of the prefill-size product Y = X W^T (wal_gemm_prefill) against
the CPU oracle.

The kernel tiles Y into 256 (fp16 scales) or 128 (fp24) rows x 64 batch rows; with few tiles it splits
the K dimension and a reduce adds the splits, so the cases below cover both
launches (split and whole), ragged row blocks and batch chunks, every site
count, both scale formats and up to 256 low-rank terms.

Tolerance: relative L2 per batch row against the float64 oracle, 1e-3 (bf16
activations).  Rows X[n] = e_j give column j of W bit-exactly (decoded values
are exact in bf16; every product and partial sum is exact in fp32), the
all-zero blob gives exact zeros, and two calls agree bit for bit.
"""
import numpy as np
import pytest

import synth
from oracle import dense as D
from oracle import format as F

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


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def split_count(out, inp, B, sf=0):
    """K splits of the launch (the library's rule, restated for the test
    names): while the tiles (256 x 64 with fp16 scales, 128 x 64 with fp24)
    number fewer than 256, up to one per 2-group sweep."""
    rows = 256 if sf == 0 else 128
    tiles = ((out + rows - 1) // rows) * ((B + 63) // 64)
    return 1 if tiles >= 256 else min((inp // 128 + 1) // 2, -(-256 // tiles))


def run_prefill(wal, W, info, bits, ldx=None, ldy=None):
    """Y [B][out] from the GPU; W a device blob, bits [B][in] bf16 patterns."""
    B, inp = bits.shape
    out = info.d.out
    ldx = ldx or inp
    ldy = ldy or out
    Xh = np.zeros((B, ldx), np.uint16)
    Xh[:, :inp] = bits
    X = to_dev(Xh.view(np.int16)).view(torch.bfloat16)
    Y = torch.full((B, ldy), float("nan"), dtype=torch.float32, device=dev())
    nws = wal.wal_prefill_workspace_size(info, B)
    ws = torch.full((max(nws, 4) // 4,), float("nan"), dtype=torch.float32, device=dev()) if nws else None
    wal.wal_gemm_prefill(info, W, X, Y, ws)
    torch.cuda.synchronize()
    Yh = Y.cpu().numpy().astype(np.float64)
    if ldy > out:
        assert np.isnan(Yh[:, out:]).all(), "padding of Y was written"
    return Yh[:, :out]


@pytest.mark.parametrize("out,inp,k,P,r,sf,B", [
    (300, 1024, 8, 1, 16, 0, 64),       # four splits of one sweep each
    (129, 4224, 4, 2, 7, 1, 96),        # ragged rows, fp24, 17 splits, last sweep of one group
    (1000, 4096, 0, 4, 64, 0, 200),     # 256 low-rank terms, ragged batch chunk
    (8200, 1024, 2, 2, 16, 1, 1000),    # fp24: 65 x 16 tiles, whole K, ragged rows and chunk
    (4099, 12288, 8, 1, 16, 0, 70),     # down_proj width, ragged rows
    (8192, 1152, 8, 0, 0, 0, 1024),     # whole K, no low-rank path, odd sweep count, last sweep of one group
    (16, 128, 2, 1, 1, 0, 33),          # one row tile, one group, rank 1
])
def test_shapes(wal, out, inp, k, P, r, sf, B):
    m = synth.make_matrix(320, out * 3 + inp + k, out, inp, k=k, n_paths=P, rank=r, scale_fmt=sf)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(320, out + inp, inp, B)
    print(f"prefill {out}x{inp} k={k} P={P} r={r} sf={sf} B={B} splits={split_count(out, inp, B, sf)}", flush=True)
    Y = run_prefill(wal, to_dev(blob), info, bits, ldx=inp + 64, ldy=out + 3)
    ref = D.gemm(F.pack(F.from_synth(m)), x)
    errs = [D.rel_l2(Y[n], ref[n]) for n in range(B)]
    print(f"  worst rel_l2 = {max(errs):.3e}", flush=True)
    assert max(errs) <= BF16_TOL


@pytest.fixture(scope="module")
def config3(wal):
    m = synth.config_matrix(3)
    blob, info = wal.pack_matrix(m)
    return m, blob, info


@pytest.mark.parametrize("B", [64, 2048])
def test_down_proj_full_size(wal, config3, B):
    """The 4096 x 12288 down_proj matrix at batch 64 (split K) and 2048 (the
    benchmark's launch): every output of sampled batch rows (first, last,
    chunk edges) against the oracle."""
    m, blob, info = config3
    x, bits = synth.make_x(3, 0, 12288, B)
    print(f"prefill 4096x12288 B={B} splits={split_count(4096, 12288, B)}", flush=True)
    Y = run_prefill(wal, to_dev(blob), info, bits)
    rows = sorted({0, 1, 31, 32, B // 2 + 5, B - 2, B - 1})
    ref = D.gemm(F.pack(F.from_synth(m)), x[rows])
    worst = 0.0
    for i, n in enumerate(rows):
        err = D.rel_l2(Y[n], ref[i])
        worst = max(worst, err)
        assert err <= BF16_TOL, (n, err)
    assert np.isfinite(Y).all()
    print(f"  sampled worst rel_l2 = {worst:.3e}", flush=True)


@pytest.mark.parametrize("sf,P,k,out,B", [(0, 1, 8, 200, 18), (1, 2, 2, 2048, 256), (0, 0, 4, 300, 40),
                                          (1, 1, 8, 8192, 1024)])
def test_columns_bit_exact(wal, sf, P, k, out, B):
    inp = 4224
    m = synth.make_matrix(321, sf * 8 + k, out, inp, k=k, n_paths=P, rank=16, scale_fmt=sf)
    blob, info = wal.pack_matrix(m)
    W = D.dense_W(F.from_synth(m))
    base = [0, 1, 7, 8, 15, 16, 31, 32, 63, 64, 77, 95, 96, 127, 128, 4095, 4096, 4223]
    cols = (base * (B // len(base) + 1))[:B]
    E = np.zeros((B, inp), np.float32)
    E[np.arange(B), cols] = 1.0
    bits = synth.round_bf16_bits(E)
    print(f"prefill columns {out}x{inp} sf={sf} P={P} k={k} B={B} splits={split_count(out, inp, B, sf)}", flush=True)
    Y = run_prefill(wal, to_dev(blob), info, bits)
    for n, j in enumerate(cols):
        assert np.array_equal(Y[n], W[:, j].astype(np.float32).astype(np.float64)), (n, j)


def test_zero_case_and_determinism(wal):
    m = synth.make_matrix(322, 0, 300, 4096, k=8, n_paths=1, rank=16, zero_T=True)
    m.beta[:] = 0
    m.s[:] = 0
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(322, 0, 4096, 100)
    print("prefill zero blob B=100", flush=True)
    assert not run_prefill(wal, to_dev(blob), info, bits).any()
    m = synth.make_matrix(322, 1, 8192, 4096, k=8, n_paths=1, rank=16)
    blob, info = wal.pack_matrix(m)
    W = to_dev(blob)
    for B in (100, 1024):   # split and whole
        print(f"prefill determinism B={B}", flush=True)
        Y1 = run_prefill(wal, W, info, bits if B == 100 else synth.make_x(322, 2, 4096, B)[1])
        Y2 = run_prefill(wal, W, info, bits if B == 100 else synth.make_x(322, 2, 4096, B)[1])
        assert np.array_equal(Y1, Y2)


def test_max_batch(wal):
    """The largest batch the entry point takes (WAL_MAX_PREFILL_BATCH rows of
    X) on a ragged 520 x 4224 matrix: sampled batch rows, every output,
    against the oracle, and Y finite throughout."""
    B = wal.WAL_MAX_PREFILL_BATCH
    m = synth.make_matrix(324, 0, 520, 4224, k=8, n_paths=2, rank=16)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(324, 0, 4224, B)
    print(f"prefill 520x4224 B={B} splits={split_count(520, 4224, B)}", flush=True)
    Y = run_prefill(wal, to_dev(blob), info, bits)
    assert np.isfinite(Y).all()
    rows = sorted({0, 63, 64, 8191, 8192, B - 65, B - 1})
    ref = D.gemm(F.pack(F.from_synth(m)), x[rows])
    for i, n in enumerate(rows):
        assert D.rel_l2(Y[n], ref[i]) <= BF16_TOL, n


def test_unsupported_inputs(wal):
    m = synth.make_matrix(323, 0, 64, 5120, k=4, n_paths=1, rank=16, trit_fmt=synth.TRIT_BASE3)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(323, 0, 5120, 64)
    with pytest.raises(wal.WalError) as ei:
        run_prefill(wal, to_dev(blob), info, bits)
    assert ei.value.status == -9
    m = synth.make_matrix(323, 1, 64, 1024, k=4, n_paths=1, rank=16)
    blob, info = wal.pack_matrix(m)
    X = torch.zeros((64, 1024), dtype=torch.float32, device=dev())
    Y = torch.zeros((64, 64), dtype=torch.float32, device=dev())
    ws = torch.zeros(wal.wal_prefill_workspace_size(info, 64) // 4, dtype=torch.float32, device=dev())
    with pytest.raises(wal.WalError) as ei:
        wal.wal_gemm_prefill(info, to_dev(blob), X, Y, ws)
    assert ei.value.status == -9
