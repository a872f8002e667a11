"""GPU parity of libwal's HIP kernels against the CPU oracle, through the C ABI.

Tolerances (per output vector, relative L2 against the float64 oracle):
1e-3 with bf16 activations and 1e-5 with fp32 activations.  Columns x = e_j
must come back bit-exactly (every W entry and partial sum is a multiple of
2^-24 below 2^-2, so fp32 holds them exactly whatever the order), and the
all-zero case returns exact zeros.
"""
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


def x_tensor(x_f32, x_bits):
    if x_bits is None:
        return to_dev(x_f32.astype(np.float32))
    return to_dev(x_bits.view(np.int16)).view(torch.bfloat16)


def run_gemv(wal, blob, info, x_f32, x_bits):
    W = to_dev(blob)
    xt = x_tensor(x_f32, x_bits)
    y = torch.full((info.d.out,), float("nan"), dtype=torch.float32, device=dev())
    nws = wal.wal_workspace_size(info, 1)
    ws = torch.zeros(max(nws, 4) // 4, dtype=torch.float32, device=dev())
    wal.wal_gemv(info, W, xt, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


def case(wal, m, xbf16=True, seed=0):
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(200 + seed, m.out + m.inp, m.inp, bf16=xbf16)
    y = run_gemv(wal, blob, info, x[0], None if bits is None else bits[0])
    ref = D.gemv(F.pack(F.from_synth(m)), x[0])
    return y, ref


def test_config0_fp32(wal):
    m = synth.config_matrix(0)
    blob, info = wal.pack_matrix(m)
    x, _ = synth.config_x(0)
    print("config 0: 256x512 fp32 x", flush=True)
    y = run_gemv(wal, blob, info, x[0], None)
    ref = D.gemv(F.pack(F.from_synth(m)), x[0])
    assert D.rel_l2(y, ref) <= F32_TOL


def test_config1_bf16(wal):
    m = synth.config_matrix(1)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.config_x(1)
    print("config 1: 12288x4096 rank-16 bf16 x", flush=True)
    y = run_gemv(wal, blob, info, x[0], bits[0])
    ref = D.gemv(F.pack(F.from_synth(m)), x[0])
    err = D.rel_l2(y, ref)
    print(f"config 1 rel_l2 = {err:.3e}", flush=True)
    assert err <= BF16_TOL


@pytest.mark.parametrize("out,inp,k,P,r,sf,xbf16", [
    (1, 128, 8, 0, 0, 0, True),          # single row, single group
    (7, 384, 2, 1, 1, 0, True),          # partial pass, rank 1
    (129, 4096, 4, 2, 16, 1, True),      # ragged tiles, fp24 scales on 2-bit codes
    (1000, 4224, 8, 1, 16, 0, True),     # second pass of one group
    (300, 8320, 0, 4, 64, 0, True),      # four paths of rank 64 (256 low-rank terms)
    (4099, 12288, 8, 1, 16, 0, True),    # down_proj width, three passes, ragged rows
    (65, 1024, 8, 3, 7, 1, False),       # fp32 activations, odd rank
    (96, 4224, 8, 2, 8, 0, False),       # fp32 activations, two paths of rank 8, two passes
    (513, 4096, 2, 0, 0, 1, False),
])
def test_shapes(wal, out, inp, k, P, r, sf, xbf16):
    m = synth.make_matrix(300, out * 3 + inp + k, out, inp, k=k, n_paths=P, rank=r, scale_fmt=sf)
    print(f"shape {out}x{inp} k={k} P={P} r={r} sf={sf} bf16={xbf16}", flush=True)
    y, ref = case(wal, m, xbf16)
    assert D.rel_l2(y, ref) <= (BF16_TOL if xbf16 else F32_TOL)


@pytest.mark.parametrize("sf,P", [(0, 1), (1, 2)])
def test_columns_bit_exact(wal, sf, P):
    m = synth.make_matrix(301, sf, 200, 4224, k=8, n_paths=P, rank=16, scale_fmt=sf)
    blob, info = wal.pack_matrix(m)
    L = F.from_synth(m)
    W = D.dense_W(L)
    for j in [0, 1, 77, 128, 4095, 4096, 4223]:
        e = np.zeros(4224, np.float32)
        e[j] = 1.0
        bits = synth.round_bf16_bits(e)
        print(f"column {j} sf={sf}", flush=True)
        y = run_gemv(wal, blob, info, e, bits)
        assert np.array_equal(y, W[:, j].astype(np.float32).astype(np.float64)), j


@pytest.mark.parametrize("out,inp,k,P,r,sf,b3", [
    (1000, 4224, 8, 1, 16, 0, False),    # two passes, the second of one group
    (300, 12288, 2, 0, 0, 1, False),     # three passes, no low-rank path
    (129, 8320, 4, 2, 7, 0, False),
    (200, 17408, 4, 2, 16, 1, True),     # base-3, four passes, ragged last pass
])
def test_wide_single_split_and_whole(wal, out, inp, k, P, r, sf, b3):
    """A matrix wider than one pass runs its passes in separate workgroups
    when the workspace holds the per-pass partial sums, else every workgroup
    takes all passes of its rows: both agree with the oracle."""
    m = synth.make_matrix(305, out + inp + k, out, inp, k=k, n_paths=P, rank=r, scale_fmt=sf,
                          trit_fmt=synth.TRIT_BASE3 if b3 else synth.TRIT_2BIT)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(305, out, inp)
    ref = D.gemv(F.pack(F.from_synth(m)), x[0])
    W, xt = to_dev(blob), x_tensor(x[0], bits[0])
    full = wal.wal_workspace_size(info, 1)
    # the workspace up to the end of its low-rank part (the zero region, the
    # partials): no room for the passes' partial sums
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    zonly = wal.WAL_WS_ZERO_BYTES + up(max(4 * P * r * ((inp + 4095) // 4096), 8 * P * r * ((inp + 8191) // 8192)))
    for nbytes in (full, zonly):
        print(f"wide {out}x{inp} k={k} P={P} base3={b3} workspace {nbytes} B", flush=True)
        y = torch.full((out,), float("nan"), dtype=torch.float32, device=dev())
        ws = torch.zeros(nbytes // 4, dtype=torch.float32, device=dev()) if nbytes else None
        wal.wal_gemv(info, W, xt, y, ws)
        torch.cuda.synchronize()
        assert D.rel_l2(y.cpu().numpy().astype(np.float64), ref) <= BF16_TOL, nbytes


def test_zero_case_returns_exact_zero(wal):
    m = synth.make_matrix(302, 0, 300, 4096, k=0, n_paths=0, zero_T=True)
    y, _ = case(wal, m)
    assert not y.any()
    m = synth.make_matrix(302, 1, 300, 4096, k=8, n_paths=1, rank=16, zero_T=True)
    m.beta[:] = 0
    m.s[:] = 0
    y, _ = case(wal, m)
    assert not y.any()


def test_deterministic(wal):
    m = synth.make_matrix(303, 0, 2048, 4096, k=8, n_paths=1, rank=16)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(303, 0, 4096)
    y1 = run_gemv(wal, blob, info, x[0], bits[0])
    y2 = run_gemv(wal, blob, info, x[0], bits[0])
    assert np.array_equal(y1, y2)


def grouped(wal, items, x_bf16=True):
    """items: [(blob, info, x_bits or x_f32)] -> list of y (numpy)."""
    Ws = [to_dev(b) for b, _, _ in items]
    xs = [to_dev(xb.view(np.int16)).view(torch.bfloat16) if x_bf16 else to_dev(xb) for _, _, xb in items]
    ys = [torch.full((i.d.out,), float("nan"), dtype=torch.float32, device=dev()) for _, i, _ in items]
    infos = [i for _, i, _ in items]
    _, wsb = wal.wal_grouped_plan_size(infos, 0, wal.WAL_X_BF16 if x_bf16 else wal.WAL_X_F32)
    ws = torch.zeros(max(wsb, 4) // 4, dtype=torch.float32, device=dev())
    plan, g = wal.wal_grouped_plan(infos, Ws, xs, ys, ws, wal.WAL_X_BF16 if x_bf16 else wal.WAL_X_F32)
    plan_dev = to_dev(plan)
    wal.wal_gemv_grouped(g, plan_dev)
    torch.cuda.synchronize()
    return [y.cpu().numpy().astype(np.float64) for y in ys], (Ws, xs, ys, ws, plan_dev, g)


def test_grouped_mixed_shapes(wal):
    shapes = [(4096, 4096, 8, 1), (1024, 4096, 8, 0), (300, 12288, 8, 1), (129, 384, 2, 2),
              (1, 128, 4, 0), (2000, 4224, 0, 1), (12288, 4096, 8, 1)]
    items, refs = [], []
    for i, (o, n, k, P) in enumerate(shapes):
        m = synth.make_matrix(304, i, o, n, k=k, n_paths=P, rank=16)
        blob, info = wal.pack_matrix(m)
        x, bits = synth.make_x(304, i, n)
        items.append((blob, info, bits[0]))
        refs.append(D.gemv(F.pack(F.from_synth(m)), x[0]))
    print("grouped: 7 mixed shapes", flush=True)
    ys, _ = grouped(wal, items)
    for y, ref in zip(ys, refs):
        assert D.rel_l2(y, ref) <= BF16_TOL


def test_grouped_full_sweep_sampled(wal):
    """The 252-matrix Qwen3-8B-shaped sweep at full size, in the launch
    configuration the benchmark times; sampled rows of every matrix are
    checked against the oracle one by one, and a second launch must
    reproduce the first bit for bit."""
    from ternary_hybrid_bit_amd import workloads
    print("sweep: generating 252 matrices", flush=True)
    items = workloads.sweep()
    print("sweep: launching", flush=True)
    ys, keep = grouped(wal, items)
    Ws, xs, ys_dev, ws, plan_dev, g = keep
    wal.wal_gemv_grouped(g, plan_dev)
    torch.cuda.synchronize()
    for i, (y, yd) in enumerate(zip(ys, ys_dev)):
        assert np.array_equal(y, yd.cpu().numpy().astype(np.float64)), i
    rng = np.random.default_rng(11)
    worst = 0.0
    for i, (blob, info, xb) in enumerate(items):
        out = info.d.out
        rows = np.unique(np.concatenate([[0, out - 1], rng.integers(0, out, 6)]))
        x = synth.bf16_bits_to_f32(xb)
        ref = D.gemv_rows(blob, x, rows)
        err = D.rel_l2(ys[i][rows], ref)
        worst = max(worst, err)
        assert err <= BF16_TOL, (i, err)
        assert np.isfinite(ys[i]).all()
    print(f"sweep sampled worst rel_l2 = {worst:.3e}", flush=True)
