"""GPU parity of the base-3 (five trits per byte) kernels against the CPU oracle.

The configuration with 27B-model shapes stores T in the base-3 container with
24-bit group scales, a per-matrix sparse count k and two binary low-rank paths.
Tolerance: relative L2 per output vector <= 1e-3 (bf16 activations).  Columns
x = e_j must come back bit-exactly, including columns on both sides of every
place where a 128-trit group boundary falls inside a lane's 80 trits.
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


def run_gemv(wal, blob, info, x_bits):
    W = to_dev(blob)
    xt = to_dev(x_bits.view(np.int16)).view(torch.bfloat16)
    y = torch.full((info.d.out,), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.zeros(max(wal.wal_workspace_size(info, 1), 4) // 4, dtype=torch.float32, device=dev())
    wal.wal_gemv(info, W, xt, y, ws)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("mid", [0, 1])
def test_config4_full(wal, mid):
    m = synth.config_matrix(4, mid)
    print(f"config 4 matrix {mid}: {m.out}x{m.inp} base-3 fp24 k={m.k} 2 paths", flush=True)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.config_x(4, mid)
    y = run_gemv(wal, blob, info, bits[0])
    ref = D.gemv(F.pack(F.from_synth(m)), x[0])
    err = D.rel_l2(y, ref)
    print(f"config 4 matrix {mid} rel_l2 = {err:.3e}", flush=True)
    assert err <= BF16_TOL


@pytest.mark.parametrize("out,inp,k,P,r,sf", [
    (1, 128, 8, 0, 0, 1),          # one row, one group
    (7, 384, 2, 1, 1, 0),          # partial pass, fp16 scales, rank 1
    (129, 5120, 8, 2, 16, 1),      # one full pass, ragged rows
    (300, 5248, 4, 1, 16, 1),      # second pass of one group
    (65, 10368, 0, 3, 7, 0),       # two passes and one group, k = 0, odd rank
    (1000, 17408, 8, 2, 16, 1),    # 27B MLP width: four passes, ragged last pass
    (2051, 640, 2, 4, 64, 1),      # many rows over several segments, 256 low-rank terms
])
def test_base3_shapes(wal, out, inp, k, P, r, sf):
    m = synth.make_matrix(400, out + inp + k, out, inp, k=k, n_paths=P, rank=r, trit_fmt=synth.TRIT_BASE3,
                          scale_fmt=sf)
    print(f"base-3 shape {out}x{inp} k={k} P={P} r={r} sf={sf}", flush=True)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(401, out + inp, inp)
    y = run_gemv(wal, blob, info, bits[0])
    ref = D.gemv(F.pack(F.from_synth(m)), x[0])
    assert D.rel_l2(y, ref) <= BF16_TOL


def test_base3_columns_bit_exact(wal):
    """Columns on both sides of the in-lane group boundaries (lane trits 16,
    32, 48, 64), of group, lane and pass boundaries, and in the last pass."""
    inp = 10368
    m = synth.make_matrix(402, 0, 260, inp, k=8, n_paths=2, rank=16, trit_fmt=synth.TRIT_BASE3,
                          scale_fmt=synth.SCALE_FP24)
    blob, info = wal.pack_matrix(m)
    W = D.dense_W(F.from_synth(m))
    cols = [0, 15, 16, 31, 32, 47, 48, 63, 64, 79, 80, 127, 128, 255, 256, 383, 384, 5119, 5120, 5247,
            10239, 10240, 10367]
    for j in cols:
        e = np.zeros(inp, np.float32)
        e[j] = 1.0
        print(f"base-3 column {j}", flush=True)
        y = run_gemv(wal, blob, info, synth.round_bf16_bits(e))
        assert np.array_equal(y, W[:, j].astype(np.float32).astype(np.float64)), j


def test_base3_zero_case(wal):
    m = synth.make_matrix(403, 0, 300, 5120, k=0, n_paths=0, zero_T=True, trit_fmt=synth.TRIT_BASE3,
                          scale_fmt=synth.SCALE_FP24)
    blob, info = wal.pack_matrix(m)
    _, bits = synth.make_x(403, 0, 5120)
    assert not run_gemv(wal, blob, info, bits[0]).any()


def test_base3_rejects_fp32_activations(wal):
    m = synth.make_matrix(404, 0, 8, 128, k=2, trit_fmt=synth.TRIT_BASE3)
    blob, info = wal.pack_matrix(m)
    W = to_dev(blob)
    x = torch.zeros(128, dtype=torch.float32, device=dev())
    y = torch.zeros(8, dtype=torch.float32, device=dev())
    with pytest.raises(wal.WalError) as ei:
        wal.wal_gemv(info, W, x, y)
    assert ei.value.status == -9


def test_grouped_mixed_2bit_and_base3(wal):
    """One grouped call over 2-bit and base-3 matrices of several classes."""
    specs = [(4096, 4096, 8, 1, 0, 0), (17408, 5120, 2, 2, 1, 1), (300, 5248, 4, 0, 1, 1),
             (1024, 4096, 8, 0, 0, 0), (5120, 17408, 4, 2, 1, 1), (129, 384, 2, 2, 0, 1)]
    Ws, xs, ys, infos, refs = [], [], [], [], []
    for i, (o, n, k, P, tf, sf) in enumerate(specs):
        m = synth.make_matrix(405, i, o, n, k=k, n_paths=P, rank=16, trit_fmt=tf, scale_fmt=sf)
        blob, info = wal.pack_matrix(m)
        x, bits = synth.make_x(405, i, n)
        Ws.append(to_dev(blob))
        xs.append(to_dev(bits[0].view(np.int16)).view(torch.bfloat16))
        ys.append(torch.full((o,), float("nan"), dtype=torch.float32, device=dev()))
        infos.append(info)
        refs.append(D.gemv(F.pack(F.from_synth(m)), x[0]))
    print("grouped: 2-bit and base-3 classes", flush=True)
    _, wsb = wal.wal_grouped_plan_size(infos)
    ws = torch.zeros(max(wsb, 4) // 4, dtype=torch.float32, device=dev())
    plan, g = wal.wal_grouped_plan(infos, Ws, xs, ys, ws, wal.WAL_X_BF16)
    assert g.n_classes >= 4
    plan_dev = to_dev(plan)
    wal.wal_gemv_grouped(g, plan_dev)
    torch.cuda.synchronize()
    for y, ref in zip(ys, refs):
        assert D.rel_l2(y.cpu().numpy(), ref) <= BF16_TOL


def test_base3_body_sampled_rows(wal):
    """The first 8 matrices of the 27B-shaped base-3 body that bench.py's
    sweep3 workload times (full shapes 17408 x 5120 and 5120 x 17408, fp24,
    two rank-16 paths, k drawn per matrix), planned as it plans them: one
    grouped plan per k class, grid from the device.  Sampled rows of every
    matrix against the oracle."""
    from ternary_hybrid_bit_amd import workloads
    items = workloads.packed_config(synth.BASE3_BODY, list(range(8)), workers=1)
    infos = [i for _, i, _ in items]
    Ws = [to_dev(b) for b, _, _ in items]
    xs = [to_dev(xb.view(np.int16)).view(torch.bfloat16) for _, _, xb in items]
    ys = [torch.full((i.d.out,), float("nan"), dtype=torch.float32, device=dev()) for i in infos]
    rng = np.random.default_rng(41)
    for k in sorted(set(int(i.d.k) for i in infos)):
        ids = [j for j, i in enumerate(infos) if int(i.d.k) == k]
        print(f"base-3 body: class k={k}, matrices {ids}", flush=True)
        inf = [infos[j] for j in ids]
        _, wsb = wal.wal_grouped_plan_size(inf)
        ws = torch.zeros(max(wsb, 4) // 4, dtype=torch.float32, device=dev())
        plan, g = wal.wal_grouped_plan(inf, [Ws[j] for j in ids], [xs[j] for j in ids], [ys[j] for j in ids], ws,
                                       wal.WAL_X_BF16)
        wal.wal_gemv_grouped(g, to_dev(plan))
        torch.cuda.synchronize()
        for j in ids:
            rows = np.sort(rng.choice(infos[j].d.out, 64, replace=False))
            x = synth.bf16_bits_to_f32(items[j][2]).astype(np.float64)
            ref = D.gemv_rows(items[j][0], x, rows)
            assert D.rel_l2(ys[j].cpu().numpy()[rows].astype(np.float64), ref) <= BF16_TOL, (k, j)
