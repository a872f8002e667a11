"""The allocation-free product (wal_gemv_noalloc) against wal_gemv.

wal_gemv_noalloc runs wal_gemv's kernels with the library's per-device scratch
array as the workspace.  Two calls in a row, the second on a smaller matrix
(so the scratch holds the first call's contents when the second starts), then
the first again: each output must equal wal_gemv's on the same inputs bit for
bit (the same kernels, every sum in a fixed order), and match the oracle
within the tolerance of its activation type (rel-L2 1e-3 for bf16, 1e-5 for
fp32, on sampled rows).
"""
import numpy as np
import pytest

import synth
from oracle import dense as D
from oracle import format as F

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wal():
    import ternary_hybrid_bit_amd as w
    return w


def dev():
    return torch.device("cuda:0")


def case(wal, seed, out, inp, k, paths, x_bf16, trit_fmt=synth.TRIT_2BIT, scale_fmt=synth.SCALE_FP16):
    m = synth.make_matrix(seed, 0, out, inp, k=k, n_paths=paths, rank=16 if paths else 0,
                          trit_fmt=trit_fmt, scale_fmt=scale_fmt)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(seed, 0, inp)
    if x_bf16:
        xt = torch.from_numpy(bits[0].view(np.int16)).to(dev()).view(torch.bfloat16)
    else:
        xt = torch.from_numpy(x[0].astype(np.float32)).to(dev())
    return m, blob, info, x[0], xt


def run_both(wal, blob, info, xt):
    W = torch.from_numpy(blob).to(dev())
    y_ref = torch.full((info.d.out,), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.zeros(max(wal.wal_workspace_size(info, 1), 4) // 4, dtype=torch.float32, device=dev())
    wal.wal_gemv(info, W, xt, y_ref, ws)
    y = torch.full((info.d.out,), float("nan"), dtype=torch.float32, device=dev())
    wal.wal_gemv_noalloc(info, W, xt, y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), y_ref.cpu().numpy()


def check_oracle(blob, x, y, tol, rows=None):
    rows = np.arange(y.size) if rows is None else rows
    ref = D.gemv_rows(blob, x, rows)
    assert D.rel_l2(y[rows], ref) <= tol


def test_noalloc_matches_gemv_twice(wal):
    print("[no_alloc] call 1: 4096 x 12288 (three passes, split into the scratch), k=8, rank 16, bf16 x",
          flush=True)
    _, b1, i1, x1, xt1 = case(wal, 801, 4096, 12288, 8, 1, True)
    y1, r1 = run_both(wal, b1, i1, xt1)
    assert np.array_equal(y1, r1)
    check_oracle(b1, x1, y1, 1e-3, np.random.default_rng(0).choice(4096, 256, replace=False))

    print("[no_alloc] call 2 (smaller): 520 x 5120, k=4, two rank-16 paths, fp32 x", flush=True)
    _, b2, i2, x2, xt2 = case(wal, 802, 520, 5120, 4, 2, False)
    y2, r2 = run_both(wal, b2, i2, xt2)
    assert np.array_equal(y2, r2)
    check_oracle(b2, x2, y2, 1e-5)

    print("[no_alloc] call 3 (smaller still): 96 x 640 base-3, fp24, k=2, one path, bf16 x", flush=True)
    _, b3, i3, x3, xt3 = case(wal, 803, 96, 640, 2, 1, True, synth.TRIT_BASE3, synth.SCALE_FP24)
    y3, r3 = run_both(wal, b3, i3, xt3)
    assert np.array_equal(y3, r3)
    check_oracle(b3, x3, y3, 1e-3)

    print("[no_alloc] call 4: the first matrix again", flush=True)
    y4, _ = run_both(wal, b1, i1, xt1)
    assert np.array_equal(y4, y1)


def test_noalloc_without_lowrank(wal):
    print("[no_alloc] 300 x 4224, k=0, no paths, bf16 x", flush=True)
    _, b, i, x, xt = case(wal, 804, 300, 4224, 0, 0, True)
    y, r = run_both(wal, b, i, xt)
    assert np.array_equal(y, r)
    check_oracle(b, x, y, 1e-3)
