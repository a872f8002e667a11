"""GPU tests of the normalised Hadamard-128 rotation (wal_rotate_h128) against
the CPU oracle (oracle/rotation.py), and of products of a rotated blob.

* fp32 output: every element within the fp32 rounding bound of the float64
  rotation of the same input (8 add or subtract stages and one multiply:
  |err| <= 1e-6 * sum_j |x_j| / sqrt(128) over the element's group);
* bf16 output: every element is the float64 value rounded to nearest even,
  except where that value lies within the fp32 bound of a rounding midpoint
  (then either neighbour is accepted), and such elements are rare;
* special vectors: a basis vector gives +-fp32(1/sqrt(128)) exactly;
* in place, ragged row counts, padded pitches, fp32 and bf16 inputs;
* a rotated product: wal_gemv of a base-3 / fp24 blob on the rotated bf16 x
  matches the oracle product on the oracle's rotated, bf16-rounded x
  (relative L2 <= 1e-3, as for every bf16 product).
"""
import numpy as np
import pytest

import synth
from oracle import dense as D
from oracle import format as F
from oracle import rotation as Rt

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wal():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import ternary_hybrid_bit_amd as w
    return w


def dev():
    return torch.device("cuda:0")


def bf16_rne(v):
    """float64 -> bf16 bit patterns, round to nearest even (via float32; the
    values here are float32-exact or checked against the bound separately)."""
    return synth.round_bf16_bits(np.asarray(v, dtype=np.float32))


def group_bound(x, rows, inp):
    g = np.abs(x.reshape(rows, inp // 128, 128)).sum(axis=2) / np.sqrt(128)
    return np.repeat(g, 128, axis=1).reshape(rows, inp) * 1e-6


def run(wal, x_host, x_bf16, out_bf16, ldx=None, ldo=None, inplace=False):
    rows, inp = x_host.shape
    ldx = ldx or inp
    ldo = ldo or inp
    if x_bf16:
        xb = np.zeros((rows, ldx), np.uint16)
        xb[:, :inp] = synth.round_bf16_bits(x_host)
        X = torch.from_numpy(xb.view(np.int16)).to(dev()).view(torch.bfloat16)
    else:
        xf = np.zeros((rows, ldx), np.float32)
        xf[:, :inp] = x_host
        X = torch.from_numpy(xf).to(dev())
    if inplace:
        O = X
    elif out_bf16:
        O = torch.full((rows, ldo), float("nan"), dtype=torch.bfloat16, device=dev())
    else:
        O = torch.full((rows, ldo), float("nan"), dtype=torch.float32, device=dev())
    wal.wal_rotate_h128(X[:, :inp] if not inplace else X[:, :inp], O[:, :inp])
    torch.cuda.synchronize()
    o = O.float().cpu().numpy().astype(np.float64)
    if not inplace and ldo > inp:
        assert np.isnan(o[:, inp:]).all(), "padding of out was written"
    return o[:, :inp]


@pytest.mark.parametrize("rows,inp,x_bf16", [(1, 128, True), (3, 384, True), (5, 5120, False),
                                              (37, 12288, True), (2048, 4096, True)])
def test_fp32_output_within_bound(wal, rows, inp, x_bf16):
    x, bits = synth.make_x(340, rows + inp, inp, rows, bf16=x_bf16)
    print(f"rotate {rows}x{inp} bf16 in={x_bf16} -> fp32", flush=True)
    got = run(wal, x, x_bf16, out_bf16=False, ldx=inp + 64 if rows < 100 else None)
    ref = Rt.rotate(x.astype(np.float64))
    assert (np.abs(got - ref) <= group_bound(x, rows, inp)).all()


@pytest.mark.parametrize("rows,inp", [(4, 1024), (300, 5120)])
def test_bf16_output_rounds_to_nearest(wal, rows, inp):
    x, _ = synth.make_x(341, rows, inp, rows)
    print(f"rotate {rows}x{inp} -> bf16", flush=True)
    got = run(wal, x, True, out_bf16=True, ldo=inp + 64)
    ref = Rt.rotate(x.astype(np.float64))
    want = synth.bf16_bits_to_f32(bf16_rne(ref)).astype(np.float64)
    diff = got != want
    # a miss is allowed only next to a rounding midpoint, within the fp32 bound
    lo = synth.bf16_bits_to_f32(bf16_rne(ref - group_bound(x, rows, inp))).astype(np.float64)
    hi = synth.bf16_bits_to_f32(bf16_rne(ref + group_bound(x, rows, inp))).astype(np.float64)
    assert ((got == lo) | (got == hi))[diff].all()
    assert diff.mean() < 5e-3


def test_basis_vectors_exact_and_in_place(wal):
    rows, inp = 3, 384
    x = np.zeros((rows, inp), np.float32)
    for r, (g, k) in enumerate([(0, 0), (1, 77), (2, 127)]):
        x[r, g * 128 + k] = 1.0
    H = Rt.sylvester()
    for inplace in (False, True):
        got = run(wal, x, False, out_bf16=False, inplace=inplace)
        for r, (g, k) in enumerate([(0, 0), (1, 77), (2, 127)]):
            want = np.zeros(inp)
            want[g * 128:(g + 1) * 128] = H[:, k] * np.float64(np.float32(1 / np.sqrt(128)))
            assert np.array_equal(got[r], want), (inplace, r)
    xb, _ = synth.make_x(342, 0, 1024, 8)
    a = run(wal, xb, True, out_bf16=True)
    b = run(wal, xb, True, out_bf16=True, inplace=True)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("out,inp,k,P,r,b3", [(300, 5120, 4, 2, 16, True), (257, 4096, 8, 1, 16, False)])
def test_rotated_blob_product(wal, out, inp, k, P, r, b3):
    """y = W'(R x) on the GPU (rotation, then the packed product) against the
    oracle's product of W' with its own rotated, bf16-rounded x."""
    m = synth.make_matrix(343, out + inp, out, inp, k=k, n_paths=P, rank=r, scale_fmt=1 if b3 else 0,
                          trit_fmt=synth.TRIT_BASE3 if b3 else synth.TRIT_2BIT)
    blob, info = wal.pack_matrix(m)
    x, _ = synth.make_x(343, out, inp)
    X = torch.from_numpy(synth.round_bf16_bits(x[0]).view(np.int16)).to(dev()).view(torch.bfloat16)
    Xr = torch.empty_like(X)
    wal.wal_rotate_h128(X, Xr)
    y = torch.full((out,), float("nan"), dtype=torch.float32, device=dev())
    ws = torch.zeros(max(wal.wal_workspace_size(info, 1), 4) // 4, dtype=torch.float32, device=dev())
    wal.wal_gemv(info, torch.from_numpy(blob).to(dev()), Xr, y, ws)
    torch.cuda.synchronize()
    xr = synth.bf16_bits_to_f32(bf16_rne(Rt.rotate(synth.bf16_bits_to_f32(synth.round_bf16_bits(x[0])).astype(np.float64))))
    ref = D.gemv(F.pack(F.from_synth(m)), xr.astype(np.float64))
    err = D.rel_l2(y.cpu().numpy().astype(np.float64), ref)
    print(f"rotated product {out}x{inp} base3={b3}: rel_l2 {err:.2e}", flush=True)
    assert err <= 1e-3
