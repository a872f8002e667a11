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
  (relative L2 <= 1e-3, as for every bf16 product);
* the rotation inside the products (WAL_X_ROT_H128): equal bit for bit to
  wal_rotate_h128 followed by the plain product (both formats, bf16 and
  fp32 x, one pass, split passes, passes in turn, ragged widths, grouped
  plans fused and by phases, the allocation-free entry point, the forced
  fallback of the low-rank wait), x left untouched, and within the product
  tolerance of the oracle on the oracle's rotated x.
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


# ---------------------------------------------------------------------------
# The rotation fused into the products (x_dtype | WAL_X_ROT_H128): every
# workgroup that reads x rotates the columns it needs, with wal_rotate_h128's
# arithmetic, so a fused product equals rotate-then-multiply bit for bit.

def x_dev(x_host, xbf16):
    if xbf16:
        return torch.from_numpy(synth.round_bf16_bits(x_host).view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_host, dtype=np.float32)).to(dev())


def oracle_rotated_x(x_host, xbf16):
    """The oracle's rotated x in the type the product takes: float64 rotation
    of the (bf16-rounded) activations, rounded to bf16 for bf16 x."""
    if xbf16:
        xr = Rt.rotate(synth.bf16_bits_to_f32(synth.round_bf16_bits(x_host)).astype(np.float64))
        return synth.bf16_bits_to_f32(bf16_rne(xr)).astype(np.float64)
    return Rt.rotate(np.asarray(x_host, np.float32).astype(np.float64))


def ws_for(wal, info, mode):
    if mode == "none":
        return None
    return torch.zeros(max(wal.wal_workspace_size(info, 1), 4) // 4, dtype=torch.float32, device=dev())


FUSED_CASES = [
    # label, out, in, k, paths, rank, trit format, scale format, bf16 x, workspace
    ("2bit-one-pass", 257, 4096, 8, 1, 16, synth.TRIT_2BIT, synth.SCALE_FP16, True, "full"),
    ("2bit-split-passes", 300, 12288, 4, 2, 16, synth.TRIT_2BIT, synth.SCALE_FP16, True, "full"),
    ("2bit-passes-in-turn", 130, 12288, 8, 0, 0, synth.TRIT_2BIT, synth.SCALE_FP16, True, "none"),
    ("2bit-fp32-ragged", 190, 8320, 2, 1, 8, synth.TRIT_2BIT, synth.SCALE_FP24, False, "full"),
    ("2bit-fp32-in-turn", 77, 4224, 0, 0, 0, synth.TRIT_2BIT, synth.SCALE_FP16, False, "none"),
    ("base3-one-pass", 300, 5120, 4, 2, 16, synth.TRIT_BASE3, synth.SCALE_FP24, True, "full"),
    ("base3-split-passes", 200, 17408, 2, 2, 16, synth.TRIT_BASE3, synth.SCALE_FP24, True, "full"),
    ("base3-passes-in-turn", 96, 10368, 8, 0, 0, synth.TRIT_BASE3, synth.SCALE_FP16, True, "none"),
    ("base3-k0-ragged", 150, 5248, 0, 1, 16, synth.TRIT_BASE3, synth.SCALE_FP24, True, "full"),
]


@pytest.mark.parametrize("label,out,inp,k,P,r,tf,sf,xbf16,wsm", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_fused_rotation_equals_two_launches(wal, label, out, inp, k, P, r, tf, sf, xbf16, wsm):
    print(f"[rot fused] {label}: {out}x{inp} k={k} paths={P} bf16={xbf16} ws={wsm}", flush=True)
    m = synth.make_matrix(350, out + inp + k, out, inp, k=k, n_paths=P, rank=r, scale_fmt=sf, trit_fmt=tf)
    blob, info = wal.pack_matrix(m)
    x, _ = synth.make_x(351, out + k, inp, bf16=False)
    W = torch.from_numpy(blob).to(dev())
    X = x_dev(x[0], xbf16)
    X0 = X.clone()
    # two launches: the rotation, then the plain product
    Xr = torch.empty_like(X)
    wal.wal_rotate_h128(X.view(1, -1), Xr.view(1, -1))
    y2 = torch.full((out,), float("nan"), dtype=torch.float32, device=dev())
    wal.wal_gemv(info, W, Xr, y2, ws_for(wal, info, wsm))
    # one launch that rotates x itself (fresh workspace, and the same one again)
    ws = ws_for(wal, info, wsm)
    y1 = torch.full((out,), float("nan"), dtype=torch.float32, device=dev())
    wal.wal_gemv(info, W, X, y1, ws, rotate=True)
    torch.cuda.synchronize()
    a, b = y1.cpu().numpy(), y2.cpu().numpy()
    assert np.array_equal(a, b), f"max |diff| {np.nanmax(np.abs(a - b))}"
    assert torch.equal(X.view(torch.int16) if xbf16 else X, X0.view(torch.int16) if xbf16 else X0)   # x untouched
    y1.fill_(float("nan"))
    wal.wal_gemv(info, W, X, y1, ws, rotate=True)
    torch.cuda.synchronize()
    assert np.array_equal(y1.cpu().numpy(), a)
    ref = D.gemv(F.pack(F.from_synth(m)), oracle_rotated_x(x[0], xbf16))
    err = D.rel_l2(a.astype(np.float64), ref)
    print(f"[rot fused] {label}: rel_l2 vs oracle {err:.2e}", flush=True)
    assert err <= (1e-3 if xbf16 else 1e-5)


def test_fused_rotation_no_alloc_and_fallback(wal):
    """The allocation-free entry point rotates the same way, and a consumer
    whose bounded wait for the low-rank terms gives up rotates x itself to
    compute them (sums in another order: agreement to rounding)."""
    for b3 in (False, True):
        out, inp = (700, 12288) if not b3 else (520, 17408)
        print(f"[rot fused] no-alloc and forced fallback, base3={b3}", flush=True)
        m = synth.make_matrix(352, out, out, inp, k=4, n_paths=2, rank=16,
                              trit_fmt=synth.TRIT_BASE3 if b3 else synth.TRIT_2BIT,
                              scale_fmt=synth.SCALE_FP24 if b3 else synth.SCALE_FP16)
        blob, info = wal.pack_matrix(m)
        x, _ = synth.make_x(353, out, inp, bf16=False)
        W, X = torch.from_numpy(blob).to(dev()), x_dev(x[0], True)
        ws = ws_for(wal, info, "full")
        y = torch.full((out,), float("nan"), dtype=torch.float32, device=dev())
        wal.wal_gemv(info, W, X, y, ws, rotate=True)
        y_na = torch.full((out,), float("nan"), dtype=torch.float32, device=dev())
        wal.wal_gemv_noalloc(info, W, X, y_na, rotate=True)
        torch.cuda.synchronize()
        want = y.cpu().numpy()
        assert np.array_equal(y_na.cpu().numpy(), want)
        assert wal.sync_fallbacks(ws) == 0
        # epoch copies seeded apart: the waits give up and fall back
        words = ws.view(-1).view(torch.uint8)[:wal.WAL_SYNC_BYTES].view(torch.int32)
        e0 = int(words[32].item())
        for rr in range(1, 16):
            words[32 * (1 + rr)] = e0 + 1
        y.fill_(float("nan"))
        wal.wal_gemv(info, W, X, y, ws, rotate=True)
        torch.cuda.synchronize()
        assert wal.sync_fallbacks(ws) > 0
        assert D.rel_l2(y.cpu().numpy().astype(np.float64), want.astype(np.float64)) <= 1e-5
        wal.clear_sync_fallbacks(ws)


@pytest.mark.parametrize("grid", [0, 64])
def test_fused_rotation_grouped_plan(wal, grid):
    """A grouped plan with WAL_X_ROT_H128 (every matrix rotated; with grid 64
    the wide matrices run their passes in turn) against the plan without it on
    x rotated by wal_rotate_h128: bit for bit, fused and with the low-rank
    jobs as a launch of their own."""
    print(f"[rot fused] grouped plan, grid={grid}", flush=True)
    shapes = [(512, 4096, 8, 1), (1024, 4096, 8, 2), (300, 4224, 4, 1), (777, 12288, 8, 0), (96, 12288, 2, 1)]
    ms = [synth.make_matrix(354, i, o, n, k=k, n_paths=p, rank=16 if p else 0) for i, (o, n, k, p) in enumerate(shapes)]
    packed = [wal.pack_matrix(m) for m in ms]
    infos = [i for _, i in packed]
    Ws = [torch.from_numpy(b).to(dev()) for b, _ in packed]
    xs = [x_dev(synth.make_x(355, i, m.inp, bf16=False)[0][0], True) for i, m in enumerate(ms)]
    xr = [torch.empty_like(x) for x in xs]
    for a, b in zip(xs, xr):
        wal.wal_rotate_h128(a.view(1, -1), b.view(1, -1))

    def plan_run(x_list, flags, phases=None):
        ys = [torch.full((m.out,), float("nan"), dtype=torch.float32, device=dev()) for m in ms]
        _, wsb = wal.wal_grouped_plan_size(infos, grid, flags)
        ws = torch.zeros(max(wsb, 4) // 4, dtype=torch.float32, device=dev())
        plan, g = wal.wal_grouped_plan(infos, Ws, x_list, ys, ws, flags, grid)
        assert g.x_dtype == flags
        pd = torch.from_numpy(plan).to(dev())
        if phases is None:
            wal.wal_gemv_grouped(g, pd)
        else:
            for ph in phases:
                wal.wal_gemv_grouped_phases(g, pd, ph)
        torch.cuda.synchronize()
        return [y.cpu().numpy() for y in ys]

    want = plan_run(xr, wal.WAL_X_BF16)
    got = plan_run(xs, wal.WAL_X_BF16 | wal.WAL_X_ROT_H128)
    got2 = plan_run(xs, wal.WAL_X_BF16 | wal.WAL_X_ROT_H128, phases=[wal.WAL_PHASE_LOWRANK, wal.WAL_PHASE_STREAM])
    for i, (a, b, c) in enumerate(zip(want, got, got2)):
        assert np.array_equal(a, b), i
        assert np.array_equal(a, c), i
    for i, m in enumerate(ms):
        x = synth.make_x(355, i, m.inp, bf16=False)[0][0]
        ref = D.gemv(F.pack(F.from_synth(m)), oracle_rotated_x(x, True))
        assert D.rel_l2(got[i].astype(np.float64), ref) <= 1e-3
