"""Fused launches: the low-rank pre-pass inside the streaming launch.

A product's first workgroups compute the low-rank terms; the streaming
workgroups wait for them (bounded, through synchronisation words) only when
they store their rows.  These tests check,
through the C ABI:

* repeated calls give identical outputs (every call returns the words to
  zero), for a grouped plan and for a single product, split and not split;
* a wait that cannot end gives up, counts itself in the fallback word, and
  the workgroup computes the low-rank terms itself (in another summation
  order than the producers: outputs agree with a normal call's to rounding,
  FALLBACK_TOL), and every kernel ends.  The words are mended, so the next call waits normally.  The
  condition is forced from the host: the copies of the epoch (which the
  tags of a call's partials derive from) are seeded with values that
  disagree, so producers and most consumers derive different tags.
"""
import numpy as np
import pytest

import synth
from oracle import dense as D
from oracle import format as F

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BF16_TOL = 1e-3
FALLBACK_TOL = 1e-5   # rel-L2 between a fallback call and a normal one (fp32 sums in another order)
SYNC_LINE = 32      # u32 words per line of the synchronisation words
EPOCH_COPIES = 16   # copies of the epoch: word 0 of lines 1..16


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


def bf16(bits):
    return to_dev(bits.view(np.int16)).view(torch.bfloat16)


def sync_words(ws):
    return ws.view(-1).view(torch.uint8)[:4352].view(torch.int32).cpu().numpy()


def seed_epochs(ws):
    """Epoch copies 1..15 one ahead of copy 0."""
    words = ws.view(-1).view(torch.uint8)[:4352].view(torch.int32)
    for r in range(1, EPOCH_COPIES):
        words[SYNC_LINE * (1 + r)] = int(sync_words(ws)[SYNC_LINE]) + 1
    torch.cuda.synchronize()


def check_sync_words(ws, fallbacks_cleared=True):
    """Everything back to zero except the epoch copies, which agree."""
    w = sync_words(ws)
    epochs = w[SYNC_LINE:SYNC_LINE * (1 + EPOCH_COPIES):SYNC_LINE]
    assert np.all(epochs == epochs[0]) and epochs[0] > 0
    rest = w.copy()
    rest[SYNC_LINE:SYNC_LINE * (1 + EPOCH_COPIES):SYNC_LINE] = 0
    if not fallbacks_cleared:
        rest[0] = 0
    assert not rest.any()


def grouped_case(wal, seed):
    shapes = [(512, 4096, 1), (1024, 4096, 2), (300, 4224, 1), (777, 12288, 0)]
    ms = [synth.make_matrix(seed, i, o, n, k=8, n_paths=p, rank=16) for i, (o, n, p) in enumerate(shapes)]
    packed = [wal.pack_matrix(m) for m in ms]
    xs_host = [synth.make_x(seed, i, m.inp) for i, m in enumerate(ms)]
    infos = [i for _, i in packed]
    Ws = [to_dev(b) for b, _ in packed]
    xs = [bf16(bits[0]) for _, bits in xs_host]
    ys = [torch.full((m.out,), float("nan"), dtype=torch.float32, device=dev()) for m in ms]
    _, wsb = wal.wal_grouped_plan_size(infos)
    ws = torch.zeros(max(wsb, 4) // 4, dtype=torch.float32, device=dev())
    plan, g = wal.wal_grouped_plan(infos, Ws, xs, ys, ws, wal.WAL_X_BF16)
    plan_dev = to_dev(plan)
    refs = [D.gemv(b, x[0]) for (b, _), (x, _) in zip(packed, xs_host)]
    return g, plan_dev, ys, refs, (Ws, xs, ws)


def close(a, b):
    return D.rel_l2(np.asarray(a, np.float64), np.asarray(b, np.float64)) <= FALLBACK_TOL


def check(ys, refs):
    for y, r in zip(ys, refs):
        assert D.rel_l2(y.cpu().numpy().astype(np.float64), r) <= BF16_TOL


def run_grouped(wal, g, plan_dev, ys):
    for y in ys:
        y.fill_(float("nan"))
    wal.wal_gemv_grouped(g, plan_dev)
    torch.cuda.synchronize()
    return [y.cpu().numpy().copy() for y in ys]


def test_grouped_repeated_calls_identical(wal):
    print("[fused] grouped plan of 4 matrices, 5 calls", flush=True)
    g, plan_dev, ys, refs, keep = grouped_case(wal, 701)
    outs = [run_grouped(wal, g, plan_dev, ys) for _ in range(5)]
    check(ys, refs)
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    ws = keep[2]
    assert wal.sync_fallbacks(ws) == 0
    check_sync_words(ws)


def test_grouped_wait_gives_up_and_falls_back(wal):
    print("[fused] grouped plan, epoch copies seeded apart: the bounded waits give up", flush=True)
    g, plan_dev, ys, refs, keep = grouped_case(wal, 702)
    ws = keep[2]
    assert g.n_zjobs > 0
    normal = run_grouped(wal, g, plan_dev, ys)
    seed_epochs(ws)
    fell_back = run_grouped(wal, g, plan_dev, ys)   # every kernel ended
    n_fell = wal.sync_fallbacks(ws)
    assert n_fell > 0
    for a, b in zip(normal, fell_back):
        assert close(a, b)
    check_sync_words(ws, fallbacks_cleared=False)   # the epoch copies agree again
    print("[fused] grouped plan, the next call waits normally", flush=True)
    again = run_grouped(wal, g, plan_dev, ys)
    for a, b in zip(normal, again):
        assert np.array_equal(a, b)
    assert wal.sync_fallbacks(ws) == n_fell
    wal.clear_sync_fallbacks(ws)
    check_sync_words(ws)


@pytest.mark.parametrize("out,inp,paths,base3", [(1000, 4096, 1, False), (600, 12288, 2, False),
                                                 (520, 17408, 2, True)])
def test_single_repeated_and_wait_gives_up(wal, out, inp, paths, base3):
    print(f"[fused] single {out}x{inp} paths={paths} base3={base3}", flush=True)
    m = synth.make_matrix(703, out + inp, out, inp, k=4, n_paths=paths, rank=16,
                          trit_fmt=synth.TRIT_BASE3 if base3 else synth.TRIT_2BIT,
                          scale_fmt=synth.SCALE_FP24 if base3 else synth.SCALE_FP16)
    blob, info = wal.pack_matrix(m)
    x, bits = synth.make_x(703, out, inp)
    ref = D.gemv(F.pack(F.from_synth(m)), x[0])
    W, xt = to_dev(blob), bf16(bits[0])
    ws = torch.zeros(wal.wal_workspace_size(info, 1) // 4, dtype=torch.float32, device=dev())
    y = torch.full((out,), float("nan"), dtype=torch.float32, device=dev())

    def call():
        y.fill_(float("nan"))
        wal.wal_gemv(info, W, xt, y, ws)
        torch.cuda.synchronize()
        return y.cpu().numpy().copy()

    outs = [call() for _ in range(3)]
    assert D.rel_l2(outs[0].astype(np.float64), ref) <= BF16_TOL
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    assert wal.sync_fallbacks(ws) == 0
    print("[fused] single, epoch copies seeded apart", flush=True)
    seed_epochs(ws)
    assert close(call(), outs[0])
    assert wal.sync_fallbacks(ws) > 0
    wal.clear_sync_fallbacks(ws)
    assert np.array_equal(call(), outs[0])
    assert wal.sync_fallbacks(ws) == 0
    check_sync_words(ws)
    counters = ws.view(-1)[wal.WAL_SYNC_BYTES // 4:wal.WAL_WS_ZERO_BYTES // 4]
    assert not counters.view(torch.int32).cpu().numpy().any()   # the arrival counters


def test_one_workspace_serves_shapes_in_turn(wal):
    """The zero region (synchronisation words, arrival counters) has one place
    and size for every shape: a smaller product's low-rank partials do not
    land on a split product's arrival counters."""
    print("[fused] one workspace: 4096x12288 split, 520x5120 two paths, 4096x12288 again", flush=True)
    big = synth.make_matrix(704, 0, 4096, 12288, k=8, n_paths=1, rank=16)
    small = synth.make_matrix(705, 0, 520, 5120, k=4, n_paths=2, rank=16)
    (bb, bi), (sb, si) = wal.pack_matrix(big), wal.pack_matrix(small)
    (_, xb), (xs_f, xs) = synth.make_x(704, 0, 12288), synth.make_x(705, 0, 5120)
    size = max(wal.wal_workspace_size(bi, 1), wal.wal_workspace_size(si, 1))
    ws = torch.zeros(size // 4, dtype=torch.float32, device=dev())
    Wb, Ws_ = to_dev(bb), to_dev(sb)
    yb = torch.full((4096,), float("nan"), dtype=torch.float32, device=dev())
    ys = torch.full((520,), float("nan"), dtype=torch.float32, device=dev())
    wal.wal_gemv(bi, Wb, bf16(xb[0]), yb, ws)
    torch.cuda.synchronize()
    first = yb.cpu().numpy().copy()
    # the smaller product's partials fill the workspace past the zero region
    ws.view(-1)[wal.WAL_WS_ZERO_BYTES // 4:].fill_(3.0)
    wal.wal_gemv(si, Ws_, bf16(xs[0]), ys, ws)
    yb.fill_(float("nan"))
    wal.wal_gemv(bi, Wb, bf16(xb[0]), yb, ws)
    torch.cuda.synchronize()
    assert np.array_equal(yb.cpu().numpy(), first)
    assert D.rel_l2(ys.cpu().numpy().astype(np.float64), D.gemv(sb, xs_f[0])) <= BF16_TOL
    assert wal.sync_fallbacks(ws) == 0


def split_case(wal, seed, specs):
    """A grouped plan (grid from the device) of matrices `specs` = [(out, in,
    k, paths, trit_fmt, scale_fmt)], all on one x per matrix."""
    ms = [synth.make_matrix(seed, i, o, n, k=k, n_paths=p, rank=16, trit_fmt=tf, scale_fmt=sf)
          for i, (o, n, k, p, tf, sf) in enumerate(specs)]
    packed = [wal.pack_matrix(m) for m in ms]
    xs_host = [synth.make_x(seed, i, m.inp) for i, m in enumerate(ms)]
    infos = [i for _, i in packed]
    Ws = [to_dev(b) for b, _ in packed]
    xs = [bf16(bits[0]) for _, bits in xs_host]
    ys = [torch.full((m.out,), float("nan"), dtype=torch.float32, device=dev()) for m in ms]
    _, wsb = wal.wal_grouped_plan_size(infos)
    ws = torch.zeros(max(wsb, 4) // 4, dtype=torch.float32, device=dev())
    plan, g = wal.wal_grouped_plan(infos, Ws, xs, ys, ws, wal.WAL_X_BF16)
    return g, to_dev(plan), ys, packed, xs_host, (Ws, xs, ws)


@pytest.mark.parametrize("base3", [False, True])
def test_grouped_split_passes(wal, base3):
    """Few rows, several passes: the plan runs the passes of each 16-row group
    in separate workgroups (more workgroups than 16-row groups), and the
    workgroup that completes a group adds its passes.  Outputs match the
    oracle on sampled rows, repeat bit for bit, agree to rounding after a
    forced fallback, and every arrival counter is zero after each call."""
    if base3:
        specs = [(2048, 17408, 4, 2, synth.TRIT_BASE3, synth.SCALE_FP24),
                 (1000, 10240, 2, 1, synth.TRIT_BASE3, synth.SCALE_FP24)]
    else:
        specs = [(4096, 12288, 8, 1, synth.TRIT_2BIT, synth.SCALE_FP16),
                 (1000, 8960, 8, 2, synth.TRIT_2BIT, synth.SCALE_FP16)]
    print(f"[fused] grouped split passes, base3={base3}", flush=True)
    g, plan_dev, ys, packed, xs_host, keep = split_case(wal, 711 + base3, specs)
    groups = sum(-(-o // 16) for o, *_ in specs)
    assert sum(g.class_grid[k] for k in range(g.n_classes)) > groups   # the passes are split
    ws = keep[2]
    counters = ws.view(-1)[wal.WAL_SYNC_BYTES // 4:wal.WAL_WS_ZERO_BYTES // 4].view(torch.int32)
    normal = run_grouped(wal, g, plan_dev, ys)
    rng = np.random.default_rng(5)
    for (blob, info), (x, _), y in zip(packed, xs_host, normal):
        rows = rng.choice(info.d.out, 128, replace=False)
        assert D.rel_l2(y[rows].astype(np.float64), D.gemv_rows(blob, x[0], rows)) <= BF16_TOL
    for _ in range(3):
        again = run_grouped(wal, g, plan_dev, ys)
        assert all(np.array_equal(a, b) for a, b in zip(normal, again))
        assert not counters.cpu().numpy().any()
    seed_epochs(ws)
    fell_back = run_grouped(wal, g, plan_dev, ys)
    assert wal.sync_fallbacks(ws) > 0
    assert all(close(a, b) for a, b in zip(normal, fell_back))
    wal.clear_sync_fallbacks(ws)
    check_sync_words(ws)
    assert not counters.cpu().numpy().any()
