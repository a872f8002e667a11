"""GPU tests of the chained grouped products and their HIP graph
(wal_gemv_grouped_seq, wal_graph_create / launch / destroy).

The chain is two layers of a decode step with real data dependencies:
q|k|v read h, o reads q's output, gate|up read o's output, down reads
gate's output and gives the next layer's h (fp32 activations throughout, so
every product reads the one before it).  Each product is checked against the
CPU oracle on the input the GPU gave it (relative L2 <= 1e-5, fp32
activations); graph replays must reproduce the eager chain bit for bit, with
eager work and host synchronisations between them, and a replay after x
changed in place must match a fresh eager run.  The same chain with every
product rotating its own input (WAL_X_ROT_H128, the 27B card's rotated
blobs) is checked against the oracle on the rotated inputs, and its graph
replays against its eager run.  One layer of the 8B-shaped body at full size
(4096-12288 rows and columns, fp32 activations) runs the same dependent
chain, checked on sampled rows and replayed bit for bit.
"""
import numpy as np
import pytest

import synth
from oracle import dense as D
from oracle import format as F
from oracle import rotation as Rt

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
# (name, out, in, low-rank paths) of one layer, q k v o gate up down
LAYER = [("q", 512, 256, 1), ("k", 128, 256, 0), ("v", 128, 256, 1), ("o", 256, 512, 1),
         ("gate", 768, 256, 1), ("up", 768, 256, 0), ("down", 256, 768, 1)]
LAYERS = 2


@pytest.fixture(scope="module")
def wal():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    import ternary_hybrid_bit_amd as w
    return w


def dev():
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def chain(wal):
    """Matrices, device buffers and the 4 * LAYERS grouped plans of the chain."""
    mats, Ws, ys = {}, {}, {}
    for layer in range(LAYERS):
        for j, (name, out, inp, P) in enumerate(LAYER):
            m = synth.make_matrix(330, 7 * layer + j, out, inp, k=8, n_paths=P, rank=16)
            blob, info = wal.pack_matrix(m)
            mats[layer, name] = (m, blob, info)
            Ws[layer, name] = torch.from_numpy(blob).to(dev())
            ys[layer, name] = torch.full((out,), float("nan"), dtype=torch.float32, device=dev())
    x0, _ = synth.make_x(330, 99, LAYER[0][2], bf16=False)
    h0 = torch.from_numpy(x0[0].copy()).to(dev())
    groups = []   # (names, x tensor) per grouped product, in order
    for layer in range(LAYERS):
        h = h0 if layer == 0 else ys[layer - 1, "down"]
        groups += [(["q", "k", "v"], h), (["o"], ys[layer, "q"]), (["gate", "up"], ys[layer, "o"]),
                   (["down"], ys[layer, "gate"])]
    sizes = [wal.wal_grouped_plan_size([mats[0, n][2] for n in names], 0, wal.WAL_X_F32)[1] for names, _ in groups]
    ws = torch.zeros(max(max(sizes), 4) // 4, dtype=torch.float32, device=dev())
    plans, per_layer = [], []
    for gi, (names, x) in enumerate(groups):
        layer = gi // 4
        infos = [mats[layer, n][2] for n in names]
        plan, g = wal.wal_grouped_plan(infos, [Ws[layer, n] for n in names], [x] * len(names),
                                       [ys[layer, n] for n in names], ws, wal.WAL_X_F32)
        plans.append((g, torch.from_numpy(plan).to(dev())))
        per_layer.append((layer, names, x))
    return dict(mats=mats, ys=ys, h0=h0, plans=plans, groups=per_layer, keep=(Ws, ws))


def outputs(c):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().copy() for k, v in c["ys"].items()}


def clear(c):
    for v in c["ys"].values():
        v.fill_(float("nan"))


def test_chain_matches_oracle_step_by_step(wal, chain):
    clear(chain)
    print("chain: eager, 8 grouped products", flush=True)
    wal.wal_gemv_grouped_seq(chain["plans"])
    got = outputs(chain)
    for layer, names, x in chain["groups"]:
        xin = x.cpu().numpy().astype(np.float64)   # the input the GPU product read
        for n in names:
            m, _, _ = chain["mats"][layer, n]
            ref = D.gemv(F.pack(F.from_synth(m)), xin)
            err = D.rel_l2(got[layer, n].astype(np.float64), ref)
            assert err <= F32_TOL, (layer, n, err)


def test_graph_replays_match_eager(wal, chain):
    clear(chain)
    wal.wal_gemv_grouped_seq(chain["plans"])
    eager = outputs(chain)
    g = wal.WalGraph(chain["plans"])
    try:
        for rep in range(3):
            clear(chain)                       # eager work between the replays
            torch.cuda.synchronize()
            print(f"graph replay {rep}", flush=True)
            g.launch()
            got = outputs(chain)
            for k in eager:
                assert np.array_equal(got[k], eager[k]), (rep, k)
        # new input, in place: a replay reads it, as a fresh eager chain does
        chain["h0"].mul_(-0.5)
        clear(chain)
        g.launch()
        replay = outputs(chain)
        clear(chain)
        wal.wal_gemv_grouped_seq(chain["plans"])
        fresh = outputs(chain)
        for k in fresh:
            assert np.array_equal(replay[k], fresh[k]), k
        assert not np.array_equal(fresh[0, "q"], eager[0, "q"])
    finally:
        g.close()
        chain["h0"].mul_(-2.0)


def test_graph_capture_error_creates_nothing(wal, chain):
    """A product that fails its checks while capturing returns its status."""
    import ctypes
    g, plan = chain["plans"][0]
    bad = wal.wal_grouped_info.from_buffer_copy(g)
    bad.rows_per_batch = 3
    infos = (wal.wal_grouped_info * 2)(g, bad)
    plans = (ctypes.c_void_p * 2)(plan.data_ptr(), plan.data_ptr())
    h = ctypes.c_void_p()
    assert wal._lib.wal_graph_create(2, infos, plans, ctypes.byref(h)) == -1
    assert not h.value


@pytest.fixture(scope="module")
def rot_chain(wal, chain):
    """The chain's matrices and inputs with plans that rotate x (fp32) first."""
    mats = chain["mats"]
    ys = {k: torch.full_like(v, float("nan")) for k, v in chain["ys"].items()}
    flags = wal.WAL_X_F32 | wal.WAL_X_ROT_H128
    groups = []
    for layer in range(LAYERS):
        h = chain["h0"] if layer == 0 else ys[layer - 1, "down"]
        groups += [(["q", "k", "v"], h), (["o"], ys[layer, "q"]), (["gate", "up"], ys[layer, "o"]),
                   (["down"], ys[layer, "gate"])]
    sizes = [wal.wal_grouped_plan_size([mats[0, n][2] for n in names], 0, flags)[1] for names, _ in groups]
    ws = torch.zeros(max(max(sizes), 4) // 4, dtype=torch.float32, device=dev())
    Ws = chain["keep"][0]
    plans, per_layer = [], []
    for gi, (names, x) in enumerate(groups):
        layer = gi // 4
        infos = [mats[layer, n][2] for n in names]
        plan, g = wal.wal_grouped_plan(infos, [Ws[layer, n] for n in names], [x] * len(names),
                                       [ys[layer, n] for n in names], ws, flags)
        assert g.x_dtype == flags
        plans.append((g, torch.from_numpy(plan).to(dev())))
        per_layer.append((layer, names, x))
    return dict(mats=mats, ys=ys, plans=plans, groups=per_layer, keep=ws)


def test_rotated_chain_oracle_and_graph(wal, rot_chain):
    c = rot_chain
    clear(c)
    print("rotated chain: eager, 8 grouped products", flush=True)
    wal.wal_gemv_grouped_seq(c["plans"])
    eager = outputs(c)
    for layer, names, x in c["groups"]:
        xin = Rt.rotate(x.cpu().numpy().astype(np.float64))   # the rotation of the input the GPU read
        for n in names:
            m, _, _ = c["mats"][layer, n]
            ref = D.gemv(F.pack(F.from_synth(m)), xin)
            err = D.rel_l2(eager[layer, n].astype(np.float64), ref)
            assert err <= F32_TOL, (layer, n, err)
    g = wal.WalGraph(c["plans"])
    try:
        for rep in range(3):
            clear(c)
            torch.cuda.synchronize()
            print(f"rotated graph replay {rep}", flush=True)
            g.launch()
            got = outputs(c)
            for k in eager:
                assert np.array_equal(got[k], eager[k]), (rep, k)
    finally:
        g.close()


def test_full_size_layer_chain_fp32(wal):
    """One Qwen3-8B-shaped layer at full size with real data dependencies:
    q|k|v read h, o reads q's output, gate|up read o's output, down reads
    gate's output (fp32 activations, 2-bit / fp16 / k = 8 blobs of the
    sweep, the down product's passes split over workgroups).  Sampled rows
    of every product match the oracle on the input the GPU gave it, and two
    graph replays reproduce the eager chain bit for bit."""
    from ternary_hybrid_bit_amd import workloads
    print("full-size layer: packing 7 matrices", flush=True)
    items = workloads.sweep(layers=1)
    names = ["q", "k", "v", "o", "gate", "up", "down"]
    infos = {n: info for n, (_, info, _) in zip(names, items)}
    blobs = {n: blob for n, (blob, _, _) in zip(names, items)}
    Ws = {n: torch.from_numpy(blobs[n]).to(dev()) for n in names}
    ys = {n: torch.full((infos[n].d.out,), float("nan"), dtype=torch.float32, device=dev()) for n in names}
    x0, _ = synth.make_x(331, 0, 4096, bf16=False)
    h = torch.from_numpy(x0[0].copy()).to(dev())
    groups = [(["q", "k", "v"], h), (["o"], ys["q"]), (["gate", "up"], ys["o"]), (["down"], ys["gate"])]
    sizes = [wal.wal_grouped_plan_size([infos[n] for n in g], 0, wal.WAL_X_F32)[1] for g, _ in groups]
    ws = torch.zeros(max(max(sizes), 4) // 4, dtype=torch.float32, device=dev())
    plans = []
    for g, x in groups:
        plan, gi = wal.wal_grouped_plan([infos[n] for n in g], [Ws[n] for n in g], [x] * len(g), [ys[n] for n in g],
                                        ws, wal.WAL_X_F32)
        plans.append((gi, torch.from_numpy(plan).to(dev())))
    print("full-size layer: eager chain", flush=True)
    wal.wal_gemv_grouped_seq(plans)
    torch.cuda.synchronize()
    eager = {n: ys[n].cpu().numpy().copy() for n in names}
    rng = np.random.default_rng(12)
    for g, x in groups:
        xin = x.cpu().numpy().astype(np.float64)   # the input the GPU product read
        assert np.isfinite(xin).all()
        for n in g:
            out = infos[n].d.out
            rows = np.unique(np.concatenate([[0, out - 1], rng.integers(0, out, 6)]))
            ref = D.gemv_rows(blobs[n], xin, rows)
            err = D.rel_l2(eager[n][rows].astype(np.float64), ref)
            assert err <= F32_TOL, (n, err)
    gr = wal.WalGraph(plans)
    try:
        for rep in range(2):
            for v in ys.values():
                v.fill_(float("nan"))
            torch.cuda.synchronize()
            print(f"full-size layer: graph replay {rep}", flush=True)
            gr.launch()
            torch.cuda.synchronize()
            for n in names:
                assert np.array_equal(ys[n].cpu().numpy(), eager[n]), (rep, n)
    finally:
        gr.close()
    assert wal.sync_fallbacks(ws) == 0
