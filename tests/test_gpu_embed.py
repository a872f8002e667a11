"""GPU parity of the embedding-row lookups (wal_embed_rows for INT3/g128 and
INT4/g128 tables, wal_embed_rows_mixed for a table of INT3 and INT4 rows and a
row map) against the CPU oracle (oracle/int3.py, oracle/int4.py), through the
C ABI.

Every value is s * q with a binary16 scale and a code of at most 4 bits, so
it is exact in fp32: fp32 output must equal the oracle bit for bit, and bf16
output must equal the oracle's value rounded to nearest even.  Indices
outside [0, V), negative ones included, and map entries outside their table
give rows of zeros; columns past the row width are left untouched.
"""
import numpy as np
import pytest

from oracle import int3 as I3
from oracle import int4 as I4

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


def make(seed, bits, V, inp):
    """Codes uniform on the format's range; scales |N(0, 1)| / 64 in fp16."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 60, seed]))
    lo = -(1 << (bits - 1))
    q = rng.integers(lo, -lo, size=(V, inp)).astype(np.int8)
    s = (np.abs(rng.standard_normal((V, inp // 128))) / 64).astype(np.float16).astype(np.float32)
    return q, s


def pack(wal, bits, q, s):
    return wal.wal_int3_pack(q, s) if bits == 3 else wal.wal_int4_pack(q, s)


def oracle_rows(bits, blob, V, inp, ids):
    return (I3 if bits == 3 else I4).rows(blob, V, inp, ids)


def run(wal, blob, bits, V, inp, ids, dtype, ldo=None):
    ldo = ldo or inp
    W = torch.from_numpy(blob).to(dev())
    d_ids = torch.from_numpy(np.asarray(ids, np.int32)).to(dev())
    out = torch.full((len(ids), ldo), float("nan"), dtype=dtype, device=dev())
    wal.wal_embed_rows(W, bits, V, inp, d_ids, out)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    if ldo > inp:
        assert np.isnan(o[:, inp:]).all(), "padding of out was written"
    return o[:, :inp]


def expect(ref, dtype):
    r = torch.from_numpy(ref.astype(np.float32))
    return (r.to(torch.bfloat16).float() if dtype == torch.bfloat16 else r).numpy()


@pytest.mark.parametrize("bits", [3, 4])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,inp,ldo", [(1, 128, None), (7, 384, 392), (1000, 4224, None), (300, 12288, 12296),
                                        (65, 2048, None), (40, 2176, 2184)])
def test_rows_exact(wal, bits, dtype, V, inp, ldo):
    q, s = make(V + inp + bits, bits, V, inp)
    blob = pack(wal, bits, q, s)
    rng = np.random.default_rng(V * 7 + bits)
    ids = np.concatenate([[0, V - 1, V, -1, 0], rng.integers(0, V, 37), [V + 12345, -(1 << 31), 2**31 - 1]])
    print(f"embed int{bits} {V}x{inp} n={len(ids)} {dtype}", flush=True)
    got = run(wal, blob, bits, V, inp, ids, dtype, ldo)
    ref = oracle_rows(bits, blob, V, inp, ids)
    assert np.array_equal(got, expect(ref, dtype))
    for n, v in enumerate(ids):
        if not 0 <= v < V:
            assert not got[n].any(), n


@pytest.mark.parametrize("bits", [3, 4])
def test_qwen3_8b_vocabulary(wal, bits):
    """A 151936 x 4096 embedding (the 8B models' vocabulary and width) at full
    size: a batch of 2048 token ids, every output of 256 sampled tokens
    against the oracle and all 2048 rows finite."""
    V, inp, n = 151936, 4096, 2048
    q, s = make(bits, bits, V, inp)
    blob = pack(wal, bits, q, s)
    ids = np.random.default_rng(bits).integers(0, V, n)
    ids[:4] = [0, V - 1, 1, V - 2]
    print(f"embed int{bits} {V}x{inp} n={n}", flush=True)
    got = run(wal, blob, bits, V, inp, ids, torch.bfloat16)
    assert np.isfinite(got).all()
    pick = np.unique(np.concatenate([[0, 1, 2, 3, n - 1], np.random.default_rng(5).integers(0, n, 251)]))
    ref = oracle_rows(bits, blob, V, inp, ids[pick])
    assert np.array_equal(got[pick], expect(ref, torch.bfloat16))


def mixed_tables(wal, seed, V, inp, frac4=0.25):
    """A vocabulary of V rows, a seeded quarter of them INT4 (the rest INT3),
    each table packed on its own; row_map in the library's convention."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 61, seed]))
    is4 = np.zeros(V, bool)
    is4[rng.choice(V, int(V * frac4), replace=False)] = True
    V4 = int(is4.sum())
    V3 = V - V4
    q3, s3 = make(seed, 3, V3, inp)
    q4, s4 = make(seed + 1, 4, V4, inp)
    b3, b4 = wal.wal_int3_pack(q3, s3), wal.wal_int4_pack(q4, s4)
    row_map = np.empty(V, np.int64)
    row_map[~is4] = rng.permutation(V3)
    row_map[is4] = -1 - rng.permutation(V4)
    return b3, V3, b4, V4, row_map.astype(np.int32)


def run_mixed(wal, b3, V3, b4, V4, inp, row_map, ids, dtype, ldo=None):
    ldo = ldo or inp
    W3, W4 = torch.from_numpy(b3).to(dev()), torch.from_numpy(b4).to(dev())
    m = torch.from_numpy(np.asarray(row_map, np.int32)).to(dev())
    d_ids = torch.from_numpy(np.asarray(ids, np.int32)).to(dev())
    out = torch.full((len(ids), ldo), float("nan"), dtype=dtype, device=dev())
    wal.wal_embed_rows_mixed(W3, V3, W4, V4, inp, m, d_ids, out)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    if ldo > inp:
        assert np.isnan(o[:, inp:]).all(), "padding of out was written"
    return o[:, :inp]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,inp,ldo", [(4, 128, None), (40, 384, 392), (1000, 5120, None), (333, 2176, 2184)])
def test_mixed_rows_exact(wal, dtype, V, inp, ldo):
    b3, V3, b4, V4, row_map = mixed_tables(wal, V + inp, V, inp)
    rng = np.random.default_rng(V)
    ids = np.concatenate([[0, V - 1, V, -1], rng.integers(0, V, 40), [-(1 << 31), 2**31 - 1]])
    print(f"embed mixed {V}x{inp} (int3 {V3}, int4 {V4}) n={len(ids)} {dtype}", flush=True)
    got = run_mixed(wal, b3, V3, b4, V4, inp, row_map, ids, dtype, ldo)
    ref = I3.rows_mixed(b3, V3, b4, V4, inp, row_map, ids)
    assert np.array_equal(got, expect(ref, dtype))
    # map entries past their tables give zero rows; the others are unchanged
    bad = row_map.copy()
    bad[0], bad[V - 1] = V3, -1 - V4
    got_b = run_mixed(wal, b3, V3, b4, V4, inp, bad, ids, dtype, ldo)
    assert np.array_equal(got_b, expect(I3.rows_mixed(b3, V3, b4, V4, inp, bad, ids), dtype))
    assert not got_b[0].any() and not got_b[1].any()


def test_mixed_27b_vocabulary(wal):
    """A 248320 x 5120 mixed table (the 27B model's vocabulary and width, a
    quarter of the rows INT4): 2048 token ids, 256 sampled rows exact."""
    V, inp, n = 248320, 5120, 2048
    b3, V3, b4, V4, row_map = mixed_tables(wal, 7, V, inp)
    ids = np.random.default_rng(8).integers(0, V, n)
    print(f"embed mixed {V}x{inp} (int3 {V3}, int4 {V4}) n={n}", flush=True)
    got = run_mixed(wal, b3, V3, b4, V4, inp, row_map, ids, torch.bfloat16)
    assert np.isfinite(got).all()
    pick = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(9).integers(0, n, 254)]))
    ref = I3.rows_mixed(b3, V3, b4, V4, inp, row_map, ids[pick])
    assert np.array_equal(got[pick], expect(ref, torch.bfloat16))

