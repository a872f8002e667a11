"""Pins of the CPU oracle against facts other than itself.

Every check here is CPU-only.  A plausible mistake in the oracle (a dropped
term, a wrong sign or index, a transposed operand, a wrong scale decode)
fails at least one of them:

* golden bytes worked by hand from the format readings (codes, sites, scales,
  sign planes, header fields);
* byte totals printed on the WAL2-Ternary-27B card, which fix the 2-bit code
  plus fp16-scale density exactly and the base-3 density approximately;
* exact-rational brute force of the operator's definition on tiny matrices,
  written directly from the logical arrays with Fraction arithmetic;
* special cases that reduce to library routines (numpy matmul, scipy sparse);
* invariants: the all-zero case, columns e_j, linearity, round trips,
  exhaustive codec sweeps.
"""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest
import scipy.sparse

import synth
from oracle import dense as D
from oracle import format as F

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def tiny(out, inp, k, paths, rank, tf=0, sf=0, seed=0, zero_T=False):
    m = synth.make_matrix(100 + seed, out * 1000 + inp + 7 * k + paths, out, inp, k=k,
                          n_paths=paths, rank=rank, trit_fmt=tf, scale_fmt=sf, zero_T=zero_T)
    return F.from_synth(m)


def brute_y(L, x):
    """y_n = sum_j W[n, j] x_j with W from the definition, in exact rationals.

    W[n, j] = alpha[n, g] T[n, j] + beta[n, g] R[n, j]
              + sum_p sum_r s_p[r] U_p[n, r] V_p[j, r],   g = j // 128,
    R[n, j] = sign of the site of group g at position j - 128 g, else 0.
    """
    xs = [Fraction(float(v)) for v in x]
    y = []
    for n in range(L.out):
        acc = Fraction(0)
        R = {}
        for g in range(L.inp // 128):
            for i in range(L.k):
                R[g * 128 + int(L.site_pos[n, g, i])] = int(L.site_sign[n, g, i])
        for j in range(L.inp):
            g = j // 128
            w = Fraction(float(L.alpha[n, g])) * int(L.T[n, j])
            if j in R:
                w += Fraction(float(L.beta[n, g])) * R[j]
            for p in range(L.U.shape[0]):
                for r in range(L.U.shape[2]):
                    w += Fraction(float(L.s[p, r])) * int(L.U[p, n, r]) * int(L.V[p, j, r])
            acc += w * xs[j]
        y.append(acc)
    return y


# --------------------------------------------------------------------------
# Golden bytes worked from the format readings.

def test_golden_2bit_codes():
    # trits (+1, -1, 0, +1) -> codes 01, 11, 00, 01 at bits 0-1, 2-3, 4-5, 6-7
    # -> 0b01_00_11_01 = 0x4D
    T = np.array([[1, -1, 0, 1] * 32], dtype=np.int8)
    assert F.encode_codes_2bit(T)[0, 0] == 0x4D
    T = np.zeros((1, 128), np.int8)
    T[0, 127] = -1                       # last trit of the row: byte 31, bits 6-7 = 11
    assert F.encode_codes_2bit(T)[0, 31] == 0xC0
    assert not F.encode_codes_2bit(T)[0, :31].any()


def test_golden_base3_bytes():
    # (+1, -1, 0, +1, 0) -> digits (2, 0, 1, 2, 1) -> 2 + 0*3 + 1*9 + 2*27 + 1*81 = 146 = 0x92
    T = np.zeros((1, 128), np.int8)
    T[0, :5] = [1, -1, 0, 1, 0]
    row = F.encode_codes_base3(T)[0]
    assert row[0] == 0x92
    # five zero trits -> digits 1,1,1,1,1 -> 121 = 0x79; 128 trits -> 26 bytes, the
    # 26th holds trits 125..127 and two zero-trit fillers; the row pads to 32 bytes
    assert len(row) == 32 and row[1] == 0x79 and (row[26:] == 0x79).all()
    T[0, 125:128] = [-1, -1, -1]         # digits 0,0,0,1,1 -> 27 + 81 = 108
    assert F.encode_codes_base3(T)[0, 25] == 108
    T = np.full((1, 5), 1, np.int8)
    T = np.pad(T, ((0, 0), (0, 123)))
    assert F.encode_codes_base3(T)[0, 0] == 242   # all digits 2 -> 3^5 - 1


def test_golden_site_bytes():
    pos = np.array([[[5, 127]]], np.uint8)
    sign = np.array([[[-1, 1]]], np.int8)
    assert list(F.encode_sites(pos, sign)[0, 0]) == [0x85, 0x7F]


def test_golden_scales():
    # 0.02 as fp32 = 0x3CA3D70A; fp24 keeps 0x3CA3D7 and stores it little-endian D7 A3 3C
    v = np.array([np.float32(0.02)]).view(np.uint32) & np.uint32(0xFFFFFF00)
    v = v.view(np.float32)
    b = F._scale_bytes(v, F.SCALE_FP24)
    assert list(b) == [0xD7, 0xA3, 0x3C]
    assert float(F._scale_values(b, 1, F.SCALE_FP24)[0]) == 0.019999980926513672
    # fp16 1.0 = 0x3C00 -> bytes 00 3C ; -2.0 = 0xC000
    assert list(F._scale_bytes(np.array([1.0, -2.0], np.float32), F.SCALE_FP16)) == [0, 0x3C, 0, 0xC0]
    with pytest.raises(F.FormatError):
        F._scale_bytes(np.array([0.1], np.float32), F.SCALE_FP16)     # not an fp16 value
    with pytest.raises(F.FormatError):
        F._scale_bytes(np.array([np.float32(0.02)]), F.SCALE_FP24)    # low byte non-zero


def test_golden_sign_planes_and_header():
    L = tiny(2, 128, 2, 1, 9)
    L.U[0] = 1
    L.U[0, 1, 8] = -1                    # row 1, rank 8 -> byte 1 of row 1, bit 0
    L.V[0] = 1
    L.V[0, 9, 0] = -1                    # column 9 of rank 0 -> byte 1 of rank 0's row, bit 1
    blob = F.pack(L)
    h = F.parse_header(blob)
    assert h["magic"] == 0x314C4157 and blob[:4] == b"WAL1"
    U = np.frombuffer(blob, np.uint8)[h["U0"]: h["U0"] + 4].reshape(2, 2)
    assert U.tolist() == [[0, 0], [0, 1]]
    V = np.frombuffer(blob, np.uint8)[h["V0"]: h["V0"] + 16 * 9].reshape(9, 16)
    assert V[0, 1] == 0x02 and V.sum() == 2
    assert struct.unpack("<I", blob[8:12])[0] == 2 and struct.unpack("<I", blob[12:16])[0] == 128
    assert h["codes"] == 256 and h["codes"] % 256 == 0 and h["total"] % 256 == 0


# --------------------------------------------------------------------------
# Byte totals printed on the pages.

def test_pq2_total_matches_page_exactly():
    """2-bit codes + one fp16 scale per 128 (our k = 0, no-path format) is
    34 bytes per 128 weights; with F32 exceptions this reproduces the
    WAL2-Ternary-27B card's PQ2_0 tensor bytes to the byte."""
    g = GOLD["wal2_27b"]
    for out, inp in [(5120, 17408), (17408, 5120), (1024, 5120), (256, 128)]:
        sz = F.plane_sizes(out, inp, 0, 0, 0, F.TRIT_2BIT, F.SCALE_FP16)
        assert sz["codes"] + sz["alpha"] == out * inp * 34 // 128
    assert g["pq2_codes_bytes_per_128"] + g["pq2_scale_bytes_per_128"] == 34
    total = g["ternary_params"] * 34 // 128 + g["exception_params"] * 4
    assert total == g["pq2_tensor_bytes"]
    assert abs(34 * 8 / 128 - g["pq2_bits_per_weight"]) < 1e-12
    assert g["ternary_params"] + g["exception_params"] == g["text_params"]
    assert g["text_params"] * 2 == g["bf16_ideal_bytes"]
    # three of the four 2-bit codes are used by the oracle's encoder
    T = np.array([[-1, 0, 1, 0] * 32], np.int8)
    codes = set(((F.encode_codes_2bit(T)[0, :, None] >> np.array([0, 2, 4, 6])) & 3).ravel().tolist())
    assert codes == {0, 1, 3} and len(codes) == g["pq2_codes_used_of_4"]


def test_base3_total_matches_page_continuous_packing():
    """Continuous five-trits-per-byte rows, bf16 scales per 128 and bf16
    exceptions land within 0.01 % of the card's base-3 tensor bytes; packing
    each 128-trit group into its own 26 bytes overshoots by more than 1 %."""
    g = GOLD["wal2_27b"]
    P = g["ternary_params"]
    # our row width for the card's hidden size: 5120 trits -> exactly 1024 bytes
    assert F.row_stride(5120, F.TRIT_BASE3) == 5120 // 5
    continuous = P * 8 // 5 // 8 + P // 128 * 2 + g["exception_params"] * 2
    per_group = P // 128 * 26 + P // 128 * 2 + g["exception_params"] * 2
    printed = g["base3_tensor_bytes"]
    assert abs(continuous - printed) / printed < 1e-4
    assert (per_group - printed) / printed > 0.01
    assert abs(printed * 8 / g["text_params"] - g["base3_bits_per_param"]) < 1e-5
    assert abs(g["bf16_ideal_bytes"] / printed - g["ratio_bf16_to_base3"]) < 0.01
    assert abs(g["bf16_ideal_bytes"] / g["pq2_tensor_bytes"] - g["ratio_bf16_to_pq2"]) < 0.01


def test_sweep_counts_match_page():
    g = GOLD["wal_ternary_8b"]
    shapes = synth.sweep_shapes()
    assert len(shapes) == g["body_matrices"] == g["layers"] * 7
    mask = synth.sweep_lowrank_mask()
    assert mask.sum() == g["walb2_matrices"] and (~mask).sum() == g["base_only_matrices"]
    # the body's packed bytes in this format sit near the card's "about 2.3 GB"
    # executable cache (2.39e9 bytes = 2.23 GiB)
    tot = sum(F.algorithmic_bytes(o, i, 8, int(m), 16, 0, 0) for (o, i), m in zip(shapes, mask))
    assert abs(tot / 2**30 - g["executable_cache_gb_approx"]) < 0.15


def test_algorithmic_bytes_hand_worked():
    """Bytes a product reads, worked by hand from the layout (codes in/4 per
    row for 2-bit, ceil(in/5) for base-3; k site bytes and one alpha (+ beta
    when k > 0) of 2 (fp16) or 3 (fp24) bytes per row and 128-column group;
    per path rank*in/8 V bytes, out*ceil(rank/8) U bytes and 2*rank s bytes),
    against the oracle's count."""
    # 256 x 512, k = 8, fp16, no paths: 32768 codes + 256*4*8 sites
    # + 256*4*2 alpha + 256*4*2 beta
    assert 256 * 512 // 4 + 8192 + 2048 + 2048 == 45_056
    assert F.algorithmic_bytes(256, 512, 8, 0, 0, F.TRIT_2BIT, F.SCALE_FP16) == 45_056
    # 12288 x 4096, k = 8, fp16, one rank-16 path:
    # 12,582,912 codes + 3,145,728 sites + 1,572,864 alpha/beta
    # + 8,192 V + 24,576 U + 32 s
    assert 12_582_912 + 3_145_728 + 1_572_864 + 8_192 + 24_576 + 32 == 17_334_304
    assert F.algorithmic_bytes(12288, 4096, 8, 1, 16, F.TRIT_2BIT, F.SCALE_FP16) == 17_334_304
    # 4096 x 12288 (the down shape): the same total
    assert F.algorithmic_bytes(4096, 12288, 8, 1, 16, F.TRIT_2BIT, F.SCALE_FP16) == 17_334_304
    # 17408 x 5120, base-3, fp24, two rank-16 paths: codes 17408 * 1024,
    # alpha 17408*40*3, paths 2 * (10240 V + 34816 U + 32 s), then per k the
    # sites 17408*40*k and beta 2,088,960
    base = 17_825_792 + 2_088_960 + 90_176
    want = {0: 20_004_928, 2: 23_486_528, 4: 24_879_168, 8: 27_664_448}
    for k, v in want.items():
        extra = 0 if k == 0 else 17408 * 40 * k + 2_088_960
        assert base + extra == v
        assert F.algorithmic_bytes(17408, 5120, k, 2, 16, F.TRIT_BASE3, F.SCALE_FP24) == v
        # 5120 x 17408: 5120 * ceil(17408 / 5) = 5120 * 3482 code bytes, 2,048
        # more than above; alpha 5120*136*3 is the same; row padding not counted
        assert F.algorithmic_bytes(5120, 17408, k, 2, 16, F.TRIT_BASE3, F.SCALE_FP24) == v + 2_048
    # 2-bit vs base-3 rows: a padded base-3 row (1024 -> stride 1024, 3482 ->
    # 3488) still counts ceil(in / 5)
    assert F.algorithmic_bytes(1, 640, 0, 0, 0, F.TRIT_BASE3, F.SCALE_FP16) == 128 + 10


def test_sweep_bytes_hand_worked():
    """The 252-matrix body: per layer q, o 4096x4096 (5,767,168 B each), k, v
    1024x4096 (1,441,792 B each), gate, up 12288x4096 and down 4096x12288
    (17,301,504 B each) at k = 8, fp16; a rank-16 path adds 2*(in + out) + 32
    bytes on each of the 213 drawn matrices."""
    per_layer = 2 * 5_767_168 + 2 * 1_441_792 + 3 * 17_301_504
    assert per_layer * 36 == 2_387_607_552
    shapes = synth.sweep_shapes()
    mask = synth.sweep_lowrank_mask()
    lowrank = sum(2 * (i + o) + 32 for (o, i), m in zip(shapes, mask) if m)
    assert 2_387_607_552 + lowrank == 2_392_197_792
    tot = sum(F.algorithmic_bytes(o, i, 8, int(m), 16, 0, 0) for (o, i), m in zip(shapes, mask))
    assert tot == 2_392_197_792


def test_rel_l2_hand_worked():
    """rel_l2 = ||y - y_ref|| / ||y_ref||, worked by hand."""
    # y - y_ref = (3, -1): sqrt(10) / 5
    assert D.rel_l2([3.0, 4.0], [0.0, 5.0]) == pytest.approx(np.sqrt(10.0) / 5.0, rel=1e-15)
    # the reference is the denominator, not y: (0, 5) vs (3, 4) gives sqrt(10)/5 too
    # but (1, 0) vs (2, 0) is 1/2 one way and 1 the other
    assert D.rel_l2([1.0, 0.0], [2.0, 0.0]) == pytest.approx(0.5, rel=1e-15)
    assert D.rel_l2([2.0, 0.0], [1.0, 0.0]) == pytest.approx(1.0, rel=1e-15)
    # (1, 2, 2) vs (1, 2, 3): 1 / sqrt(14)
    assert D.rel_l2([1.0, 2.0, 2.0], [1.0, 2.0, 3.0]) == pytest.approx(1.0 / np.sqrt(14.0), rel=1e-15)
    # equal vectors: exactly 0; zero vs zero: 0; anything else vs zero: inf
    assert D.rel_l2([1.5, -2.0], [1.5, -2.0]) == 0.0
    assert D.rel_l2([0.0, 0.0], [0.0, -0.0]) == 0.0
    assert D.rel_l2([1e-30, 0.0], [0.0, 0.0]) == float("inf")
    # a 2-D input is one vector (the norm over every element)
    assert D.rel_l2([[3.0], [4.0]], [[0.0], [5.0]]) == pytest.approx(np.sqrt(10.0) / 5.0, rel=1e-15)
    # float32 inputs are taken at their exact values
    assert D.rel_l2(np.float32([1.0, 0.0]), np.float32([2.0, 0.0])) == 0.5


# --------------------------------------------------------------------------
# Exact-rational brute force.

@pytest.mark.parametrize("out,inp,k,paths,rank,tf,sf", [
    (1, 128, 0, 0, 0, 0, 0), (2, 128, 2, 0, 0, 0, 0), (3, 256, 8, 1, 8, 0, 0),
    (2, 256, 4, 2, 3, 1, 1), (3, 128, 8, 1, 8, 1, 0), (1, 256, 0, 1, 8, 0, 1),
])
def test_bruteforce_integer_x_exact(out, inp, k, paths, rank, tf, sf):
    L = tiny(out, inp, k, paths, rank, tf, sf)
    x = np.random.default_rng(5).integers(-3, 4, size=inp).astype(np.float64)
    y = D.gemv(F.pack(L), x)
    exact = brute_y(L, x)
    assert [Fraction(float(v)) for v in y] == exact


@pytest.mark.parametrize("bf16", [True, False])
def test_bruteforce_random_x_within_fp64_bound(bf16):
    L = tiny(3, 256, 8, 2, 8, 0, 1)
    x, _ = synth.make_x(9, 1, 256, bf16=bf16)
    x = x[0]
    y = D.gemv(F.pack(L), x)
    exact = brute_y(L, x)
    W = D.dense_W(L)
    bound = 256 * 2.0 ** -52 * (np.abs(W) @ np.abs(x.astype(np.float64)))
    for n in range(3):
        assert abs(Fraction(float(y[n])) - exact[n]) <= Fraction(float(bound[n]))


def test_columns_match_definition_exactly():
    """x = e_j returns column j of W exactly (every W entry is a multiple of
    2^-24 below 2^-2, so the column is exact in any precision >= fp32)."""
    L = tiny(3, 256, 8, 2, 16, 1, 1)
    blob = F.pack(L)
    for j in [0, 1, 5, 127, 128, 200, 255]:
        e = np.zeros(256)
        e[j] = 1.0
        y = D.gemv(blob, e)
        col = brute_y(L, e)
        assert [Fraction(float(v)) for v in y] == col
        assert np.array_equal(y.astype(np.float32).astype(np.float64), y)


# --------------------------------------------------------------------------
# Special cases that reduce to library routines.

def test_block_scaled_ternary_is_plain_matmul():
    """k = 0 and no paths: a block-scaled ternary product (the PQ2_0 layout of
    the WAL2-Ternary-27B card), (T * repeat(alpha, 128)) @ x."""
    L = tiny(16, 512, 0, 0, 0)
    x = np.random.default_rng(1).standard_normal(512)
    ref = (L.T * np.repeat(L.alpha.astype(np.float64), 128, axis=1)) @ x
    np.testing.assert_allclose(D.gemv(F.pack(L), x), ref, rtol=1e-13, atol=1e-13)


def test_pure_sparse_matches_scipy_coo():
    L = tiny(8, 384, 8, 0, 0, zero_T=True)
    x = np.random.default_rng(2).standard_normal(384)
    rows, cols, vals = [], [], []
    for n in range(8):
        for g in range(3):
            for i in range(8):
                rows.append(n)
                cols.append(128 * g + int(L.site_pos[n, g, i]))
                vals.append(float(L.beta[n, g]) * int(L.site_sign[n, g, i]))
    S = scipy.sparse.coo_matrix((vals, (rows, cols)), shape=(8, 384)).tocsr()
    np.testing.assert_allclose(D.gemv(F.pack(L), x), S @ x, rtol=1e-13, atol=1e-14)


def test_pure_lowrank_matches_factored_product():
    L = tiny(8, 256, 0, 2, 16, zero_T=True)
    x = np.random.default_rng(3).standard_normal(256)
    ref = sum(L.U[p].astype(np.float64) @ (L.s[p].astype(np.float64) * (L.V[p].astype(np.float64).T @ x))
              for p in range(2))
    np.testing.assert_allclose(D.gemv(F.pack(L), x), ref, rtol=1e-12, atol=1e-14)


def test_all_zero_returns_zero():
    L = tiny(4, 256, 0, 0, 0, zero_T=True)
    x = np.random.default_rng(4).standard_normal(256)
    assert not D.gemv(F.pack(L), x).any()
    L = tiny(4, 256, 8, 1, 4, zero_T=True)
    L.beta[:] = 0
    L.s[:] = 0
    assert not D.gemv(F.pack(L), x).any()


def test_linearity():
    L = tiny(8, 256, 4, 1, 8)
    blob = F.pack(L)
    rng = np.random.default_rng(6)
    x1, x2 = rng.standard_normal(256), rng.standard_normal(256)
    lhs = D.gemv(blob, 0.75 * x1 - 2.5 * x2)
    rhs = 0.75 * D.gemv(blob, x1) - 2.5 * D.gemv(blob, x2)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_gemm_rows_equal_gemv():
    L = tiny(8, 256, 8, 1, 8)
    blob = F.pack(L)
    X = np.random.default_rng(7).standard_normal((5, 256))
    Y = D.gemm(blob, X)
    for b in range(5):
        np.testing.assert_allclose(Y[b], D.gemv(blob, X[b]), rtol=1e-13, atol=1e-15)


# --------------------------------------------------------------------------
# Codecs: exhaustive sweeps and round trips.

def test_base3_codec_is_a_bijection_on_243_bytes():
    trits = np.array(np.meshgrid(*[[-1, 0, 1]] * 5, indexing="ij")).reshape(5, -1).T  # 243 x 5
    T = np.zeros((243, 128), np.int8)
    T[:, :5] = trits
    b = F.encode_codes_base3(T)[:, 0]
    assert sorted(b.tolist()) == list(range(243))
    # digit i of the byte is trit i + 1 (least significant digit first)
    for row, byte in zip(trits, b):
        v = int(byte)
        for i in range(5):
            v, d = divmod(v, 3)
            assert d == row[i] + 1
    back = F.decode_codes_base3(F.encode_codes_base3(T), 128)
    assert np.array_equal(back, T)


@pytest.mark.parametrize("bad", [243, 250, 255])
def test_base3_rejects_bytes_above_242(bad):
    L = tiny(1, 128, 0, 0, 0, tf=1)
    blob = bytearray(F.pack(L))
    blob[256] = bad
    blob[176:184] = struct.pack("<Q", F.checksum(bytes(blob)))
    with pytest.raises(F.FormatError):
        F.unpack(bytes(blob))


def test_2bit_rejects_code_10():
    L = tiny(1, 128, 0, 0, 0)
    blob = bytearray(F.pack(L))
    blob[256 + 3] = (blob[256 + 3] & ~(3 << 4)) | (2 << 4)
    blob[176:184] = struct.pack("<Q", F.checksum(bytes(blob)))
    with pytest.raises(F.FormatError):
        F.unpack(bytes(blob))


def test_every_2bit_code_at_a_probe_position():
    """Each stored code at one position, read through the whole oracle with
    x = e_j: 00 -> 0, 01 -> +alpha, 11 -> -alpha."""
    L = tiny(1, 128, 0, 0, 0, zero_T=True)
    L.alpha[:] = 0.5
    for j in (0, 37, 127):
        for code, want in ((0, 0.0), (1, 0.5), (3, -0.5)):
            blob = bytearray(F.pack(L))
            blob[256 + j // 4] |= code << (2 * (j % 4))
            blob[176:184] = struct.pack("<Q", F.checksum(bytes(blob)))
            e = np.zeros(128)
            e[j] = 1
            assert D.gemv(bytes(blob), e)[0] == want


def test_every_site_byte():
    """All 256 site bytes through the oracle (k = 2, T = 0, beta = 1): the
    probe byte's site adds sign * x[pos] with pos = low 7 bits, sign = - iff bit 7."""
    L = tiny(1, 128, 2, 0, 0, zero_T=True)
    L.beta[:] = 1.0
    x = np.arange(1, 129, dtype=np.float64)
    for v in range(256):
        pos, neg = v & 0x7F, v >> 7
        other = 0 if pos else 1                        # a second, distinct site
        lo, hi = sorted([(pos, v), (other, other)])
        blob = bytearray(F.pack(L))
        h = F.parse_header(blob)
        blob[h["sites"]] = lo[1]
        blob[h["sites"] + 1] = hi[1]
        blob[176:184] = struct.pack("<Q", F.checksum(bytes(blob)))
        y = D.gemv(bytes(blob), x)[0]
        assert y == (-1 if neg else 1) * (pos + 1) + (other + 1)


def test_each_lowrank_sign_bit():
    """Flipping one stored U or V bit flips exactly that factor entry."""
    L = tiny(2, 128, 0, 1, 8, zero_T=True)
    base = F.unpack(F.pack(L))
    blob = bytearray(F.pack(L))
    h = F.parse_header(blob)
    for plane, idx, check in (("U0", 1, lambda A, B: (A.U != B.U).sum() == 1 and A.U[0, 0, 1] == -B.U[0, 0, 1]),
                              ("V0", 2, lambda A, B: (A.V != B.V).sum() == 1 and A.V[0, 2, 0] == -B.V[0, 2, 0])):
        b2 = bytearray(blob)
        b2[h[plane]] ^= 1 << (idx if plane == "U0" else 2)
        b2[176:184] = struct.pack("<Q", F.checksum(bytes(b2)))
        assert check(F.unpack(bytes(b2)), base)


@pytest.mark.parametrize("cfg", [0, 1, 4])
def test_roundtrip_config_shapes(cfg):
    if cfg == 4:
        m = synth.make_matrix(4, 0, 64, 17408, k=4, n_paths=2, rank=16, trit_fmt=1, scale_fmt=1)
    elif cfg == 1:
        m = synth.make_matrix(1, 0, 96, 4096, k=8, n_paths=1, rank=16)
    else:
        m = synth.config_matrix(0)
    L = F.from_synth(m)
    back = F.unpack(F.pack(L))
    for f in ["T", "site_pos", "site_sign", "alpha", "U", "V", "s"]:
        assert np.array_equal(getattr(L, f), getattr(back, f)), f
    if L.k:
        assert np.array_equal(L.beta, back.beta)


def test_rejections():
    L = tiny(2, 256, 4, 1, 4)
    good = F.pack(L)
    F.unpack(good)
    bad = bytearray(good)
    bad[0] ^= 1
    with pytest.raises(F.FormatError):
        F.unpack(bytes(bad))                       # magic
    bad = bytearray(good)
    bad[4] = 2
    with pytest.raises(F.FormatError):
        F.unpack(bytes(bad))                       # version
    bad = bytearray(good)
    bad[-1] ^= 0xFF
    with pytest.raises(F.FormatError):
        F.unpack(bytes(bad))                       # checksum
    with pytest.raises(F.FormatError):
        F.unpack(good[:-256])                      # short
    L2 = tiny(2, 256, 4, 1, 4)
    L2.site_pos[0, 0, 1] = L2.site_pos[0, 0, 0]
    with pytest.raises(F.FormatError):
        F.pack(L2)                                 # duplicate site
    L3 = tiny(2, 256, 4, 1, 4)
    L3.k = 3
    with pytest.raises(F.FormatError):
        F.pack(L3)
    L4 = tiny(2, 256, 4, 1, 4)
    L4.T[0, 0] = 2
    with pytest.raises(F.FormatError):
        F.pack(L4)


def test_unpack_rows_equals_full_unpack():
    for tf, sf, k, P in [(0, 0, 8, 1), (1, 1, 2, 2), (0, 1, 0, 0)]:
        L = tiny(9, 384, k, P, 5, tf, sf)
        blob = F.pack(L)
        rows = [0, 3, 8, 3]
        sub = F.unpack_rows(blob, rows)
        full = F.unpack(blob)
        for f in ["T", "site_pos", "site_sign", "alpha", "U"]:
            a = getattr(full, f)
            want = a[:, rows] if f == "U" else a[rows]
            assert np.array_equal(getattr(sub, f), want), f
        assert np.array_equal(sub.V, full.V) and np.array_equal(sub.s, full.s)
        x = np.random.default_rng(8).standard_normal(384)
        np.testing.assert_allclose(D.gemv_rows(blob, x, rows), D.gemv(blob, x)[rows], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# The normalised Hadamard-128 rotation (oracle/rotation.py)

def test_sylvester_entries_match_popcount_closed_form():
    """Sylvester's H has entry (-1)^popcount(i & j): a closed form of its own,
    independent of the doubling."""
    from oracle import rotation as Rt
    H = Rt.sylvester()
    i = np.arange(128)[:, None]
    j = np.arange(128)[None, :]
    pop = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(H, np.where(pop % 2 == 0, 1, -1))


def test_sylvester_is_orthogonal_and_symmetric():
    from oracle import rotation as Rt
    H = Rt.sylvester()
    assert np.array_equal(H @ H.T, 128 * np.eye(128, dtype=np.int64))
    assert np.array_equal(H, H.T)
    assert H[0].sum() == 128 and all(H[r].sum() == 0 for r in range(1, 128))


def test_rotation_special_vectors():
    """A constant group maps to sqrt(128) c at its first entry; a basis vector
    e_k of group g maps to column k of H / sqrt(128) inside group g only."""
    from oracle import rotation as Rt
    x = np.zeros(3 * 128)
    x[128:256] = 2.5
    y = Rt.rotate(x)
    expect = np.zeros(3 * 128)
    expect[128] = 2.5 * np.sqrt(128)
    assert np.allclose(y, expect, rtol=0, atol=1e-12)
    H = Rt.sylvester()
    for g, k in [(0, 0), (0, 77), (2, 127)]:
        e = np.zeros(3 * 128)
        e[g * 128 + k] = 1.0
        y = Rt.rotate(e)
        assert np.allclose(y[g * 128:(g + 1) * 128], H[:, k] / np.sqrt(128), rtol=0, atol=1e-15)
        assert not np.delete(y, np.arange(g * 128, (g + 1) * 128)).any()


def test_rotation_is_an_orthogonal_involution():
    """R is symmetric and orthogonal: it keeps norms, R R = I, and the rotated
    weights give the original product (W R)(R x) = W x."""
    from oracle import rotation as Rt
    rng = np.random.default_rng(5)
    X = rng.standard_normal((4, 512))
    Y = Rt.rotate(X)
    assert np.allclose(np.linalg.norm(Y, axis=1), np.linalg.norm(X, axis=1), rtol=1e-13)
    assert np.allclose(Rt.rotate(Y), X, rtol=0, atol=1e-12)
    W = rng.standard_normal((3, 512))
    Wr = Rt.rotate(W)          # rows of W R (R symmetric)
    assert np.allclose(Wr @ Y.T, W @ X.T, rtol=1e-12, atol=1e-12)


def test_rotation_rejects_partial_blocks():
    from oracle import rotation as Rt
    with pytest.raises(ValueError):
        Rt.rotate(np.zeros(200))


# ---------------------------------------------------------------------------
# INT4/g128 packed matrices (oracle/int4.py)

def test_int4_golden_bytes():
    """Worked by hand from the layout reading: nibble codes in two's
    complement, element 2i low; binary16 scales little-endian after them."""
    from oracle import int4 as I
    q = np.zeros((1, 128), dtype=np.int64)
    q[0, :8] = [-8, -7, -1, 0, 1, 2, 3, 7]
    b = I.pack(q, np.array([[0.5]]))
    assert b.size == 66
    assert list(b[:4]) == [0x98, 0x0F, 0x21, 0x73] and not b[4:64].any()
    assert list(b[64:]) == [0x00, 0x38]                       # 0.5 = 0x3800


def test_int4_size_matches_head_estimate():
    """The Qwen3-8B head (151936 x 4096) packs to ~0.32 GB, the figure the
    8B cards' INT4/g128 head implies."""
    from oracle import int4 as I
    n = I.size(151936, 4096)
    assert n == 151936 * 2048 + 151936 * 32 * 2 == 320_888_832


def test_int4_bruteforce_exact():
    """Tiny matrices against the definition in exact rationals."""
    from oracle import int4 as I
    rng = np.random.default_rng(7)
    V, inp = 3, 256
    q = rng.integers(-8, 8, size=(V, inp))
    s = rng.choice([0.25, 0.5, 1.5, -0.75, 2.0 ** -10, 3.0], size=(V, inp // 128))
    x = rng.integers(-5, 6, size=inp)
    y = I.gemv(I.pack(q, s), V, inp, x)
    for v in range(V):
        exact = sum(Fraction(float(s[v, j // 128])) * int(q[v, j]) * int(x[j]) for j in range(inp))
        assert Fraction(float(y[v])) == exact


def test_int4_columns_and_roundtrip():
    from oracle import int4 as I
    rng = np.random.default_rng(8)
    V, inp = 5, 384
    q = rng.integers(-8, 8, size=(V, inp))
    s = rng.integers(-64, 64, size=(V, 3)) / 16.0
    b = I.pack(q, s)
    q2, s2 = I.unpack(b, V, inp)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    for j in (0, 1, 127, 128, 383):
        e = np.zeros(inp)
        e[j] = 1.0
        assert np.array_equal(I.gemv(b, V, inp, e), s[:, j // 128] * q[:, j])
    rows = [4, 0, 2]
    x = rng.standard_normal(inp)
    assert np.allclose(I.gemv_rows(b, V, inp, x, rows), I.gemv(b, V, inp, x)[rows], rtol=0, atol=1e-12)


def test_int4_rejections():
    from oracle import int4 as I
    ok_s = np.ones((1, 1))
    with pytest.raises(ValueError):
        I.pack(np.full((1, 128), 8), ok_s)
    with pytest.raises(ValueError):
        I.pack(np.full((1, 128), -9), ok_s)
    with pytest.raises(ValueError):
        I.pack(np.zeros((1, 128), dtype=np.int64), np.array([[0.1]]))   # not binary16-exact
    with pytest.raises(ValueError):
        I.pack(np.zeros((1, 200), dtype=np.int64), np.ones((1, 1)))


def test_int4_rows_exact():
    """INT4 row lookup: every selected row equals s * q worked as exact
    rationals from the codes and scales; out-of-range ids give zero rows."""
    from oracle import int4 as I
    rng = np.random.default_rng(13)
    V, inp = 5, 256
    q = rng.integers(-8, 8, size=(V, inp))
    s = rng.integers(-64, 64, size=(V, 2)) / 16.0
    b = I.pack(q, s)
    ids = np.array([4, -3, 0, 4, 5, 2])
    R = I.rows(b, V, inp, ids)
    for n, v in enumerate(ids):
        if 0 <= v < V:
            assert [Fraction(float(t)) for t in R[n]] == [Fraction(float(s[v, j // 128])) * int(q[v, j])
                                                          for j in range(inp)]
        else:
            assert not R[n].any()


# ---------------------------------------------------------------------------
# INT3/g128 packed matrices and embedding rows (oracle/int3.py)

def test_int3_golden_bytes():
    """Worked by hand from the layout reading: one LSB-first bit stream per
    row, element j at stream bits 3j..3j+2, two's-complement codes."""
    from oracle import int3 as I
    q = np.zeros((1, 128), dtype=np.int64)
    q[0, :8] = [-4, 3, -1, 0, 1, 2, -2, -3]          # codes 100 011 111 000 001 010 110 101
    b = I.pack(q, np.array([[2.0]]))
    assert b.size == 48 + 2
    assert list(b[:3]) == [0xDC, 0x11, 0xB9] and not b[3:48].any()
    assert list(b[48:]) == [0x00, 0x40]                     # 2.0 = 0x4000


def test_int3_size_of_8b_embedding():
    from oracle import int3 as I
    assert I.size(151936, 4096) == 151936 * 1536 + 151936 * 32 * 2 == 243_097_600


def test_int3_rows_exact_roundtrip_and_rejections():
    from oracle import int3 as I
    rng = np.random.default_rng(9)
    V, inp = 6, 384
    q = rng.integers(-4, 4, size=(V, inp))
    s = rng.integers(-64, 64, size=(V, 3)) / 8.0
    b = I.pack(q, s)
    q2, s2 = I.unpack(b, V, inp)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    ids = np.array([5, 0, 5, 2, -1, 6])
    R = I.rows(b, V, inp, ids)
    for n, v in enumerate(ids):
        if 0 <= v < V:
            exact = [Fraction(float(s[v, j // 128])) * int(q[v, j]) for j in range(inp)]
            assert [Fraction(float(t)) for t in R[n]] == exact
        else:
            assert not R[n].any()
    with pytest.raises(ValueError):
        I.pack(np.full((1, 128), 4), np.ones((1, 1)))
    with pytest.raises(ValueError):
        I.pack(np.full((1, 128), -5), np.ones((1, 1)))
    with pytest.raises(ValueError):
        I.pack(np.zeros((1, 128), dtype=np.int64), np.array([[0.3]]))


# ---------------------------------------------------------------------------
# INT5/g128 packed matrices (oracle/int5.py)

def test_int5_golden_bytes():
    """Worked by hand from the layout reading: element j at stream bits
    5j..5j+4, stream bit b in bit b % 8 of byte b // 8, two's complement.
    Codes 1, -1, 15, -16 are 00001, 11111, 01111, 10000 (bit 0 first):
    stream bits 0..19 = 1 0000 11111 1111 0 0000 1, i.e. bytes 0xE1, 0x3F, 0x08."""
    from oracle import int5 as I
    q = np.zeros((1, 128), dtype=np.int64)
    q[0, :4] = [1, -1, 15, -16]
    b = I.pack(q, np.array([[0.5]]))
    assert b.size == 80 + 2
    assert list(b[:3]) == [0xE1, 0x3F, 0x08] and not b[3:80].any()
    assert list(b[80:]) == [0x00, 0x38]                       # 0.5 = 0x3800
    q = np.full((2, 128), -1, dtype=np.int64)                  # all ones: every code byte 0xFF
    b = I.pack(q, np.array([[1.0], [-2.0]]))
    assert (b[:160] == 0xFF).all() and list(b[160:]) == [0x00, 0x3C, 0x00, 0xC0]


def test_int5_bruteforce_exact():
    """Tiny matrices against the definition in exact rationals."""
    from oracle import int5 as I
    rng = np.random.default_rng(17)
    V, inp = 3, 256
    q = rng.integers(-16, 16, size=(V, inp))
    s = rng.choice([0.25, 0.5, 1.5, -0.75, 2.0 ** -10, 3.0], size=(V, inp // 128))
    x = rng.integers(-5, 6, size=inp)
    y = I.gemv(I.pack(q, s), V, inp, x)
    for v in range(V):
        exact = sum(Fraction(float(s[v, j // 128])) * int(q[v, j]) * int(x[j]) for j in range(inp))
        assert Fraction(float(y[v])) == exact


def test_int5_reduces_to_int4():
    """Codes inside [-8, 7] are the INT4 head's codes: the two packed forms
    of the same q and s give the same product (INT4 pinned above)."""
    from oracle import int4 as I4
    from oracle import int5 as I5
    rng = np.random.default_rng(18)
    V, inp = 7, 384
    q = rng.integers(-8, 8, size=(V, inp))
    s = rng.integers(-64, 64, size=(V, 3)) / 32.0
    x = rng.standard_normal(inp)
    assert np.array_equal(I5.gemv(I5.pack(q, s), V, inp, x), I4.gemv(I4.pack(q, s), V, inp, x))


def test_int5_columns_roundtrip_and_rejections():
    from oracle import int5 as I
    rng = np.random.default_rng(19)
    V, inp = 5, 384
    q = rng.integers(-16, 16, size=(V, inp))
    s = rng.integers(-64, 64, size=(V, 3)) / 16.0
    b = I.pack(q, s)
    assert b.size == I.size(V, inp) == V * 240 + V * 6
    q2, s2 = I.unpack(b, V, inp)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)
    for j in (0, 1, 6, 7, 8, 127, 128, 383):
        e = np.zeros(inp)
        e[j] = 1.0
        assert np.array_equal(I.gemv(b, V, inp, e), s[:, j // 128] * q[:, j])
    x = rng.standard_normal(inp)
    assert np.allclose(I.gemv_rows(b, V, inp, x, [4, 0, 2]), I.gemv(b, V, inp, x)[[4, 0, 2]], rtol=0, atol=1e-12)
    ok_s = np.ones((1, 1))
    for bad in (16, -17):
        with pytest.raises(ValueError):
            I.pack(np.full((1, 128), bad), ok_s)
    with pytest.raises(ValueError):
        I.pack(np.zeros((1, 128), dtype=np.int64), np.array([[0.1]]))
    with pytest.raises(ValueError):
        I.pack(np.zeros((1, 200), dtype=np.int64), np.ones((1, 1)))


def test_mixed_embedding_rows():
    """The RC1 mixed table: a map of all INT3 rows (or all INT4 rows) gives
    the pinned single-format lookups; a mixed map gives, row by row, s * q of
    the table the map names, in exact rationals; ids or map entries out of
    range give zero rows."""
    from oracle import int3 as I3
    from oracle import int4 as I4
    rng = np.random.default_rng(24)
    V, inp = 12, 256
    q3 = rng.integers(-4, 4, size=(V, inp))
    s3 = rng.integers(-64, 64, size=(V, 2)) / 8.0
    q4 = rng.integers(-8, 8, size=(V, inp))
    s4 = rng.integers(-64, 64, size=(V, 2)) / 16.0
    b3, b4 = I3.pack(q3, s3), I4.pack(q4, s4)
    ids = np.array([0, 11, 5, 5, -1, 12, 3])
    assert np.array_equal(I3.rows_mixed(b3, V, b4, V, inp, np.arange(V), ids), I3.rows(b3, V, inp, ids))
    assert np.array_equal(I3.rows_mixed(b3, V, b4, V, inp, -1 - np.arange(V), ids), I4.rows(b4, V, inp, ids))
    # 8 INT3 rows and 4 INT4 rows, interleaved; two map entries past their tables
    row_map = np.array([0, -1, 1, 2, -2, 3, 4, -3, 5, 6, -4, 7])
    row_map_bad = row_map.copy()
    row_map_bad[2], row_map_bad[4] = 8, -5        # INT3 table of 8 rows, INT4 of 4
    t3, t4 = I3.pack(q3[:8], s3[:8]), I4.pack(q4[:4], s4[:4])
    R = I3.rows_mixed(t3, 8, t4, 4, inp, row_map, np.arange(V))
    Rb = I3.rows_mixed(t3, 8, t4, 4, inp, row_map_bad, np.arange(V))
    for v in range(V):
        m = row_map[v]
        if m >= 0:
            exact = [Fraction(float(s3[m, j // 128])) * int(q3[m, j]) for j in range(inp)]
        else:
            exact = [Fraction(float(s4[-1 - m, j // 128])) * int(q4[-1 - m, j]) for j in range(inp)]
        assert [Fraction(float(t)) for t in R[v]] == exact
        if v in (2, 4):
            assert not Rb[v].any()
        else:
            assert np.array_equal(Rb[v], R[v])

