"""CPU tests of libwal's host side through its C ABI.

* the library loads and exports every function include/wal.h declares;
* the C++ packer writes the same bytes as the oracle's independent numpy
  packer, on every workload configuration's shapes and formats;
* wal_unpack inverts wal_pack; wal_packed_size matches the oracle's layout;
* malformed inputs are rejected with their documented status before use.
No GPU call is made here.
"""
import os
import re
import struct

import numpy as np
import pytest

import synth
import ternary_hybrid_bit_amd as wal
from oracle import format as F

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "wal.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wal_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    import ctypes
    lib = ctypes.CDLL(wal.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(wal.exported_symbols())


def test_status_strings():
    for code in range(0, -10, -1):
        assert wal.wal_status_str(code).startswith(wal.STATUS[code])


def _same_bytes(m):
    cpp, info = wal.pack_matrix(m)
    ref = np.frombuffer(F.pack(F.from_synth(m)), dtype=np.uint8)
    assert cpp.size == ref.size == info.total_bytes
    diff = np.nonzero(cpp != ref)[0]
    assert diff.size == 0, f"first differing byte {diff[:8]}"
    return cpp, info


@pytest.mark.parametrize("cfg,mid", [(0, 0), (1, 0), (3, 0), (4, 0), (4, 1)])
def test_cpp_pack_matches_oracle_full_configs(cfg, mid):
    m = synth.config_matrix(cfg, mid)
    cpp, info = _same_bytes(m)
    lay = F.layout(m.out, m.inp, m.k, m.n_paths, m.rank, m.trit_fmt, m.scale_fmt)
    assert info.off_codes == lay["codes"] and info.total_bytes == lay["total"]
    assert info.algorithmic_bytes == F.algorithmic_bytes(m.out, m.inp, m.k, m.n_paths, m.rank,
                                                         m.trit_fmt, m.scale_fmt)


@pytest.mark.parametrize("mid", [0, 1, 2, 6, 8, 13])
def test_cpp_pack_matches_oracle_sweep_matrices(mid):
    """Sweep matrices of each shape (q, k, v, down with and without a path)."""
    _same_bytes(synth.config_matrix(2, mid))


@pytest.mark.parametrize("out,inp,k,P,r,tf,sf", [
    (1, 128, 0, 0, 0, 0, 0), (3, 384, 2, 1, 3, 0, 1), (5, 640, 4, 3, 9, 1, 0),
    (7, 1152, 8, 4, 64, 1, 1), (2, 17408, 8, 2, 16, 1, 1), (2, 128, 2, 1, 1, 1, 0),
])
def test_cpp_pack_matches_oracle_edge_shapes(out, inp, k, P, r, tf, sf):
    m = synth.make_matrix(50, out * 7 + inp, out, inp, k=k, n_paths=P, rank=r, trit_fmt=tf, scale_fmt=sf)
    cpp, _ = _same_bytes(m)
    back = wal.wal_unpack(cpp)
    assert np.array_equal(back["T"], m.T)
    assert np.array_equal(back["alpha"], m.alpha)
    if k:
        assert np.array_equal(back["site_pos"], m.site_pos)
        assert np.array_equal(back["site_sign"], m.site_sign)
        assert np.array_equal(back["beta"], m.beta)
    if P:
        assert np.array_equal(back["U"], m.U) and np.array_equal(back["V"], m.V)
        assert np.array_equal(back["s"], m.s)


def test_packed_size_matches_oracle_layout():
    for (o, i, k, P, r, tf, sf) in [(12288, 4096, 8, 1, 16, 0, 0), (5120, 17408, 4, 2, 16, 1, 1),
                                    (256, 512, 8, 0, 0, 0, 0), (17408, 5120, 0, 2, 16, 1, 1)]:
        info = wal.wal_packed_size(wal.make_desc(o, i, k, P, r, tf, sf))
        lay = F.layout(o, i, k, P, r, tf, sf)
        assert info.total_bytes == lay["total"]
        assert info.off_alpha == lay["alpha"] and info.off_beta == lay["beta"]
        for p in range(P):
            assert info.off_V[p] == lay[f"V{p}"] and info.off_U[p] == lay[f"U{p}"]
            assert info.off_s[p] == lay[f"s{p}"]
        assert info.row_stride == F.row_stride(i, tf)


def _status_of(fn):
    with pytest.raises(wal.WalError) as e:
        fn()
    return e.value.status


def test_pack_rejects_bad_logical_inputs():
    m = synth.make_matrix(51, 0, 4, 256, k=4, n_paths=1, rank=4)
    d = wal.make_desc(4, 256, 4, 1, 4)

    def pack(**kw):
        a = dict(T=m.T, site_pos=m.site_pos, site_sign=m.site_sign, alpha=m.alpha, beta=m.beta,
                 U=m.U, V=m.V, s=m.s)
        a.update(kw)
        return wal.wal_pack(d, **a)

    T = m.T.copy(); T[1, 3] = 2
    assert _status_of(lambda: pack(T=T)) == -3
    sp = m.site_pos.copy(); sp[0, 0, 1] = sp[0, 0, 0]
    assert _status_of(lambda: pack(site_pos=sp)) == -3
    sp = m.site_pos.copy(); sp[0, 0, 3] = 128
    assert _status_of(lambda: pack(site_pos=sp)) == -3
    sg = m.site_sign.copy(); sg[2, 1, 0] = 0
    assert _status_of(lambda: pack(site_sign=sg)) == -3
    U = m.U.copy(); U[0, 0, 0] = 0
    assert _status_of(lambda: pack(U=U)) == -3
    a = m.alpha.copy(); a[0, 0] = 0.1
    assert _status_of(lambda: pack(alpha=a)) == -4
    s = m.s.copy(); s[0, 0] = 1e-5 + 1e-9
    assert _status_of(lambda: pack(s=s)) == -4
    assert _status_of(lambda: wal.wal_pack(wal.make_desc(4, 200, 4, 1, 4), m.T)) == -2
    assert _status_of(lambda: wal.wal_pack(wal.make_desc(4, 256, 3, 1, 4), m.T)) == -2
    assert _status_of(lambda: wal.wal_pack(wal.make_desc(4, 256, 4, 5, 4), m.T)) == -2
    assert _status_of(lambda: wal.wal_pack(wal.make_desc(4, 256, 4, 1, 65), m.T)) == -2
    assert _status_of(lambda: wal.wal_pack(d, m.T, None, None, m.alpha, m.beta, m.U, m.V, m.s)) == -1


def test_fp24_pack_rejects_low_bits():
    m = synth.make_matrix(52, 0, 2, 128, k=2, n_paths=0, trit_fmt=1, scale_fmt=1)
    a = m.alpha.copy()
    a.view(np.uint32)[0, 0] |= 1
    d = wal.make_desc(2, 128, 2, 0, 0, 1, 1)
    assert _status_of(lambda: wal.wal_pack(d, m.T, m.site_pos, m.site_sign, a, m.beta)) == -4


def _refresh(blob):
    b = bytearray(blob)
    b[176:184] = struct.pack("<Q", F.checksum(bytes(b)))
    return np.frombuffer(bytes(b), dtype=np.uint8).copy()


def test_verify_rejects_corruption():
    m = synth.make_matrix(53, 0, 4, 256, k=8, n_paths=1, rank=9, trit_fmt=0)
    blob, info = wal.pack_matrix(m)
    assert wal.wal_verify(blob) == 0
    bad = blob.copy(); bad[0] ^= 1
    assert wal.wal_verify(bad) == -7                                   # magic
    bad = blob.copy(); bad[4] = 9
    assert wal.wal_verify(bad) == -7                                   # version
    bad = blob.copy(); bad[info.off_codes + 5] ^= 0x10
    assert wal.wal_verify(bad) == -7                                   # checksum
    assert wal.wal_verify(blob[:-256].copy()) == -5                    # short
    bad = blob.copy(); bad[info.off_codes] = (bad[info.off_codes] & 0xFC) | 2
    assert wal.wal_verify(_refresh(bad)) == -3                         # code 10
    bad = blob.copy(); bad[info.off_sites + 1] = bad[info.off_sites]
    assert wal.wal_verify(_refresh(bad)) == -3                         # repeated site
    bad = blob.copy(); bad[info.off_U[0] + 1] |= 0x80                  # pad bit of U (rank 9)
    assert wal.wal_verify(_refresh(bad)) == -3
    bad = blob.copy(); bad[40] ^= 1
    assert wal.wal_verify(bad) == -7                                   # layout field
    bad = blob.copy(); bad[200] = 1
    assert wal.wal_verify(bad) == -7                                   # reserved bytes


def test_verify_rejects_base3_corruption():
    m = synth.make_matrix(54, 0, 2, 384, k=0, n_paths=0, trit_fmt=1)
    blob, info = wal.pack_matrix(m)
    assert wal.wal_verify(blob) == 0
    bad = blob.copy(); bad[info.off_codes + 3] = 243
    assert wal.wal_verify(_refresh(bad)) == -3
    # 384 trits = 76.8 bytes: byte 76 holds 4 trits + 1 filler digit that must be 1
    bad = blob.copy(); bad[info.off_codes + 76] = (bad[info.off_codes + 76] % 81)   # filler digit -> 0
    assert wal.wal_verify(_refresh(bad)) == -3
    bad = blob.copy(); bad[info.off_codes + 79] = 0                     # row padding
    assert wal.wal_verify(_refresh(bad)) == -3


def test_inspect_reads_header():
    m = synth.make_matrix(55, 0, 6, 640, k=2, n_paths=2, rank=5, trit_fmt=1, scale_fmt=1)
    blob, info = wal.pack_matrix(m)
    got = wal.wal_inspect(blob)
    assert (got.d.out, got.d.in_, got.d.k, got.d.n_paths, got.d.rank) == (6, 640, 2, 2, 5)
    assert got.total_bytes == info.total_bytes and got.off_s[1] == info.off_s[1]


def test_workspace_size():
    """Synchronisation words (4352 bytes: 33 lines of 128) and 4096 arrival
    counters, the same for every shape | low-rank partials z [chunk][batch][terms] (one chunk
    per 4096 columns) | partial sums [slices][batch][out] of the small-batch
    kernels (one slice per 1024 columns), each padded to 256 bytes."""
    def up(v):
        return (v + 255) // 256 * 256

    def zsplits(inp, terms, B):   # column splits of the low-rank pre-pass
        G = inp // 128
        tiles = -(-B // 16) * -(-terms // 16)
        s = min(max(1, -(-1024 // tiles)), 8, G)
        per = -(-G // s)
        return -(-G // per)

    def expect(out, inp, terms, B):
        chunks, slices = (inp + 4095) // 4096, (inp + 1023) // 1024
        z = max(4 * terms * B * chunks, 8 * terms * ((inp + 8191) // 8192))   # fp32, or tagged for batch 1
        return 4352 + 4 * 4096 + up(z) + up(4 * slices * B * out)

    info = wal.wal_packed_size(wal.make_desc(12288, 4096, 8, 1, 16))
    assert wal.wal_workspace_size(info, 1) == expect(12288, 4096, 16, 1) == 20736 + 256 + 4 * 49152
    assert wal.wal_workspace_size(info, 32) == expect(12288, 4096, 16, 32)
    assert wal.WAL_WS_ZERO_BYTES == 20736
    info = wal.wal_packed_size(wal.make_desc(4096, 12288, 8, 1, 16))
    for B in (1, 4, 16, 17, 32):
        assert wal.wal_workspace_size(info, B) == expect(4096, 12288, 16, B)
    assert wal.wal_workspace_size(wal.wal_packed_size(wal.make_desc(256, 512, 8)), 1) == expect(256, 512, 0, 1)
    with pytest.raises(wal.WalError):
        wal.wal_workspace_size(info, 33)


def test_prefill_workspace_size():
    """Low-rank partials z [zc][batch][terms] (zc column splits that bring the
    pre-pass to about 1024 wavefronts, at most 8) | per-split partial sums
    [splits][batch][out] when the K dimension is split: splits are made only
    while the tiles (256 rows with fp16 scales, 128 with fp24, by 64 batch
    rows) number fewer than 256, at most one per 2-group sweep."""
    def up(v):
        return (v + 255) // 256 * 256

    def zsplits(inp, terms, B):   # column splits of the low-rank pre-pass
        G = inp // 128
        tiles = -(-B // 16) * -(-terms // 16)
        s = min(max(1, -(-1024 // tiles)), 8, G)
        per = -(-G // s)
        return -(-G // per)

    def expect(out, inp, terms, B):
        tiles = ((out + 255) // 256) * ((B + 63) // 64)
        sweeps = (inp // 128 + 1) // 2
        nsplit = 1 if tiles >= 256 else min(sweeps, -(-256 // tiles))
        z = up(4 * terms * B * zsplits(inp, terms, B)) if terms else 0
        return z + (up(4 * nsplit * B * out) if nsplit > 1 else 0), nsplit

    info = wal.wal_packed_size(wal.make_desc(4096, 12288, 8, 1, 16))
    for B in (1, 64, 96, 200, 256, 512, 1024, 2048):
        n, nsplit = expect(4096, 12288, 16, B)
        assert wal.wal_prefill_workspace_size(info, B) == n, B
    assert expect(4096, 12288, 16, 64)[1] == 16 and expect(4096, 12288, 16, 1024)[1] == 1
    info = wal.wal_packed_size(wal.make_desc(64, 512, 0))
    assert wal.wal_prefill_workspace_size(info, 1) == up(4 * 2 * 1 * 64)   # two splits of one sweep each
    info = wal.wal_packed_size(wal.make_desc(64, 256, 0))
    assert wal.wal_prefill_workspace_size(info, 1) == 0                     # one sweep: nothing to split
    info = wal.wal_packed_size(wal.make_desc(16384, 512, 0))
    assert wal.wal_prefill_workspace_size(info, 1024) == 0                 # no paths, no split
    fp24 = wal.wal_packed_size(wal.make_desc(4096, 12288, 8, 1, 16, scale_fmt=1))
    n = wal.wal_prefill_workspace_size(fp24, 512)   # 32 x 8 tiles: whole K
    assert n == up(4 * 16 * 512 * zsplits(12288, 16, 512))
    assert wal.wal_prefill_workspace_size(fp24, 256) == up(4 * 16 * 256 * zsplits(12288, 16, 256)) + up(4 * 2 * 256 * 4096)
    with pytest.raises(wal.WalError):
        wal.wal_prefill_workspace_size(info, 0)
    with pytest.raises(wal.WalError):
        wal.wal_prefill_workspace_size(info, wal.WAL_MAX_PREFILL_BATCH + 1)


def test_product_calls_check_arguments_before_any_launch():
    """Host-side checks of the product entry points return their status
    before touching the GPU (the pointers below are never dereferenced)."""
    import ctypes
    info = wal.wal_packed_size(wal.make_desc(64, 256, 8, 1, 16))
    lib = wal._lib
    W, x, y, ws = 0x10000, 0x20000, 0x30000, 0x40000
    n1 = wal.wal_workspace_size(info, 1)
    ok_args = (ctypes.byref(info), W, x, wal.WAL_X_BF16, y, ws, n1, None)
    assert lib.wal_gemv(ctypes.byref(info), W + 16, x, 1, y, ws, n1, None) == -6     # W not 256-aligned
    assert lib.wal_gemv(ctypes.byref(info), W, x + 2, 1, y, ws, n1, None) == -6      # x not 16-aligned
    assert lib.wal_gemv(ctypes.byref(info), W, x, 1, y + 2, ws, n1, None) == -6      # y not 4-aligned
    assert lib.wal_gemv(ctypes.byref(info), W, x, 1, y, ws, 8, None) == -5           # workspace too small
    assert lib.wal_gemv(ctypes.byref(info), W, x, 1, y, None, 0, None) == -1         # workspace missing
    assert lib.wal_gemv(ctypes.byref(info), W, x, 1, y, ws + 8, n1, None) == -6      # workspace misaligned
    assert lib.wal_gemv(ctypes.byref(info), W, x, 7, y, ws, n1, None) == -1          # dtype
    assert lib.wal_gemv(ctypes.byref(info), None, x, 1, y, ws, n1, None) == -1
    assert lib.wal_gemv(ctypes.byref(info), W, x, 1, x + 64, ws, n1, None) == -1     # y overlaps x
    assert lib.wal_gemv(ctypes.byref(info), W, x, 1, y, x, n1, None) == -1           # workspace overlaps x
    bad = wal.wal_info.from_buffer_copy(info)
    bad.off_alpha += 256
    assert lib.wal_gemv(ctypes.byref(bad), *ok_args[1:]) == -7                       # inconsistent info
    need = wal.wal_workspace_size(info, 2)
    gs = lambda *a: lib.wal_gemm_small(ctypes.byref(info), *a)  # noqa: E731
    assert gs(W, x, 1, 0, 256, y, 64, 0, ws, need, None) == -1               # batch 0
    assert gs(W, x, 1, 33, 256, y, 64, 0, ws, need, None) == -1              # batch > 32
    assert gs(W, x, 1, 2, 256, y, 64, 3, ws, need, None) == -1               # mode
    assert gs(W, x, 1, 2, 255, y, 64, 0, ws, need, None) == -1               # ldx < in
    assert gs(W, x, 1, 2, 256, y, 63, 0, ws, need, None) == -1               # ldy < out
    assert gs(W, x, 1, 2, 260, y, 64, 0, ws, need, None) == -6               # row pitch
    assert gs(W, x, 1, 2, 256, y, 64, 0, ws, need - 4, None) == -5           # workspace too small
    assert gs(W, x, 1, 2, 256, y, 64, 0, None, 0, None) == -1                # workspace missing
    assert gs(W, x, 1, 2, 256, y, 64, 0, x + 256, need, None) == -1          # workspace overlaps X
    need = wal.wal_prefill_workspace_size(info, 64)
    gp = lambda *a: lib.wal_gemm_prefill(ctypes.byref(info), *a)  # noqa: E731
    assert gp(W, x, 1, 0, 256, y, 64, ws, need, None) == -1                  # batch 0
    assert gp(W, x, 1, 16385, 256, y, 64, ws, need, None) == -1              # batch too large
    assert gp(W, x, 0, 64, 256, y, 64, ws, need, None) == -9                 # fp32 activations
    assert gp(W, x, 1, 64, 255, y, 64, ws, need, None) == -1                 # ldx < in
    assert gp(W, x, 1, 64, 260, y, 64, ws, need, None) == -6                 # row pitch
    assert gp(W, x, 1, 64, 256, y, 64, ws, need - 4, None) == -5             # workspace too small
    assert gp(W, x, 1, 64, 256, y, 64, None, 0, None) == -1                  # workspace missing
    assert gp(W, x, 1, 64, 256, x + 256, 64, ws, need, None) == -1           # Y overlaps X
    assert gp(W, x, 1, 16384, 1 << 17, y, 64, ws, need, None) == -2          # X beyond 2 GiB
    assert lib.wal_gemv_grouped(None, 0x1000, None) == -1
    assert lib.wal_gemv_grouped_seq(0, None, None, None) == -1
    # the rotation flag: accepted by the batch-1 products (their other checks
    # still apply), refused by the batched ones, other flag bits rejected
    R = wal.WAL_X_ROT_H128
    assert lib.wal_gemv(ctypes.byref(info), W, x, 1 | R, y, ws, 8, None) == -5          # flag accepted
    assert lib.wal_gemv(ctypes.byref(info), W, x, 1 | 32, y, ws, n1, None) == -1        # unknown flag
    assert lib.wal_gemv(ctypes.byref(info), W, x, 2 | R, y, ws, n1, None) == -1         # bad type, flag
    need = wal.wal_workspace_size(info, 2)
    assert gs(W, x, 1 | R, 2, 256, y, 64, 0, ws, need, None) == -9
    assert gs(W, x, 0 | R, 2, 256, y, 64, 0, ws, need, None) == -9
    need = wal.wal_prefill_workspace_size(info, 64)
    assert gp(W, x, 1 | R, 64, 256, y, 64, ws, need, None) == -9
    rot = lib.wal_rotate_h128
    assert rot(None, 1, 1, 128, 128, y, 1, 128, None) == -1                     # x missing
    assert rot(x, 1, 0, 128, 128, y, 1, 128, None) == -1                        # no rows
    assert rot(x, 2, 1, 128, 128, y, 1, 128, None) == -1                        # dtype
    assert rot(x, 1, 1, 200, 256, y, 1, 256, None) == -2                        # not a multiple of 128
    assert rot(x, 1, 1, 256, 128, y, 1, 256, None) == -1                        # ldx < in
    assert rot(x + 2, 1, 1, 128, 128, y, 1, 128, None) == -6                    # x misaligned
    assert rot(x, 1, 2, 128, 132, y, 1, 128, None) == -6                        # row pitch
    assert rot(x, 1, 2, 128, 128, x + 256, 1, 128, None) == -1                  # partial overlap
    assert rot(x, 1, 2, 128, 128, x, 0, 128, None) == -1                        # same buffer, other type
    assert lib.wal_graph_create(0, None, None, None) == -1
    h = ctypes.c_void_p()
    assert lib.wal_graph_create(0, None, None, ctypes.byref(h)) == -1
    assert lib.wal_graph_launch(None, None) == -1
    assert lib.wal_graph_destroy(None) == 0


def _plan_on_host(infos, grid, x_dtype=wal.WAL_X_BF16):
    """Build a grouped plan with fake (aligned, never dereferenced) device
    pointers; returns (plan bytes, wal_grouped_info)."""
    import ctypes
    n = len(infos)
    arr = (wal.wal_info * n)(*infos)
    pb, wsb = wal.wal_grouped_plan_size(infos, grid, x_dtype)
    plan = np.zeros(pb, np.uint8)
    base = 1 << 40
    Wp = (ctypes.c_void_p * n)(*[base + i * (1 << 28) for i in range(n)])
    xp = (ctypes.c_void_p * n)(*[base + (1 << 36) + i * (1 << 20) for i in range(n)])
    yp = (ctypes.c_void_p * n)(*[base + (1 << 37) + i * (1 << 20) for i in range(n)])
    ginfo = wal.wal_grouped_info()
    st = wal._lib.wal_grouped_plan(n, arr, Wp, xp, x_dtype, yp, base + (1 << 38), max(wsb, 256), grid,
                                   plan.ctypes.data, plan.size, ctypes.byref(ginfo))
    assert st == 0, wal.STATUS.get(st, st)
    return plan, ginfo


def _class_of(info):
    return 8 * info.d.trit_fmt + 4 * info.d.scale_fmt + {0: 0, 2: 1, 4: 2, 8: 3}[info.d.k]


def _plan_classes(plan, g):
    """[(class id, blockseg, segs)] and the low-rank jobs of a plan."""
    out = []
    for c in range(g.n_classes):
        G = g.class_grid[c]
        blockseg = np.frombuffer(plan, np.uint32, G + 1, g.class_blockseg[c])
        segs = np.frombuffer(plan, np.uint32, 4 * int(blockseg[-1]), g.class_segs[c]).reshape(-1, 4)
        out.append((g.class_id[c], blockseg, segs))
    jobs = np.frombuffer(plan, np.uint32, 2 * g.n_zjobs, g.off_zjobs).reshape(-1, 2)
    return out, jobs


def _passes(info):
    return -(-info.d.in_ // (4096 if info.d.trit_fmt == 0 else 5120))


def _row_bytes(info):
    return ((info.d.in_ // 4 if info.d.trit_fmt == 0 else (info.d.in_ + 4) // 5)
            + (info.d.in_ // 128) * (info.d.k + (2 if info.d.scale_fmt == 0 else 3) * (2 if info.d.k else 1))
            + info.d.n_paths * ((info.d.rank + 7) // 8))


def _pass_row_bytes(info, p):
    w = 4096 if info.d.trit_fmt == 0 else 5120
    pw = min(w, info.d.in_ - p * w)
    return max(1, (_row_bytes(info) * pw + info.d.in_ // 2) // info.d.in_)


@pytest.mark.parametrize("grid", [1, 7, 768, 1024, 3000, 6000])
def test_grouped_plan_covers_every_row_once(grid):
    """Per (scale format, k) class, the grouped plan splits the rows of the
    class's matrices into `grid` contiguous ranges of near-equal packed
    bytes; every row of every matrix belongs to exactly one workgroup of the
    launch of its class, for every pass.  A class with more workgroups than
    16-row groups splits its matrices of several passes by pass: segments of
    one pass start at multiples of 16 rows."""
    shapes = [(4096, 4096, 8, 1, 16, 0, 0), (1024, 4096, 8, 0, 0, 0, 0), (1024, 4096, 8, 1, 16, 0, 0),
              (4096, 4096, 8, 1, 16, 0, 0), (12288, 4096, 8, 1, 16, 0, 0), (300, 4096, 2, 0, 0, 1, 0),
              (12288, 4096, 8, 0, 0, 0, 0), (4096, 12288, 8, 1, 16, 0, 0), (1, 128, 2, 0, 0, 0, 0),
              (7, 384, 4, 4, 64, 0, 0), (129, 512, 2, 1, 8, 1, 0), (17408, 5120, 2, 2, 16, 1, 1),
              (5120, 17408, 4, 2, 16, 1, 1), (3000, 640, 8, 0, 0, 0, 1), (200, 8960, 4, 1, 16, 0, 0)]
    infos = [wal.wal_packed_size(wal.make_desc(o, i, k, P, r, trit_fmt=tf, scale_fmt=sf))
             for o, i, k, P, r, sf, tf in shapes]
    plan, g = _plan_on_host(infos, grid)
    # the synchronisation words are the workspace's (it starts with them)
    assert g.sync_dev == (1 << 40) + (1 << 38) and g.off_descs == 64
    classes, jobs = _plan_classes(plan, g)
    assert sorted(c for c, _, _ in classes) == sorted(set(_class_of(i) for i in infos))
    assert sum(len(sg) for _, _, sg in classes) == g.n_segs
    covered = [np.zeros((o, _passes(infos[m])), np.int32) for m, (o, *_) in enumerate(shapes)]
    n_split = 0
    for c, blockseg, segs in classes:
        members = [m for m in range(len(infos)) if _class_of(infos[m]) == c]
        groups = sum(-(-shapes[m][0] // 16) for m in members)
        split = grid > groups and any(_passes(infos[m]) > 1 for m in members)
        assert len(blockseg) == grid + 1 and blockseg[0] == 0
        assert np.all(np.diff(blockseg.astype(np.int64)) >= 0)
        per_block = np.zeros(grid)
        for b in range(grid):
            for m, r0, r1, pass1 in segs[blockseg[b]:blockseg[b + 1]]:
                assert _class_of(infos[m]) == c
                assert r0 < r1 <= shapes[m][0]
                assert r1 - r0 <= (1024 if c >= 8 else 4096)   # rows whose y one workgroup stages
                if pass1:
                    assert split and _passes(infos[m]) > 1 and r0 % 16 == 0
                    covered[m][r0:r1, pass1 - 1] += 1
                    per_block[b] += (r1 - r0) * _pass_row_bytes(infos[m], pass1 - 1)
                    n_split += 1
                else:
                    assert not (split and _passes(infos[m]) > 1)
                    covered[m][r0:r1, :] += 1
                    per_block[b] += (r1 - r0) * _row_bytes(infos[m])
        # streamed bytes per workgroup are balanced to within a row of the
        # class's widest matrix (16 rows of a pass in split matrices)
        def rb(m):
            return 16 * _pass_row_bytes(infos[m], 0) if split and _passes(infos[m]) > 1 else _row_bytes(infos[m])
        def total(m):
            if split and _passes(infos[m]) > 1:
                return sum(_pass_row_bytes(infos[m], p) for p in range(_passes(infos[m]))) * shapes[m][0]
            return _row_bytes(infos[m]) * shapes[m][0]
        ideal = sum(total(m) for m in members) / grid
        # small ranges (<= 256 KiB) may snap to a matrix start, within half a range
        snap = ideal / 2 if ideal <= 256 * 1024 else 0
        assert per_block.max() <= ideal + snap + max(rb(m) for m in members) + 1
    for c in covered:
        assert np.all(c == 1)
    if grid == 6000:
        assert n_split > 0   # some class has more workgroups than 16-row groups
    # one low-rank job per zjob_terms terms and 4096-column chunk of every
    # matrix that has paths: (matrix, t0 << 16 | chunk); 4-term jobs when
    # that makes at most 64 jobs, else 16-term jobs
    def jobs_of(step):
        return [(m, (t0 << 16) | cc) for m, (o, i, k, P, r, sf, tf) in enumerate(shapes)
                for cc in range((i + 4095) // 4096) for t0 in range(0, P * r, step)]
    assert g.zjob_terms == (4 if len(jobs_of(4)) <= 64 else 16)
    want = jobs_of(g.zjob_terms)
    assert sorted(map(tuple, jobs.tolist())) == sorted(want)


def test_grouped_plan_records_rotation_flag():
    """A plan built with WAL_X_ROT_H128 keeps the flag in its info (its
    launches take the kernels that rotate x) and is laid out like the plain
    plan; unknown flag bits are rejected."""
    import ctypes
    infos = [wal.wal_packed_size(wal.make_desc(o, n, 8, p, 16 if p else 0)) for o, n, p in
             [(512, 4096, 1), (300, 12288, 0)]]
    plan0, g0 = _plan_on_host(infos, 64, wal.WAL_X_BF16)
    plan1, g1 = _plan_on_host(infos, 64, wal.WAL_X_BF16 | wal.WAL_X_ROT_H128)
    assert g0.x_dtype == wal.WAL_X_BF16 and g1.x_dtype == wal.WAL_X_BF16 | wal.WAL_X_ROT_H128
    assert g0.plan_bytes == g1.plan_bytes and g0.n_segs == g1.n_segs and g0.n_zjobs == g1.n_zjobs
    _, g2 = _plan_on_host(infos, 64, wal.WAL_X_F32 | wal.WAL_X_ROT_H128)
    assert g2.x_dtype == wal.WAL_X_ROT_H128
    arr = (wal.wal_info * 2)(*infos)
    pb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    assert wal._lib.wal_grouped_plan_size(2, arr, 64, 1 | 64, ctypes.byref(pb), ctypes.byref(wb)) == -1


def test_grouped_plan_job_size():
    """Low-rank jobs of 4 terms when a plan has at most 64 of them, else of 16
    terms (per 4096-column chunk of each matrix with paths)."""
    small = [wal.wal_packed_size(wal.make_desc(4096, 4096, 8, 1, 16))] * 3
    _, g = _plan_on_host(small, 64)
    assert (g.zjob_terms, g.n_zjobs) == (4, 3 * 4)
    large = [wal.wal_packed_size(wal.make_desc(4096, 12288, 8, 1, 16))] * 20
    _, g = _plan_on_host(large, 64)
    assert (g.zjob_terms, g.n_zjobs) == (16, 20 * 3)
    edge = [wal.wal_packed_size(wal.make_desc(256, 4096, 8, 2, 32))] * 4   # 4 x 16 = 64 jobs of 4 terms
    _, g = _plan_on_host(edge, 64)
    assert (g.zjob_terms, g.n_zjobs) == (4, 64)


def test_grouped_plan_rejects_bad_arguments():
    import ctypes
    infos = [wal.wal_packed_size(wal.make_desc(64, 256, 8, 1, 16))]
    with pytest.raises(wal.WalError):
        wal.wal_grouped_plan_size(infos, 16, 7)                  # x dtype
    one = (ctypes.c_void_p * 1)(1 << 40)
    arr = (wal.wal_info * 1)(*infos)
    pb, wsb = wal.wal_grouped_plan_size(infos, 4)
    buf = np.zeros(pb, np.uint8)
    ginfo = wal.wal_grouped_info()
    y = (ctypes.c_void_p * 1)(1 << 41)
    # workspace missing, plan buffer too small, misaligned x
    assert wal._lib.wal_grouped_plan(1, arr, one, one, 1, y, None, 0, 4, buf.ctypes.data, buf.size,
                                     ctypes.byref(ginfo)) == -1
    assert wal._lib.wal_grouped_plan(1, arr, one, one, 1, y, 1 << 42, wsb, 4, buf.ctypes.data, buf.size - 64,
                                     ctypes.byref(ginfo)) == -5
    assert wal._lib.wal_grouped_plan(1, arr, one, (ctypes.c_void_p * 1)((1 << 40) + 2), 1, y, 1 << 42, wsb, 4,
                                     buf.ctypes.data, buf.size, ctypes.byref(ginfo)) == -6
    assert wal._lib.wal_gemv_grouped(ctypes.byref(wal.wal_grouped_info()), 1 << 40, None) == -1


def test_int4_pack_matches_oracle_and_rejects():
    """INT4/g128: the C++ packer writes the oracle's bytes; bad codes, inexact
    scales, shapes and short buffers are rejected; the product entry checks
    its arguments before any launch."""
    import ctypes
    from oracle import int4 as I
    rng = np.random.default_rng(21)
    for V, inp in [(1, 128), (5, 384), (64, 4224)]:
        q = rng.integers(-8, 8, size=(V, inp)).astype(np.int8)
        s = (rng.integers(-2048, 2048, size=(V, inp // 128)) / 256.0).astype(np.float32)
        b = wal.wal_int4_pack(q, s)
        assert np.array_equal(b, I.pack(q, s.astype(np.float64)))
        q2, s2 = wal.wal_int4_unpack(b, V, inp)
        assert np.array_equal(q2, q) and np.array_equal(s2, s)
    assert wal.wal_int4_size(151936, 4096) == I.size(151936, 4096)
    lib = wal._lib
    # V * in past 2^40 is refused: its byte count would wrap 64 bits at the largest shapes
    n = ctypes.c_size_t(0)
    for size in (lib.wal_int3_size, lib.wal_int4_size, lib.wal_int5_size):
        assert size(1 << 20, 1 << 20, ctypes.byref(n)) == 0
        assert size((1 << 20) + 1, 1 << 20, ctypes.byref(n)) == -2
        assert size(0xFFFFFFFF, 0xFFFFFF80, ctypes.byref(n)) == -2
    buf = np.zeros(I.size(2, 256), np.uint8)
    q = np.zeros((2, 256), np.int8)
    s = np.ones((2, 2), np.float32)
    assert lib.wal_int4_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size - 1) == -5
    assert lib.wal_int4_pack(2, 200, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -2
    q[1, 3] = 8
    assert lib.wal_int4_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -3
    q[1, 3] = 0
    s[0, 1] = 0.1
    assert lib.wal_int4_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -4
    assert not buf.any()                                   # nothing written on rejection
    g = lib.wal_int4_gemv
    W, x, y = 0x10000, 0x20000, 0x30000
    assert g(None, 2, 256, x, 1, y, None) == -1
    assert g(W, 2, 200, x, 1, y, None) == -2
    assert g(W + 16, 2, 256, x, 1, y, None) == -6
    assert g(W, 2, 256, x + 2, 1, y, None) == -6
    assert g(W, 2, 256, x, 0, y, None) == -9                # fp32 x
    assert g(W, 2, 256, x, 5, y, None) == -1


def test_int3_pack_matches_oracle_and_rejects():
    """INT3/g128: the C++ packer writes the oracle's bytes and unpacks them
    back; bad codes, inexact scales, shapes and short buffers are rejected
    with nothing written; the row lookup checks its arguments before any
    launch."""
    from oracle import int3 as I
    rng = np.random.default_rng(22)
    for V, inp in [(1, 128), (3, 384), (40, 4224)]:
        q = rng.integers(-4, 4, size=(V, inp)).astype(np.int8)
        s = (rng.integers(-2048, 2048, size=(V, inp // 128)) / 256.0).astype(np.float32)
        b = wal.wal_int3_pack(q, s)
        assert np.array_equal(b, I.pack(q, s.astype(np.float64)))
        q2, s2 = wal.wal_int3_unpack(b, V, inp)
        assert np.array_equal(q2, q) and np.array_equal(s2, s)
    assert wal.wal_int3_size(151936, 4096) == I.size(151936, 4096)
    lib = wal._lib
    buf = np.zeros(I.size(2, 256), np.uint8)
    q = np.zeros((2, 256), np.int8)
    s = np.ones((2, 2), np.float32)
    assert lib.wal_int3_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size - 1) == -5
    assert lib.wal_int3_pack(2, 200, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -2
    q[1, 3] = 4
    assert lib.wal_int3_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -3
    q[1, 3] = -5
    assert lib.wal_int3_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -3
    q[1, 3] = 0
    s[1, 1] = 1e-9
    assert lib.wal_int3_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -4
    assert not buf.any()
    e = lib.wal_embed_rows
    W, ids, out = 0x10000, 0x20000, 0x30000
    assert e(None, 3, 2, 256, ids, 1, out, 0, 256, None) == -1
    assert e(W, 5, 2, 256, ids, 1, out, 0, 256, None) == -1          # bits
    assert e(W, 3, 2, 200, ids, 1, out, 0, 256, None) == -2          # in % 128
    assert e(W, 3, 2, 256, ids, 1, out, 0, 200, None) == -1          # ldo < in
    assert e(W, 3, 2, 256, ids, 0, out, 0, 256, None) == -1          # n = 0
    assert e(W, 3, 2, 256, ids, 1, out, 7, 256, None) == -1          # out dtype
    assert e(W + 16, 4, 2, 256, ids, 1, out, 0, 256, None) == -6
    assert e(W, 4, 2, 256, ids + 2, 1, out, 0, 256, None) == -6
    assert e(W, 4, 2, 256, ids, 1, out + 4, 0, 256, None) == -6
    assert e(W, 4, 2, 256, ids, 1, out, 1, 260, None) == -6          # bf16 rows of 520 B
    assert e(W, 4, 1 << 20, 1 << 13, ids, 1, out, 0, 1 << 13, None) == -2   # 2^32 bytes


def test_int5_pack_matches_oracle_and_rejects():
    """INT5/g128: the C++ packer writes the oracle's bytes and unpacks them
    back; bad codes, inexact scales, shapes and short buffers are rejected
    with nothing written; the product entry checks its arguments first."""
    from oracle import int5 as I
    rng = np.random.default_rng(23)
    for V, inp in [(1, 128), (3, 384), (40, 4224)]:
        q = rng.integers(-16, 16, size=(V, inp)).astype(np.int8)
        s = (rng.integers(-2048, 2048, size=(V, inp // 128)) / 256.0).astype(np.float32)
        b = wal.wal_int5_pack(q, s)
        assert np.array_equal(b, I.pack(q, s.astype(np.float64)))
        q2, s2 = wal.wal_int5_unpack(b, V, inp)
        assert np.array_equal(q2, q) and np.array_equal(s2, s)
    assert wal.wal_int5_size(248320, 5120) == I.size(248320, 5120)
    lib = wal._lib
    buf = np.zeros(I.size(2, 256), np.uint8)
    q = np.zeros((2, 256), np.int8)
    s = np.ones((2, 2), np.float32)
    assert lib.wal_int5_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size - 1) == -5
    assert lib.wal_int5_pack(2, 200, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -2
    for bad in (16, -17):
        q[1, 3] = bad
        assert lib.wal_int5_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -3
    q[1, 3] = 0
    s[0, 1] = 0.1
    assert lib.wal_int5_pack(2, 256, q.ctypes.data, s.ctypes.data, buf.ctypes.data, buf.size) == -4
    assert not buf.any()
    g = lib.wal_int5_gemv
    W, x, y = 0x10000, 0x20000, 0x30000
    assert g(None, 2, 256, x, 1, y, None) == -1
    assert g(W, 2, 200, x, 1, y, None) == -2
    assert g(W, 1 << 20, 1 << 12, x, 1, y, None) == -2       # 2.6 GB: past 2^31 bytes
    assert g(W + 16, 2, 256, x, 1, y, None) == -6
    assert g(W, 2, 256, x + 2, 1, y, None) == -6
    assert g(W, 2, 256, x, 0, y, None) == -9                  # fp32 x
    assert g(W, 2, 256, x, 5, y, None) == -1


def test_embed_rows_mixed_checks():
    """The mixed-table lookup checks its arguments before any launch."""
    e = wal._lib.wal_embed_rows_mixed
    W3, W4, m, ids, out = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
    assert e(None, 3, W4, 1, 256, m, 4, ids, 1, out, 0, 256, None) == -1
    assert e(W3, 0, W4, 1, 256, m, 4, ids, 1, out, 0, 256, None) == -1      # empty INT3 table
    assert e(W3, 3, W4, 1, 200, m, 4, ids, 1, out, 0, 256, None) == -2      # in % 128
    assert e(W3, 3, W4, 1, 256, m, 4, ids, 1, out, 0, 200, None) == -1      # ldo < in
    assert e(W3, 3, W4, 1, 256, m, 4, ids, 1, out, 2, 256, None) == -1      # out dtype
    assert e(W3 + 16, 3, W4, 1, 256, m, 4, ids, 1, out, 0, 256, None) == -6
    assert e(W3, 3, W4 + 16, 1, 256, m, 4, ids, 1, out, 0, 256, None) == -6
    assert e(W3, 3, W4, 1, 256, m + 2, 4, ids, 1, out, 0, 256, None) == -6
    assert e(W3, 3, W4, 1, 256, m, 4, ids, 1, out + 8, 0, 256, None) == -6
    assert e(W3, 3, W4, 1 << 20, 1 << 13, m, 4, ids, 1, out, 0, 1 << 13, None) == -2   # INT4 table of 2^32 bytes


def test_quantised_outputs_must_not_overlap_inputs():
    """The INT4/INT5 products and the row lookups reject an output that
    overlaps an input, before any launch."""
    W, x = 0x100000, 0x200000
    for g in (wal._lib.wal_int4_gemv, wal._lib.wal_int5_gemv):
        assert g(W, 2, 256, x, 1, W + 64, None) == -1          # y inside W
        assert g(W, 2, 256, x, 1, x + 4, None) == -1           # y inside x
    e = wal._lib.wal_embed_rows
    ids = 0x300000
    assert e(W, 4, 2, 256, ids, 4, W + 256, 0, 256, None) == -1   # out inside W
    assert e(W, 4, 2, 256, ids, 4, ids - 16, 0, 256, None) == -1  # out over ids
    em = wal._lib.wal_embed_rows_mixed
    W4, m = 0x400000, 0x500000
    assert em(W, 3, W4, 1, 256, m, 4, ids, 1, m - 256, 0, 256, None) == -1   # out over the map

