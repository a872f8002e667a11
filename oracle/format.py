"""Independent numpy implementation of the WAL packed blob (format version 1).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages fix what is stored but not the bytes: packed ternary symbols,
sparse positions/signs and fp16 scales in the executable cache (WAL-Ternary-8B
card, "Build the approximately 2.3 GB executable cache"); exactly k signed
residual sites per group of 128 weights ("Representation"); 2-bit codes of
which three of the four values are used and a base-3 container of five trits
per byte (WAL2-Ternary-27B card, "Что означает битность"); 24-bit float group
scales decoded to fp32 and up to two binary low-rank paths (WAL-Ternary-27B-RC1
card, "Representation").  The byte layout below is this repository's reading
of those facts; each choice the pages leave open is named where it is made.

Blob = 256-byte header followed by planes, each starting at a multiple of 256:

  header (little-endian):
    0  u32 magic 0x314C4157 ("WAL1")   4  u32 version (1)
    8  u32 out      12 u32 in       16 u32 k        20 u32 n_paths
    24 u32 rank     28 u32 trit_fmt 32 u32 scale_fmt 36 u32 row_stride
    40 u64 total_bytes  48 u64 off_codes  56 u64 off_sites  64 u64 off_alpha
    72 u64 off_beta     80 u64 off_V[4]   112 u64 off_U[4]  144 u64 off_s[4]
    176 u64 checksum    184..255 zero

  planes, in this order: codes, sites (k > 0), alpha, beta (k > 0), then per
  path p: V_p, U_p, s_p.
"""
from __future__ import annotations

import struct
from dataclasses import dataclass
from typing import Optional

import numpy as np

MAGIC = 0x314C4157
VERSION = 1
HEADER_BYTES = 256
ALIGN = 256
GROUP = 128
MAX_PATHS = 4
MAX_RANK = 64
PAD_BASE3 = 0x79  # five zero trits: 1 + 3 + 9 + 27 + 81 = 121

TRIT_2BIT, TRIT_BASE3 = 0, 1
SCALE_FP16, SCALE_FP24 = 0, 1


class FormatError(ValueError):
    """A blob or a set of logical arrays that the format rejects (fail-closed)."""


@dataclass
class Logical:
    out: int
    inp: int
    k: int
    trit_fmt: int
    scale_fmt: int
    T: np.ndarray
    site_pos: np.ndarray
    site_sign: np.ndarray
    alpha: np.ndarray
    beta: Optional[np.ndarray]
    U: np.ndarray
    V: np.ndarray
    s: np.ndarray


def _up(n: int, a: int = ALIGN) -> int:
    return (n + a - 1) // a * a


def row_stride(inp: int, trit_fmt: int) -> int:
    """Bytes per row of the code plane.

    2-bit: four trits per byte, in/4 bytes (in is a multiple of 128).
    base-3: five trits per byte packed continuously along the row (the
    WAL2-Ternary-27B card's byte totals fit continuous packing, not a
    per-group byte count), ceil(in/5) bytes, rounded up to 16 bytes.
    """
    if trit_fmt == TRIT_2BIT:
        return inp // 4
    return _up(-(-inp // 5), 16)


def plane_sizes(out: int, inp: int, k: int, n_paths: int, rank: int,
                trit_fmt: int, scale_fmt: int) -> dict:
    """Unpadded byte size of every plane."""
    G = inp // GROUP
    sb = 2 if scale_fmt == SCALE_FP16 else 3
    sizes = {"codes": out * row_stride(inp, trit_fmt),
             "sites": out * G * k,
             "alpha": out * G * sb,
             "beta": out * G * sb if k else 0}
    for p in range(n_paths):
        sizes[f"V{p}"] = rank * (inp // 8)
        sizes[f"U{p}"] = out * ((rank + 7) // 8)
        sizes[f"s{p}"] = rank * 2
    return sizes


def layout(out: int, inp: int, k: int, n_paths: int, rank: int,
           trit_fmt: int, scale_fmt: int) -> dict:
    """Offsets of every plane and the total blob size."""
    sz = plane_sizes(out, inp, k, n_paths, rank, trit_fmt, scale_fmt)
    off = {}
    cur = HEADER_BYTES
    for name in ["codes", "sites", "alpha", "beta"]:
        if name in ("sites", "beta") and k == 0:
            off[name] = 0
            continue
        off[name] = cur
        cur = _up(cur + sz[name])
    for p in range(n_paths):
        for nm in ("V", "U", "s"):
            off[f"{nm}{p}"] = cur
            cur = _up(cur + sz[f"{nm}{p}"])
    off["total"] = cur
    return off


def algorithmic_bytes(out, inp, k, n_paths, rank, trit_fmt, scale_fmt) -> int:
    """Bytes a product must read from the weights: every plane, without the
    header, alignment padding, or base-3 row padding (ceil(in/5) per row)."""
    sz = plane_sizes(out, inp, k, n_paths, rank, trit_fmt, scale_fmt)
    if trit_fmt == TRIT_BASE3:
        sz["codes"] = out * (-(-inp // 5))
    return int(sum(sz.values()))


def _check_logical(L: Logical):
    if L.inp <= 0 or L.out <= 0 or L.inp % GROUP:
        raise FormatError("shape: in must be a positive multiple of 128")
    if L.k not in (0, 2, 4, 8):
        raise FormatError("k must be 0, 2, 4 or 8")
    if L.trit_fmt not in (0, 1) or L.scale_fmt not in (0, 1):
        raise FormatError("unknown trit or scale format")
    P = L.U.shape[0]
    if P > MAX_PATHS:
        raise FormatError("too many paths")
    if P and not (1 <= L.U.shape[2] <= MAX_RANK):
        raise FormatError("rank out of range")
    if not np.isin(L.T, (-1, 0, 1)).all():
        raise FormatError("trit outside {-1, 0, +1}")
    if L.k:
        if (L.site_pos >= GROUP).any():
            raise FormatError("site position >= 128")
        if L.k > 1 and (np.diff(L.site_pos.astype(np.int16), axis=-1) <= 0).any():
            raise FormatError("site positions must be distinct and ascending")
        if not np.isin(L.site_sign, (-1, 1)).all():
            raise FormatError("site sign outside {-1, +1}")
    if P:
        if not np.isin(L.U, (-1, 1)).all() or not np.isin(L.V, (-1, 1)).all():
            raise FormatError("U/V entry outside {-1, +1}")


def _scale_bytes(v: np.ndarray, scale_fmt: int) -> np.ndarray:
    """fp16: IEEE binary16, little-endian.  fp24: the upper three bytes of
    the little-endian fp32 pattern (sign, 8-bit exponent, 15 mantissa bits),
    the "24-bit float storage format decoded to FP32" of the RC1 card.
    A value that the target format cannot hold exactly is rejected."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    if scale_fmt == SCALE_FP16:
        h = v.astype(np.float16)
        if not np.array_equal(h.astype(np.float32), v, equal_nan=False):
            raise FormatError("scale not exactly representable in fp16")
        return h.view(np.uint8).reshape(-1)
    bits = v.view(np.uint32).reshape(-1)
    if (bits & 0xFF).any():
        raise FormatError("scale not exactly representable in fp24")
    b = bits.view(np.uint8).reshape(-1, 4)
    return np.ascontiguousarray(b[:, 1:4]).reshape(-1)


def _scale_values(raw: np.ndarray, n: int, scale_fmt: int) -> np.ndarray:
    if scale_fmt == SCALE_FP16:
        return raw[: 2 * n].view(np.float16).astype(np.float32)
    b = raw[: 3 * n].reshape(n, 3).astype(np.uint32)
    bits = (b[:, 0] << 8) | (b[:, 1] << 16) | (b[:, 2] << 24)
    return bits.view(np.float32)


def encode_codes_2bit(T: np.ndarray) -> np.ndarray:
    """Four trits per byte, trit j of a row in bits 2(j%4) and 2(j%4)+1 of
    byte j/4.  Code = the two low bits of the trit in two's complement:
    0 -> 00, +1 -> 01, -1 -> 11; 10 is never written (three of the four
    2-bit codes are used, as the WAL2-Ternary-27B card states)."""
    out, inp = T.shape
    c = (T.astype(np.int16) & 3).astype(np.uint8).reshape(out, inp // 4, 4)
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def decode_codes_2bit(codes: np.ndarray, inp: int) -> np.ndarray:
    out = codes.shape[0]
    c = np.stack([(codes >> (2 * i)) & 3 for i in range(4)], axis=-1).reshape(out, inp)
    if (c == 2).any():
        raise FormatError("invalid 2-bit trit code 10")
    return np.where(c == 3, -1, c).astype(np.int8)


def encode_codes_base3(T: np.ndarray) -> np.ndarray:
    """Five trits per byte as a base-3 number, digit d = t + 1, least
    significant digit first: byte m = sum_i d(5m+i) * 3^i.  Digits past the
    row's end are zero trits (d = 1); the row is padded to a multiple of 16
    bytes with 0x79 (five zero trits)."""
    out, inp = T.shape
    nb = -(-inp // 5)
    d = np.ones((out, nb * 5), dtype=np.uint16)
    d[:, :inp] = (T.astype(np.int16) + 1).astype(np.uint16)
    d = d.reshape(out, nb, 5)
    byte = d[..., 0] + 3 * d[..., 1] + 9 * d[..., 2] + 27 * d[..., 3] + 81 * d[..., 4]
    rows = np.full((out, row_stride(inp, TRIT_BASE3)), PAD_BASE3, dtype=np.uint8)
    rows[:, :nb] = byte.astype(np.uint8)
    return rows


def decode_codes_base3(codes: np.ndarray, inp: int) -> np.ndarray:
    out, stride = codes.shape
    nb = -(-inp // 5)
    if (codes >= 243).any():
        raise FormatError("base-3 byte >= 243")
    if (codes[:, nb:] != PAD_BASE3).any():
        raise FormatError("base-3 row padding is not 0x79")
    v = codes[:, :nb].astype(np.int16)
    digits = []
    for _ in range(5):
        digits.append(v % 3)
        v = v // 3
    d = np.stack(digits, axis=-1).reshape(out, nb * 5)
    if (d[:, inp:] != 1).any():
        raise FormatError("base-3 digits past the row end are not zero trits")
    return (d[:, :inp] - 1).astype(np.int8)


def encode_sites(pos: np.ndarray, sign: np.ndarray) -> np.ndarray:
    """One byte per site: position (0..127) in bits 0-6, bit 7 set for a
    negative sign.  Sites of a group are stored in ascending position."""
    return (pos.astype(np.uint8) | np.where(sign < 0, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def decode_sites(b: np.ndarray):
    pos = (b & 0x7F).astype(np.uint8)
    sign = np.where(b & 0x80, -1, 1).astype(np.int8)
    if b.shape[-1] > 1 and (np.diff(pos.astype(np.int16), axis=-1) <= 0).any():
        raise FormatError("site positions must be distinct and ascending")
    return pos, sign


def encode_signs(M: np.ndarray) -> np.ndarray:
    """Bits of a {+1,-1} matrix packed along its last axis, LSB first,
    a set bit meaning -1; unused bits of the last byte are zero."""
    return np.packbits(M < 0, axis=-1, bitorder="little")


def decode_signs(b: np.ndarray, n: int) -> np.ndarray:
    bits = np.unpackbits(b, axis=-1, bitorder="little", count=None)
    if bits.shape[-1] > n and bits[..., n:].any():
        raise FormatError("non-zero padding bit in a sign plane")
    return np.where(bits[..., :n] == 1, -1, 1).astype(np.int8)


def checksum(blob: bytes | np.ndarray) -> int:
    """sum over the little-endian u32 words w_i after the header of
    (i + 1) * w_i, modulo 2^64 (corruption check, not a cryptographic hash)."""
    a = np.frombuffer(blob, dtype=np.uint8)
    words = a[HEADER_BYTES:].view("<u4").astype(np.uint64)
    idx = np.arange(1, words.size + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return int(np.sum(words * idx, dtype=np.uint64))


def pack(L: Logical) -> bytes:
    """Logical arrays -> packed blob (format version 1)."""
    _check_logical(L)
    P = L.U.shape[0]
    r = L.U.shape[2] if P else 0
    if L.k and L.beta is None:
        raise FormatError("beta missing")
    lay = layout(L.out, L.inp, L.k, P, r, L.trit_fmt, L.scale_fmt)
    buf = np.zeros(lay["total"], dtype=np.uint8)

    def put(name, arr):
        a = np.ascontiguousarray(arr, dtype=np.uint8).reshape(-1)
        buf[lay[name]: lay[name] + a.size] = a

    if L.trit_fmt == TRIT_2BIT:
        put("codes", encode_codes_2bit(L.T))
    else:
        put("codes", encode_codes_base3(L.T))
    put("alpha", _scale_bytes(L.alpha, L.scale_fmt))
    if L.k:
        put("sites", encode_sites(L.site_pos, L.site_sign))
        put("beta", _scale_bytes(L.beta, L.scale_fmt))
    for p in range(P):
        put(f"V{p}", encode_signs(np.ascontiguousarray(L.V[p].T)))   # [r][in/8]
        put(f"U{p}", encode_signs(L.U[p]))                            # [out][ceil(r/8)]
        put(f"s{p}", _scale_bytes(L.s[p], SCALE_FP16))
    offs = [lay.get(f"{nm}{p}", 0) for nm in ("V", "U", "s") for p in range(MAX_PATHS)]
    hdr = struct.pack("<10I5Q", MAGIC, VERSION, L.out, L.inp, L.k, P, r, L.trit_fmt,
                      L.scale_fmt, row_stride(L.inp, L.trit_fmt), lay["total"],
                      lay["codes"], lay["sites"], lay["alpha"], lay["beta"])
    hdr += struct.pack("<12Q", *offs)
    buf[: len(hdr)] = np.frombuffer(hdr, dtype=np.uint8)
    cs = checksum(buf)
    buf[176:184] = np.frombuffer(struct.pack("<Q", cs), dtype=np.uint8)
    return buf.tobytes()


def parse_header(blob) -> dict:
    a = bytes(memoryview(blob)[:HEADER_BYTES])
    if len(a) < HEADER_BYTES:
        raise FormatError("blob shorter than the header")
    f = struct.unpack("<10I5Q", a[:80])
    names = ["magic", "version", "out", "in", "k", "n_paths", "rank", "trit_fmt",
             "scale_fmt", "row_stride", "total", "codes", "sites", "alpha", "beta"]
    h = dict(zip(names, f))
    offs = struct.unpack("<12Q", a[80:176])
    for i, nm in enumerate(("V", "U", "s")):
        for p in range(MAX_PATHS):
            h[f"{nm}{p}"] = offs[i * MAX_PATHS + p]
    h["checksum"] = struct.unpack("<Q", a[176:184])[0]
    h["reserved"] = a[184:256]
    return h


def unpack(blob, verify: bool = True) -> Logical:
    """Packed blob -> logical arrays; rejects anything the format forbids."""
    buf = np.frombuffer(bytes(blob), dtype=np.uint8)
    h = parse_header(buf)
    if h["magic"] != MAGIC or h["version"] != VERSION:
        raise FormatError("bad magic or version")
    if any(h["reserved"]):
        raise FormatError("reserved header bytes are not zero")
    out, inp, k, P, r = h["out"], h["in"], h["k"], h["n_paths"], h["rank"]
    tf, sf = h["trit_fmt"], h["scale_fmt"]
    if inp == 0 or out == 0 or inp % GROUP or k not in (0, 2, 4, 8) or tf > 1 or sf > 1:
        raise FormatError("bad shape or format field")
    if P > MAX_PATHS or (P and not 1 <= r <= MAX_RANK) or (not P and r):
        raise FormatError("bad path count or rank")
    if h["row_stride"] != row_stride(inp, tf):
        raise FormatError("row stride does not match the shape")
    lay = layout(out, inp, k, P, r, tf, sf)
    for name in ["codes", "sites", "alpha", "beta"] + [f"{n}{p}" for p in range(MAX_PATHS) for n in "VUs"]:
        if h[name] != lay.get(name, 0):
            raise FormatError(f"plane offset {name} does not match the layout")
    if h["total"] != lay["total"] or buf.size < lay["total"]:
        raise FormatError("blob size does not match the layout")
    if verify and checksum(buf[: lay["total"]]) != h["checksum"]:
        raise FormatError("checksum mismatch")
    sz = plane_sizes(out, inp, k, P, r, tf, sf)
    G = inp // GROUP

    def get(name):
        return buf[lay[name]: lay[name] + sz[name]]

    codes = get("codes").reshape(out, row_stride(inp, tf))
    T = decode_codes_2bit(codes, inp) if tf == TRIT_2BIT else decode_codes_base3(codes, inp)
    alpha = _scale_values(get("alpha"), out * G, sf).reshape(out, G)
    if k:
        pos, sign = decode_sites(get("sites").reshape(out, G, k))
        beta = _scale_values(get("beta"), out * G, sf).reshape(out, G)
    else:
        pos = np.zeros((out, G, 0), np.uint8)
        sign = np.zeros((out, G, 0), np.int8)
        beta = None
    U = np.zeros((P, out, r), np.int8)
    V = np.zeros((P, inp, r), np.int8)
    s = np.zeros((P, r), np.float32)
    for p in range(P):
        V[p] = decode_signs(get(f"V{p}").reshape(r, inp // 8), inp).T
        U[p] = decode_signs(get(f"U{p}").reshape(out, (r + 7) // 8), r)
        s[p] = _scale_values(get(f"s{p}"), r, SCALE_FP16)
    return Logical(out, inp, k, tf, sf, T, pos, sign, alpha, beta, U, V, s)


def from_synth(m) -> Logical:
    """Adopt a ``synth.Matrix`` (same fields) as oracle logical arrays."""
    return Logical(m.out, m.inp, m.k, m.trit_fmt, m.scale_fmt, m.T, m.site_pos, m.site_sign,
                   m.alpha, m.beta, m.U, m.V, m.s)


def unpack_rows(blob, rows) -> Logical:
    """Logical arrays of the selected rows only (out = len(rows)); V and s
    are whole.  Each output y_n depends on row n alone, so the oracle can
    check sampled outputs of matrices too large to decode in full."""
    buf = np.frombuffer(bytes(blob) if not isinstance(blob, np.ndarray) else blob, dtype=np.uint8)
    h = parse_header(buf)
    if h["magic"] != MAGIC or h["version"] != VERSION:
        raise FormatError("bad magic or version")
    out, inp, k, P, r = h["out"], h["in"], h["k"], h["n_paths"], h["rank"]
    tf, sf = h["trit_fmt"], h["scale_fmt"]
    rows = np.asarray(rows, dtype=np.int64)
    if rows.size == 0 or rows.min() < 0 or rows.max() >= out:
        raise FormatError("row index out of range")
    lay = layout(out, inp, k, P, r, tf, sf)
    G = inp // GROUP
    sb = 2 if sf == SCALE_FP16 else 3
    stride = row_stride(inp, tf)
    codes = buf[lay["codes"]: lay["codes"] + out * stride].reshape(out, stride)[rows]
    T = decode_codes_2bit(codes, inp) if tf == TRIT_2BIT else decode_codes_base3(codes, inp)
    araw = buf[lay["alpha"]: lay["alpha"] + out * G * sb].reshape(out, G * sb)[rows].reshape(-1)
    alpha = _scale_values(araw, rows.size * G, sf).reshape(rows.size, G)
    if k:
        sraw = buf[lay["sites"]: lay["sites"] + out * G * k].reshape(out, G, k)[rows]
        pos, sign = decode_sites(sraw)
        braw = buf[lay["beta"]: lay["beta"] + out * G * sb].reshape(out, G * sb)[rows].reshape(-1)
        beta = _scale_values(braw, rows.size * G, sf).reshape(rows.size, G)
    else:
        pos = np.zeros((rows.size, G, 0), np.uint8)
        sign = np.zeros((rows.size, G, 0), np.int8)
        beta = None
    ub = (r + 7) // 8
    U = np.zeros((P, rows.size, r), np.int8)
    V = np.zeros((P, inp, r), np.int8)
    s = np.zeros((P, r), np.float32)
    for p in range(P):
        V[p] = decode_signs(buf[lay[f"V{p}"]: lay[f"V{p}"] + r * (inp // 8)].reshape(r, inp // 8), inp).T
        U[p] = decode_signs(buf[lay[f"U{p}"]: lay[f"U{p}"] + out * ub].reshape(out, ub)[rows], r)
        s[p] = _scale_values(buf[lay[f"s{p}"]: lay[f"s{p}"] + 2 * r], r, SCALE_FP16)
    return Logical(rows.size, inp, k, tf, sf, T, pos, sign, alpha, beta, U, V, s)
