"""INT3/g128 packed matrices and embedding rows (the 8B cards' embedding),
float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The WAL-Ternary-8B cards list the embedding as "INT3/g128" and say nothing
more.  Read plainly: every weight is a signed 3-bit integer q in [-4, 3]
and every group of 128 consecutive weights of a row shares one scale s, so
E[v][j] = s[v][j // 128] * q[v][j].  This repository stores such a matrix
[V][in] (in a multiple of 128) as

    codes  [V][in * 3 / 8] bytes: row v's codes as one bit stream, element j
           at stream bits 3 j .. 3 j + 2 (the stream's bit b is bit b % 8 of
           byte b // 8), each code in two's complement
    scales [V][in / 128] IEEE binary16, little-endian, after all the codes

An embedding lookup returns whole rows: rows(ids) = E[ids].
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def size(V: int, inp: int) -> int:
    if V <= 0 or inp <= 0 or inp % GROUP:
        raise ValueError("V > 0 and in a positive multiple of 128")
    return V * inp * 3 // 8 + V * (inp // GROUP) * 2


def pack(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Codes q int [V][in] in [-4, 3] and scales s [V][in/128] -> uint8 bytes."""
    q = np.asarray(q)
    V, inp = q.shape
    nbytes = size(V, inp)
    if q.min() < -4 or q.max() > 3:
        raise ValueError("codes must lie in [-4, 3]")
    s = np.asarray(s, dtype=np.float64)
    if s.shape != (V, inp // GROUP):
        raise ValueError("scales must be [V][in / 128]")
    s16 = s.astype(np.float16)
    if not np.array_equal(s16.astype(np.float64), s):
        raise ValueError("a scale is not exactly representable in binary16")
    code = (q.astype(np.int64) & 7)                                   # two's-complement 3-bit codes
    bits = ((code[:, :, None] >> np.arange(3)) & 1).reshape(V, inp * 3)  # element j -> stream bits 3j..3j+2
    packed = np.packbits(bits.astype(np.uint8), axis=1, bitorder="little")
    out = np.empty(nbytes, dtype=np.uint8)
    out[:V * inp * 3 // 8] = packed.reshape(-1)
    out[V * inp * 3 // 8:] = s16.astype("<f2").view(np.uint8).reshape(-1)
    return out


def unpack(blob: np.ndarray, V: int, inp: int):
    """uint8 bytes -> (q int8 [V][in], s float64 [V][in/128])."""
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.size < size(V, inp):
        raise ValueError("buffer too small")
    cb = V * inp * 3 // 8
    bits = np.unpackbits(blob[:cb].reshape(V, inp * 3 // 8), axis=1, bitorder="little").reshape(V, inp, 3)
    code = (bits.astype(np.int64) << np.arange(3)).sum(axis=2)
    q = np.where(code >= 4, code - 8, code).astype(np.int8)
    s = blob[cb:size(V, inp)].view("<f2").astype(np.float64).reshape(V, inp // GROUP)
    return q, s


def dense(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """E = s (.)_g q, float64 [V][in]."""
    return np.repeat(np.asarray(s, dtype=np.float64), GROUP, axis=1) * np.asarray(q, dtype=np.float64)


def rows(blob: np.ndarray, V: int, inp: int, ids) -> np.ndarray:
    """Embedding rows E[ids] (float64); ids outside [0, V) give zero rows.
    Only the requested rows are decoded: row v's codes are bytes
    v * in * 3 / 8 .. (v + 1) * in * 3 / 8 of the codes plane and its scales
    the v-th run of in / 128 binary16 values of the scales plane."""
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.size < size(V, inp):
        raise ValueError("buffer too small")
    ids = np.asarray(ids, dtype=np.int64)
    out = np.zeros((len(ids), inp))
    ok = (ids >= 0) & (ids < V)
    if ok.any():
        sel = ids[ok]
        cb = V * inp * 3 // 8
        codes = blob[:cb].reshape(V, inp * 3 // 8)[sel]
        sc = blob[cb:size(V, inp)].reshape(V, inp // GROUP * 2)[sel]
        q, s = unpack(np.concatenate([codes.reshape(-1), sc.reshape(-1)]), len(sel), inp)
        out[ok] = dense(q, s)
    return out


def rows_mixed(blob3: np.ndarray, V3: int, blob4: np.ndarray, V4: int, inp: int, row_map, ids) -> np.ndarray:
    """Embedding rows of a table whose rows are stored either INT3/g128 or
    INT4/g128 (the WAL-Ternary-27B-RC1 card: most rows INT3, a selected
    quarter INT4).  Read here as two packed tables, [V3][in] INT3 and [V4][in]
    INT4, and a row map [V]: vocabulary row v is row m = row_map[v] of the INT3
    table when m >= 0, else row -1 - m of the INT4 table.  An id outside
    [0, V), or a map entry outside its table, gives a row of zeros."""
    from . import int4
    row_map = np.asarray(row_map, dtype=np.int64)
    ids = np.asarray(ids, dtype=np.int64)
    V = len(row_map)
    out = np.zeros((len(ids), inp))
    for n, v in enumerate(ids):
        if not 0 <= v < V:
            continue
        m = int(row_map[v])
        if m >= 0:
            if m < V3:
                out[n] = rows(blob3, V3, inp, [m])[0]
        elif -1 - m < V4:
            out[n] = int4.rows(blob4, V4, inp, [-1 - m])[0]
    return out
