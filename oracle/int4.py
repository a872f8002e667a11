"""INT4/g128 packed matrices (the LM head of the WAL-Ternary-8B cards), float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The 8B cards list the LM head as "INT4/g128" and say nothing more.  Read
plainly: every weight is a signed 4-bit integer q in [-8, 7] and every group
of 128 consecutive weights of a row shares one scale s, so W[v][j] =
s[v][j // 128] * q[v][j]; symmetric, with no zero point.  This repository
stores such a matrix [V][in] (in a multiple of 128) as

    codes  [V][in / 2] bytes: element 2i in the low nibble of byte i, 2i + 1
           in the high nibble, each nibble the two's-complement code of q
    scales [V][in / 128] IEEE binary16, little-endian

with the codes plane first and the scales plane right after it.  A scale
that binary16 cannot hold exactly is rejected (nothing is rounded).
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def size(V: int, inp: int) -> int:
    """Bytes of a packed [V][inp] matrix."""
    if V <= 0 or inp <= 0 or inp % GROUP:
        raise ValueError("V > 0 and in a positive multiple of 128")
    return V * inp // 2 + V * (inp // GROUP) * 2


def pack(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Codes q int [V][in] in [-8, 7] and scales s [V][in/128] -> uint8 bytes."""
    q = np.asarray(q)
    V, inp = q.shape
    nbytes = size(V, inp)
    if q.min() < -8 or q.max() > 7:
        raise ValueError("codes must lie in [-8, 7]")
    s = np.asarray(s, dtype=np.float64)
    if s.shape != (V, inp // GROUP):
        raise ValueError("scales must be [V][in / 128]")
    s16 = s.astype(np.float16)
    if not np.array_equal(s16.astype(np.float64), s):
        raise ValueError("a scale is not exactly representable in binary16")
    nib = (q.astype(np.int64) & 0xF).astype(np.uint8)          # two's-complement nibbles
    codes = nib[:, 0::2] | (nib[:, 1::2] << 4)
    out = np.empty(nbytes, dtype=np.uint8)
    out[:V * inp // 2] = codes.reshape(-1)
    out[V * inp // 2:] = s16.astype("<f2").view(np.uint8).reshape(-1)
    return out


def unpack(blob: np.ndarray, V: int, inp: int):
    """uint8 bytes -> (q int8 [V][in], s float64 [V][in/128])."""
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.size < size(V, inp):
        raise ValueError("buffer too small")
    codes = blob[:V * inp // 2].reshape(V, inp // 2)
    lo = (codes & 0xF).astype(np.int8)
    hi = (codes >> 4).astype(np.int8)
    q = np.empty((V, inp), dtype=np.int8)
    q[:, 0::2] = np.where(lo >= 8, lo - 16, lo)
    q[:, 1::2] = np.where(hi >= 8, hi - 16, hi)
    sb = blob[V * inp // 2:size(V, inp)]
    s = sb.view("<f2").astype(np.float64).reshape(V, inp // GROUP)
    return q, s


def dense_W(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W = s (.)_g q, float64 [V][in]."""
    return np.repeat(np.asarray(s, dtype=np.float64), GROUP, axis=1) * np.asarray(q, dtype=np.float64)


def gemv(blob: np.ndarray, V: int, inp: int, x: np.ndarray) -> np.ndarray:
    """y = W x in float64 (W built densely from the packed bytes)."""
    q, s = unpack(blob, V, inp)
    return dense_W(q, s) @ np.asarray(x, dtype=np.float64)


def gemv_rows(blob: np.ndarray, V: int, inp: int, x: np.ndarray, rows) -> np.ndarray:
    """y[rows] only, for tall matrices (the LM head) checked on sampled rows."""
    blob = np.asarray(blob, dtype=np.uint8)
    rows = np.asarray(rows)
    codes = blob[:V * inp // 2].reshape(V, inp // 2)[rows]
    sc = blob[V * inp // 2:size(V, inp)].view("<f2").reshape(V, inp // GROUP)[rows]
    sub = np.concatenate([codes.reshape(-1), sc.astype("<f2").view(np.uint8).reshape(-1)])
    return gemv(sub, len(rows), inp, x)


def rows(blob: np.ndarray, V: int, inp: int, ids) -> np.ndarray:
    """Rows W[ids] (float64), the lookup of an INT4 embedding; ids outside
    [0, V) give zero rows.  Only the requested rows are decoded."""
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.size < size(V, inp):
        raise ValueError("buffer too small")
    ids = np.asarray(ids, dtype=np.int64)
    out = np.zeros((len(ids), inp))
    ok = (ids >= 0) & (ids < V)
    if ok.any():
        sel = ids[ok]
        codes = blob[:V * inp // 2].reshape(V, inp // 2)[sel]
        sc = blob[V * inp // 2:size(V, inp)].reshape(V, inp // GROUP * 2)[sel]
        q, s = unpack(np.concatenate([codes.reshape(-1), sc.reshape(-1)]), len(sel), inp)
        out[ok] = dense_W(q, s)
    return out

