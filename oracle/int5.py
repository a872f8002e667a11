"""INT5/g128 packed matrices (the LM head of the WAL-Ternary-27B-RC1 card),
float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The RC1 card lists its LM head as "packed INT5" and gives nothing more.  Read
plainly, and in line with the other cards' symmetric INT4/g128 head: every
weight is a signed 5-bit integer q in [-16, 15], every group of 128
consecutive weights of a row shares one scale s, and W[v][j] =
s[v][j // 128] * q[v][j].  "Packed" is read as five bits per weight with no
padding.  This repository stores such a matrix [V][in] (in a multiple of
128) as

    codes  [V][in * 5 / 8] bytes: row v's codes as one bit stream, element j
           at stream bits 5 j .. 5 j + 4 (the stream's bit b is bit b % 8 of
           byte b // 8), each code in two's complement
    scales [V][in / 128] IEEE binary16, little-endian, after all the codes

A scale that binary16 cannot hold exactly is rejected (nothing is rounded).
"""
from __future__ import annotations

import numpy as np

GROUP = 128
BITS = 5


def size(V: int, inp: int) -> int:
    """Bytes of a packed [V][inp] matrix."""
    if V <= 0 or inp <= 0 or inp % GROUP:
        raise ValueError("V > 0 and in a positive multiple of 128")
    return V * inp * BITS // 8 + V * (inp // GROUP) * 2


def pack(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Codes q int [V][in] in [-16, 15] and scales s [V][in/128] -> uint8 bytes."""
    q = np.asarray(q)
    V, inp = q.shape
    nbytes = size(V, inp)
    if q.min() < -16 or q.max() > 15:
        raise ValueError("codes must lie in [-16, 15]")
    s = np.asarray(s, dtype=np.float64)
    if s.shape != (V, inp // GROUP):
        raise ValueError("scales must be [V][in / 128]")
    s16 = s.astype(np.float16)
    if not np.array_equal(s16.astype(np.float64), s):
        raise ValueError("a scale is not exactly representable in binary16")
    code = q.astype(np.int64) & 31                                        # two's-complement 5-bit codes
    bits = ((code[:, :, None] >> np.arange(BITS)) & 1).reshape(V, inp * BITS)   # element j -> bits 5j..5j+4
    cb = V * inp * BITS // 8
    out = np.empty(nbytes, dtype=np.uint8)
    out[:cb] = np.packbits(bits.astype(np.uint8), axis=1, bitorder="little").reshape(-1)
    out[cb:] = s16.astype("<f2").view(np.uint8).reshape(-1)
    return out


def unpack(blob: np.ndarray, V: int, inp: int):
    """uint8 bytes -> (q int8 [V][in], s float64 [V][in/128])."""
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.size < size(V, inp):
        raise ValueError("buffer too small")
    cb = V * inp * BITS // 8
    bits = np.unpackbits(blob[:cb].reshape(V, inp * BITS // 8), axis=1, bitorder="little").reshape(V, inp, BITS)
    code = (bits.astype(np.int64) << np.arange(BITS)).sum(axis=2)
    q = np.where(code >= 16, code - 32, code).astype(np.int8)
    s = blob[cb:size(V, inp)].view("<f2").astype(np.float64).reshape(V, inp // GROUP)
    return q, s


def dense_W(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W = s (.)_g q, float64 [V][in]."""
    return np.repeat(np.asarray(s, dtype=np.float64), GROUP, axis=1) * np.asarray(q, dtype=np.float64)


def gemv(blob: np.ndarray, V: int, inp: int, x: np.ndarray) -> np.ndarray:
    """y = W x in float64 (W built densely from the packed bytes)."""
    q, s = unpack(blob, V, inp)
    return dense_W(q, s) @ np.asarray(x, dtype=np.float64)


def gemv_rows(blob: np.ndarray, V: int, inp: int, x: np.ndarray, rows) -> np.ndarray:
    """y[rows] only, for tall matrices (the LM head) checked on sampled rows:
    row v's codes are bytes v * in * 5 / 8 .. (v + 1) * in * 5 / 8 of the
    codes plane, its scales the v-th run of in / 128 values of the scales
    plane."""
    blob = np.asarray(blob, dtype=np.uint8)
    if blob.size < size(V, inp):
        raise ValueError("buffer too small")
    rows = np.asarray(rows, dtype=np.int64)
    cb = V * inp * BITS // 8
    codes = blob[:cb].reshape(V, inp * BITS // 8)[rows]
    sc = blob[cb:size(V, inp)].reshape(V, inp // GROUP * 2)[rows]
    return gemv(np.concatenate([codes.reshape(-1), sc.reshape(-1)]), len(rows), inp, x)
