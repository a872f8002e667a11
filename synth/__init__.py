"""Seeded synthetic inputs for the packed ternary-hybrid matrix-vector product.

This module only *draws* inputs.  It produces the logical arrays of one
weight matrix (ternary base T, sparse residual sites, group scales alpha and
beta, binary low-rank factors U, V with per-rank scales s) and activation
vectors x.  It holds none of the method's arithmetic: no packing, no decoding
and no product.  Both the CPU oracle and the GPU path take their inputs from
here, so the two sides see identical values and share nothing else.

Distributions restate the five workload configurations of this repository
(matrix shapes of the Qwen3-8B body and of the 27B variant, as named on the
WAL-Ternary-8B and WAL2-Ternary-27B model pages):

* T iid with P(0) = 0.3, P(+1) = P(-1) = 0.35.
* Per 128-weight group: alpha ~ U[0.01, 0.03]; k distinct uniform site
  positions in [0, 128) with uniform signs; beta ~ U[0.005, 0.015].
* Low-rank paths: U, V uniform in {+1, -1}; s ~ U[1e-4, 1e-3].
* x ~ N(0, 1), rounded to bf16 (round to nearest even) or kept in fp32.

Scale values are drawn so that they are exactly representable in the storage
format that the configuration names: fp16 scales are rounded to nearest
(numpy's float16 cast), 24-bit scales keep the top 24 bits of the fp32
pattern (the low 8 mantissa bits are dropped, i.e. truncated).

Seeds: numpy PCG64 from ``SeedSequence([0, config_id, matrix_id])``.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

GROUP = 128

TRIT_2BIT = 0
TRIT_BASE3 = 1
SCALE_FP16 = 0
SCALE_FP24 = 1


@dataclasses.dataclass
class Matrix:
    """Logical arrays of one weight matrix (no packing applied)."""

    out: int
    inp: int
    k: int
    trit_fmt: int
    scale_fmt: int
    T: np.ndarray            # int8 [out][in], values in {-1, 0, +1}
    site_pos: np.ndarray     # uint8 [out][G][k], strictly ascending per group
    site_sign: np.ndarray    # int8 [out][G][k], values in {-1, +1}
    alpha: np.ndarray        # float32 [out][G]
    beta: Optional[np.ndarray]   # float32 [out][G], None iff k == 0
    U: np.ndarray            # int8 [P][out][r], values in {-1, +1}
    V: np.ndarray            # int8 [P][in][r], values in {-1, +1}
    s: np.ndarray            # float32 [P][r]

    @property
    def groups(self) -> int:
        return self.inp // GROUP

    @property
    def n_paths(self) -> int:
        return int(self.U.shape[0])

    @property
    def rank(self) -> int:
        return int(self.U.shape[2]) if self.U.shape[0] else 0


def rng_for(config_id: int, matrix_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, int(config_id), int(matrix_id)]))


def round_fp16(v: np.ndarray) -> np.ndarray:
    """Nearest fp16 value of each entry, returned as float32."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float32)


def truncate_fp24(v: np.ndarray) -> np.ndarray:
    """fp32 value with its low 8 mantissa bits cleared, as float32."""
    bits = np.asarray(v, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFFFF00)
    return bits.view(np.float32)


def round_bf16_bits(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) nearest to the fp32 values, ties to even."""
    b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _draw_trits(rng: np.random.Generator, shape) -> np.ndarray:
    # u ~ U[0, 1) in float32: [0, 0.3) -> 0, [0.3, 0.65) -> +1, [0.65, 1) -> -1
    u = rng.random(size=shape, dtype=np.float32)
    t = (u >= np.float32(0.3)).astype(np.int8)
    t -= 2 * (u >= np.float32(0.65)).astype(np.int8)
    return t


def _draw_sites(rng: np.random.Generator, rows: int, groups: int, k: int):
    """k distinct uniform positions in [0, 128) per (row, group), ascending."""
    n = rows * groups
    if k == 0:
        return (np.zeros((rows, groups, 0), np.uint8), np.zeros((rows, groups, 0), np.int8))
    pos = np.sort(rng.integers(0, GROUP, size=(n, k), dtype=np.int16), axis=1)
    bad = np.nonzero((np.diff(pos, axis=1) == 0).any(axis=1))[0]
    while bad.size:
        redraw = np.sort(rng.integers(0, GROUP, size=(bad.size, k), dtype=np.int16), axis=1)
        pos[bad] = redraw
        still = (np.diff(redraw, axis=1) == 0).any(axis=1)
        bad = bad[still]
    sign = np.where(rng.integers(0, 2, size=(n, k), dtype=np.uint8) == 1, 1, -1).astype(np.int8)
    return pos.astype(np.uint8).reshape(rows, groups, k), sign.reshape(rows, groups, k)


def _draw_scale(rng, shape, lo, hi, scale_fmt):
    v = rng.uniform(lo, hi, size=shape)
    if scale_fmt == SCALE_FP16:
        return round_fp16(v)
    return truncate_fp24(v.astype(np.float32))


def make_matrix(config_id: int, matrix_id: int, out: int, inp: int, *, k: int = 8,
                n_paths: int = 0, rank: int = 16, trit_fmt: int = TRIT_2BIT,
                scale_fmt: int = SCALE_FP16, zero_T: bool = False) -> Matrix:
    """Draw the logical arrays of one matrix with the configurations' distributions."""
    if inp % GROUP:
        raise ValueError("in must be a multiple of 128")
    rng = rng_for(config_id, matrix_id)
    G = inp // GROUP
    T = _draw_trits(rng, (out, inp))
    if zero_T:
        T[:] = 0
    alpha = _draw_scale(rng, (out, G), 0.01, 0.03, scale_fmt)
    pos, sign = _draw_sites(rng, out, G, k)
    beta = _draw_scale(rng, (out, G), 0.005, 0.015, scale_fmt) if k else None
    r = rank if n_paths else 0
    U = np.where(rng.integers(0, 2, size=(n_paths, out, r), dtype=np.uint8) == 1, 1, -1).astype(np.int8)
    V = np.where(rng.integers(0, 2, size=(n_paths, inp, r), dtype=np.uint8) == 1, 1, -1).astype(np.int8)
    s = round_fp16(rng.uniform(1e-4, 1e-3, size=(n_paths, r)))
    return Matrix(out, inp, k, trit_fmt, scale_fmt, T, pos, sign, alpha, beta, U, V, s)


def make_x(config_id: int, matrix_id: int, inp: int, batch: int = 1, *, bf16: bool = True):
    """Activations x ~ N(0, 1) of shape [batch][in].

    Returns ``(x_f32, x_bits)``: the exact values as float32 and, for bf16,
    the uint16 bit patterns (``None`` for fp32 activations).
    """
    rng = np.random.default_rng(np.random.SeedSequence([0, int(config_id), int(matrix_id), 7]))
    v = rng.standard_normal(size=(batch, inp)).astype(np.float32)
    if not bf16:
        return v, None
    bits = round_bf16_bits(v)
    return bf16_bits_to_f32(bits), bits


# ---------------------------------------------------------------------------
# Workload configurations (shapes and draws); the oracle and the GPU path both
# read these.

QWEN3_8B_LAYER = (  # (name, out, in) of one decoder layer's body matrices
    ("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096), ("o", 4096, 4096),
    ("gate", 12288, 4096), ("up", 12288, 4096), ("down", 4096, 12288),
)
QWEN3_8B_LAYERS = 36


def sweep_shapes():
    """The 252 (out, in) shapes of the 36-layer Qwen3-8B-shaped body, in order."""
    return [(o, i) for _ in range(QWEN3_8B_LAYERS) for (_, o, i) in QWEN3_8B_LAYER]


def sweep_lowrank_mask(n: int = 252, chosen: int = 213) -> np.ndarray:
    """Which of the 252 sweep matrices carry the rank-16 path (213 of them)."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 2, 9999]))
    mask = np.zeros(n, dtype=bool)
    mask[rng.choice(n, chosen, replace=False)] = True
    return mask


def config_matrix(config_id: int, matrix_id: int = 0) -> Matrix:
    """Matrix ``matrix_id`` of workload configuration ``config_id``."""
    if config_id == 0:
        return make_matrix(0, 0, 256, 512, k=8, n_paths=0)
    if config_id == 1:
        return make_matrix(1, 0, 12288, 4096, k=8, n_paths=1, rank=16)
    if config_id == 2:
        out, inp = sweep_shapes()[matrix_id]
        paths = 1 if sweep_lowrank_mask()[matrix_id] else 0
        return make_matrix(2, matrix_id, out, inp, k=8, n_paths=paths, rank=16)
    if config_id == 3:
        return make_matrix(3, 0, 4096, 12288, k=8, n_paths=1, rank=16)
    if config_id == 4:
        shape = [(17408, 5120), (5120, 17408)][matrix_id]
        k = config4_k(matrix_id)
        return make_matrix(4, matrix_id, shape[0], shape[1], k=k, n_paths=2, rank=16,
                           trit_fmt=TRIT_BASE3, scale_fmt=SCALE_FP24)
    if config_id == BASE3_BODY:
        out, inp = base3_body_shape(matrix_id)
        return make_matrix(BASE3_BODY, matrix_id, out, inp, k=config4_k(matrix_id), n_paths=2, rank=16,
                           trit_fmt=TRIT_BASE3, scale_fmt=SCALE_FP24)
    raise ValueError(config_id)


# A bandwidth-scale base-3 workload: a 27B-shaped body of matrices that
# alternate between the two shapes of configuration 4, each with configuration
# 4's per-matrix draw of k (uniform over {0, 2, 4, 8}), fp24 scales and two
# rank-16 paths.  BASE3_BODY_MATRICES of them hold about 2.1 GB packed.
BASE3_BODY = 40
BASE3_BODY_MATRICES = 88


def base3_body_shape(matrix_id: int):
    return [(17408, 5120), (5120, 17408)][matrix_id % 2]


def config4_k(matrix_id: int) -> int:
    """Per-matrix sparse count of the 27B-shaped configuration, uniform over {0,2,4,8}."""
    rng = np.random.default_rng(np.random.SeedSequence([0, 4, 5000 + int(matrix_id)]))
    return int((0, 2, 4, 8)[rng.integers(0, 4)])


def config_x(config_id: int, matrix_id: int = 0, batch: int = 1):
    """Activation(s) of a configuration: fp32 for configuration 0, bf16 otherwise."""
    if config_id == 0:
        return make_x(0, 0, 512, 1, bf16=False)
    if config_id == 1:
        return make_x(1, 0, 4096, batch)
    if config_id == 2:
        return make_x(2, matrix_id, sweep_shapes()[matrix_id][1], batch)
    if config_id == 3:
        x, bits = make_x(3, 0, 12288, 32)
        return x[:batch], bits[:batch]
    if config_id == 4:
        return make_x(4, matrix_id, [5120, 17408][matrix_id], batch)
    if config_id == BASE3_BODY:
        return make_x(BASE3_BODY, matrix_id, base3_body_shape(matrix_id)[1], batch)
    raise ValueError(config_id)
