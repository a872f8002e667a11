"""Normalised Hadamard-128 rotation of the activations, float64.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The WAL2-Ternary-27B card ("Архитектура") states the rotation of its packed
weights as a normalised H128 with sign_mode identity.  Read plainly: the
stored matrix is W' = W R with R = blockdiag(H/sqrt(128), ...), one block per
group of 128 input columns, H the 128 x 128 Hadamard matrix of Sylvester's
construction, and no sign flips.  R is symmetric and orthogonal, so
W x = W' (R x): a product of the rotated blob takes x~ = R x, and the weight
side is unchanged.

The matrix is built by the doubling H_1 = [1], H_2n = [[H_n, H_n],
[H_n, -H_n]] and applied with a matrix product, block by block.
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def sylvester(n: int = BLOCK) -> np.ndarray:
    """The n x n Hadamard matrix of Sylvester's doubling, int64 entries +-1."""
    H = np.ones((1, 1), dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    if H.shape[0] != n:
        raise ValueError("n must be a power of two")
    return H


def rotate(x: np.ndarray) -> np.ndarray:
    """x~ = blockdiag(H/sqrt(128)) x along the last axis (float64)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError("the length must be a multiple of 128")
    H = sylvester().astype(np.float64)
    blocks = x.reshape(x.shape[:-1] + (n // BLOCK, BLOCK))
    return (blocks @ H.T / np.sqrt(BLOCK)).reshape(x.shape)
