"""Dense float64 evaluation of the ternary-hybrid operator.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The operator is the one printed on the WAL-Ternary-8B cards (Kazakh card,
"Модель пішімі"; English card, "Representation"):

    W(x) = (alpha * T + beta * R) x + sum_r U_r (V_r^T x)

read with these choices where the pages are silent:

* alpha and beta are per row and per group of 128 consecutive columns (the
  WAL2-Ternary-27B card gives the scale group as 128, "Архитектура");
* R holds exactly k signed sites per (row, group) ("exactly 8 signed
  residual sites per group of 128 weights"; k0/k2/k4/k8 on the RC1 card);
* each binary path p carries a per-rank scale s_p, so a path adds
  U_p diag(s_p) V_p^T; several paths add (the RC1 card's "two packed binary
  low-rank residual paths").

The product is formed the plain way: build W in float64, then multiply.
"""
from __future__ import annotations

import numpy as np

from .format import GROUP, Logical, unpack


def dense_W(L: Logical) -> np.ndarray:
    """W = alpha (.)_g T + beta (.)_g R + sum_p U_p diag(s_p) V_p^T, float64 [out][in]."""
    out, inp = L.out, L.inp
    a = np.repeat(L.alpha.astype(np.float64), GROUP, axis=1)      # alpha over its 128 columns
    W = a * L.T.astype(np.float64)
    if L.k:
        G = inp // GROUP
        rows = np.repeat(np.arange(out), G * L.k)
        cols = (np.arange(G)[None, :, None] * GROUP + L.site_pos.astype(np.int64)).reshape(-1)
        vals = (L.beta.astype(np.float64)[:, :, None] * L.site_sign.astype(np.float64)).reshape(-1)
        np.add.at(W, (rows, cols), vals)                            # beta * R at the sites
    for p in range(L.U.shape[0]):
        Us = L.U[p].astype(np.float64) * L.s[p].astype(np.float64)[None, :]
        W += Us @ L.V[p].astype(np.float64).T                       # U_p diag(s_p) V_p^T
    return W


def gemv(blob, x) -> np.ndarray:
    """y = W x for one packed blob; x holds the exact activation values."""
    W = dense_W(unpack(blob))
    return W @ np.asarray(x, dtype=np.float64)


def gemm(blob, X) -> np.ndarray:
    """Y = X W^T for a batch X [B][in] (F.linear convention); returns [B][out]."""
    W = dense_W(unpack(blob))
    return np.asarray(X, dtype=np.float64) @ W.T


def rel_l2(y, y_ref) -> float:
    """||y - y_ref||_2 / ||y_ref||_2 (0 when both are zero)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.linalg.norm(y_ref)
    num = np.linalg.norm(y - y_ref)
    if den == 0:
        return 0.0 if num == 0 else float("inf")
    return float(num / den)


def gemv_rows(blob, x, rows) -> np.ndarray:
    """y[rows] = W[rows, :] x, decoding only the selected rows."""
    from .format import unpack_rows
    W = dense_W(unpack_rows(blob, rows))
    return W @ np.asarray(x, dtype=np.float64)
