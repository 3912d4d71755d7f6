"""Oracle for the hashed n-gram tables: hash, gather-add and the inlined sparse optimizer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the decoder-rtx posts by Chris McCormick (baseline-4 thread): two bigram hash tables
("2M rows, added to x0", "1M rows, added to values"), a frozen trigram table, and an optimizer
for them that is "sparse, no first moment, and only per-row magnitude", inlined in backward so
that no .grad buffer exists.  The pages give no hash or update formula; the tables workload
fixes them:

* h2 = (prev * 1000003 + cur) mod R,  h3 = ((pp * 1000003 + p) * 1000003 + cur) mod R, in exact
  integer arithmetic; a position with no previous token uses prev = V (one past the largest id),
  each sequence on its own;
* per touched row r, with g_r the sum of the per-token gradients that hashed to r:
  v_r <- beta2 * v_r + (1 - beta2) * mean(g_r^2);  w_r <- w_r - lr * g_r / (sqrt(v_r) + eps),
  using the new v_r (beta2 = 0.95, eps = 1e-8).  Rows that no token hit keep w and v.
"""
from __future__ import annotations

import numpy as np

MULT = 1000003


def hash_indices(tokens: np.ndarray, order: int, vocab: int, rows: int) -> np.ndarray:
    """tokens [B, T] -> h [B, T] int64.  Exact integer math (Python ints, object dtype)."""
    tok = np.asarray(tokens, dtype=np.int64)
    B, T = tok.shape
    pad = np.full((B, order - 1), vocab, dtype=np.int64)
    ext = np.concatenate([pad, tok], axis=1).astype(object)
    acc = ext[:, 0:T]
    for j in range(1, order):
        acc = acc * MULT + ext[:, j:j + T]
    return (acc % rows).astype(np.int64)


def gather_add(y: np.ndarray, table: np.ndarray, h: np.ndarray) -> np.ndarray:
    """y[t, :] + table[h[t], :] in float64 (rounding to the storage type is the caller's)."""
    return np.asarray(y, np.float64) + np.asarray(table, np.float64)[np.asarray(h).reshape(-1)]


def sparse_row_update(table: np.ndarray, v: np.ndarray, h: np.ndarray, dy: np.ndarray,
                      lr: float, beta2: float = 0.95, eps: float = 1e-8):
    """Vectorised per-row update; returns (new table float64, new v float64, touched rows)."""
    h = np.asarray(h, np.int64).reshape(-1)
    dy = np.asarray(dy, np.float64).reshape(h.shape[0], -1)
    rows, inv = np.unique(h, return_inverse=True)
    g = np.zeros((rows.shape[0], dy.shape[1]), np.float64)
    np.add.at(g, inv, dy)
    w = np.asarray(table, np.float64).copy()
    vv = np.asarray(v, np.float64).copy()
    vr = beta2 * vv[rows] + (1.0 - beta2) * np.mean(g * g, axis=1)
    vv[rows] = vr
    w[rows] = w[rows] - lr * g / (np.sqrt(vr)[:, None] + eps)
    return w, vv, rows
