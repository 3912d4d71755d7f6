"""Oracle of inference: next-token logits and the sampling rule (numpy, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: GPT.forward with kv_cache and GPT.generate in the training script of the "$1000 tier
nanochat run" discussion (nanochat #8).  A key/value cache changes how the forward is computed,
not what it computes: the logits after a sequence of ids are those of the plain forward over the
whole sequence at its last position (causal attention), softcapped.  generate drops the logits
below the top_k-th largest (values equal to it stay), divides by the temperature, takes the
softmax and draws one id from it with a seeded generator; temperature 0 takes the argmax.

Reading: the draw is given as a uniform number u in [0, 1) per row, inverted through the
cumulative probabilities in vocabulary order (the first id whose cumulative probability exceeds
u); the argmax takes the first of equal maxima.
"""
from __future__ import annotations

import numpy as np

from oracle import model as om


def next_logits(cfg, params, ids: np.ndarray) -> np.ndarray:
    """ids [B, T] -> softcapped logits [B, V] of the last position (full forward, no cache)."""
    ids = np.asarray(ids, dtype=np.int64)
    B, T = ids.shape
    tokens = np.concatenate([ids, np.zeros((B, 1), np.int64)], axis=1)   # targets are unused
    res = om.forward_backward(cfg.replace(batch=B, seq_len=T), params, tokens, want_grads=False,
                              want_logits=True)
    return res.logits[:, -1, :]


def sample(logits: np.ndarray, temperature: float, top_k: int, u: np.ndarray) -> np.ndarray:
    """Token per row of logits [B, V] under the generate rule with uniforms u [B]."""
    z = np.asarray(logits, dtype=np.float64)
    out = np.empty(z.shape[0], dtype=np.int64)
    for b in range(z.shape[0]):
        row = z[b].copy()
        if temperature <= 0:
            out[b] = int(np.argmax(row))
            continue
        if 0 < top_k < row.size:
            kth = np.sort(row)[::-1][top_k - 1]
            row[row < kth] = -np.inf
        row = row / temperature
        p = np.exp(row - np.max(row))
        p /= p.sum()
        c = np.cumsum(p)
        idx = int(np.searchsorted(c, u[b], side="right"))
        out[b] = min(idx, int(np.nonzero(p > 0)[0][-1]))
    return out
