"""Oracle of the dense optimizer step that follows a training step (numpy, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: the training script posted in the "$1000 tier nanochat run" discussion (nanochat #8): its
`Muon` class and `zeropower_via_newtonschulz5`, `setup_optimizers`, `get_lr_multiplier`,
`get_muon_momentum` and the gradient-accumulation loop; the modded-nanogpt README for the
Newton-Schulz precision (the iteration is run in bfloat16).

* clipping: the global L2 norm of every model gradient; when max_norm / (norm + 1e-6) < 1 every
  gradient is multiplied by that factor (the loop clips before stepping, with max_norm 1.0).
* Adam (AdamW with weight decay 0, betas 0.8 / 0.95, eps 1e-10, bias-corrected) for the token
  embedding (lr 0.2) and the LM head (lr 0.004), both scaled by (d_model / 768)^-1/2.
* Muon (lr 0.02) for every matrix of the blocks - q, k and v each as its own D x D matrix, the
  output projection, the MLP up and down projections: an exponential moving average of the
  gradient (weight 1 - momentum on the new gradient), its Nesterov form
  u = g + momentum (buf - g), five quintic Newton-Schulz steps on u, and the step
  -lr sqrt(max(1, rows / cols)) X.
* Newton-Schulz: X = u (tall matrices transposed), divided by its Frobenius norm + 1e-7, then five
  times A = X X^T, B = b A + c A A, X = a X + B X with (a, b, c) = (3.4445, -4.7750, 2.0315).
* schedules: the lr multiplier is 1 up to the last warmdown_ratio of the iterations and then falls
  linearly to final_lr_frac; Muon's momentum rises linearly from 0.85 to 0.95 over 300 iterations.

Readings (where the pages leave a step open): the Frobenius norm is that of the bf16-rounded
matrix, not itself rounded; in bf16 mode each new matrix of the iteration (X after the scaling,
A, B, X) is the exact result of its formula on bf16 inputs rounded once to bf16; the trigram
projection, a hidden D x D matrix, is stepped by Muon; the master weights are fp32 (the pages'
parameters) and the bf16 copy used by the step is their round-to-nearest-even rounding.
"""
from __future__ import annotations

import math
from typing import Dict, Tuple

import numpy as np

NS_COEFFS = (3.4445, -4.7750, 2.0315)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, ties to even) of every element, as float64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                      # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def lr_multiplier(it: int, num_iterations: int, warmup_ratio: float, warmdown_ratio: float,
                  final_lr_frac: float) -> float:
    """Learning-rate factor of iteration `it`: linear warmup, constant, linear warmdown."""
    warmup = round(warmup_ratio * num_iterations)
    warmdown = round(warmdown_ratio * num_iterations)
    if it < warmup:
        return (it + 1) / warmup
    if it <= num_iterations - warmdown:
        return 1.0
    progress = (num_iterations - it) / warmdown
    return progress + (1.0 - progress) * final_lr_frac


def muon_momentum(it: int) -> float:
    """Muon's momentum at iteration `it`: 0.85 rising linearly to 0.95 over 300 iterations."""
    frac = min(it / 300.0, 1.0)
    return (1.0 - frac) * 0.85 + frac * 0.95


def clip_factor(grads, max_norm: float) -> Tuple[float, float]:
    """(global L2 norm of all gradients, factor applied to every gradient)."""
    total = math.sqrt(sum(float(np.sum(np.asarray(g, np.float64) ** 2)) for g in grads))
    coef = max_norm / (total + 1e-6)
    return total, min(coef, 1.0)


def newton_schulz5(G: np.ndarray, steps: int = 5, bf16: bool = True) -> np.ndarray:
    """Approximate orthogonalization of a 2-D matrix by the quintic Newton-Schulz iteration.
    bf16=True keeps every matrix of the iteration in bfloat16 (exact products, one rounding per
    new matrix); bf16=False runs it exactly in float64."""
    a, b, c = NS_COEFFS
    rnd = round_bf16 if bf16 else (lambda y: y)
    X = rnd(np.asarray(G, dtype=np.float64))
    tall = X.shape[0] > X.shape[1]
    if tall:
        X = X.T
    X = rnd(X / (np.sqrt(np.sum(X * X)) + 1e-7))
    for _ in range(steps):
        A = rnd(X @ X.T)
        B = rnd(b * A + c * (A @ A))
        X = rnd(a * X + B @ X)
    return X.T if tall else X


def adam_update(p, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float,
                weight_decay: float):
    """One bias-corrected Adam step with decoupled weight decay; returns (p, m, v)."""
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    return p - lr * mhat / (np.sqrt(vhat) + eps), m, v


def muon_update(p, g, buf, lr: float, momentum: float, nesterov: bool = True, ns_steps: int = 5,
                bf16: bool = True):
    """One Muon step of a 2-D matrix; returns (p, buf)."""
    buf = buf + (1.0 - momentum) * (g - buf)
    u = g + momentum * (buf - g) if nesterov else buf
    X = newton_schulz5(u, ns_steps, bf16)
    scale = math.sqrt(max(1.0, p.shape[0] / p.shape[1]))
    return p - lr * scale * X, buf


def muon_matrices(cfg) -> list:
    """(name, tensor, row slice) of every matrix Muon steps: per layer q, k, v (row blocks of
    wqkv), wo, wfc, wpr; the trigram projection when present."""
    D = cfg.d_model
    out = []
    for l in range(cfg.n_layer):
        for i, part in enumerate(("q", "k", "v")):
            out.append((f"h{l}.{part}", f"h{l}.wqkv", slice(i * D, (i + 1) * D)))
        out.append((f"h{l}.wo", f"h{l}.wo", slice(None)))
        out.append((f"h{l}.wfc", f"h{l}.wfc", slice(None)))
        out.append((f"h{l}.wpr", f"h{l}.wpr", slice(None)))
    if cfg.has_trigram:
        out.append(("wtri", "wtri", slice(None)))
    return out


def optimizer_step(cfg, master: Dict[str, np.ndarray], grads: Dict[str, np.ndarray],
                   state: Dict[str, np.ndarray], it: int, t: int, hp: Dict[str, float],
                   bf16: bool = True):
    """One optimizer step of every model tensor.  master: fp32 weights by tensor name; grads:
    gradients by name; state: 'mom.<matrix>' Muon buffers and 'm.<name>', 'v.<name>' Adam moments
    (zeros when absent); it: iteration (schedules); t: Adam step count (1 on the first step);
    hp: lr_matrix, lr_embedding, lr_unembedding, beta1, beta2, eps, weight_decay, grad_clip,
    num_iterations, warmup_ratio, warmdown_ratio, final_lr_frac, nesterov, ns_steps.
    Returns (new master, new state, grad_norm)."""
    P = {k: np.asarray(v, np.float64).copy() for k, v in master.items()}
    S = {k: np.asarray(v, np.float64).copy() for k, v in state.items()}
    G = {k: np.asarray(v, np.float64) for k, v in grads.items()}
    norm, coef = clip_factor(G.values(), hp["grad_clip"]) if hp["grad_clip"] > 0 else (
        math.sqrt(sum(float(np.sum(g * g)) for g in G.values())), 1.0)
    G = {k: g * coef for k, g in G.items()}
    lrm = lr_multiplier(it, hp["num_iterations"], hp["warmup_ratio"], hp["warmdown_ratio"],
                        hp["final_lr_frac"])
    mu = muon_momentum(it)
    scale = (cfg.d_model / 768.0) ** -0.5
    for name, lr0 in (("lm_head", hp["lr_unembedding"] * scale), ("wte", hp["lr_embedding"] * scale)):
        m = S.get(f"m.{name}", np.zeros_like(P[name]))
        v = S.get(f"v.{name}", np.zeros_like(P[name]))
        P[name], S[f"m.{name}"], S[f"v.{name}"] = adam_update(
            P[name], G[name], m, v, t, lr0 * lrm, hp["beta1"], hp["beta2"], hp["eps"],
            hp["weight_decay"])
    for mname, tensor, rows in muon_matrices(cfg):
        p = P[tensor][rows]
        buf = S.get(f"mom.{mname}", np.zeros_like(p))
        newp, S[f"mom.{mname}"] = muon_update(p, G[tensor][rows], buf, hp["lr_matrix"] * lrm, mu,
                                              bool(hp["nesterov"]), int(hp["ns_steps"]), bf16)
        P[tensor][rows] = newp
    return P, S, norm
