"""Oracle forward and hand-derived backward of one decoder training step (numpy, float64).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source of every definition: the GPT module posted in the "$1000 tier nanochat run" discussion
(nanochat #8, a commenter's training script), read with the modded-nanogpt README's
architecture list, and the decoder-rtx posts for the table addends:

* norm(x): RMSNorm over the last dim with no weight or bias (the `norm` helper; README:
  "Removed all affine scale and bias parameters ... switched to RMSNorm").  eps = 1e-6.
* rotary: `apply_rotary_emb` splits the head dim into halves x1, x2 and returns
  [x1*cos + x2*sin, -x1*sin + x2*cos]; `_precompute_rotary_embeddings` uses
  inv_freq = base^-(2i/Hd), base 10000, positions 0..T-1.
* attention (`CausalSelfAttention.forward`): q = x Wq^T, k, v alike; rotary on q and k; then
  QK-norm (norm(q), norm(k) per head); causal softmax(q k^T / sqrt(Hd)) v; output projection.
* block (`Block.forward`): x = x + attn(norm(x)); x = x + mlp(norm(x)).
* MLP: c_fc (D -> 4D), squared activation, c_proj (4D -> D).  The activation is ReLU^2 (the
  README's "ReLU^2 activation" and the decoder-rtx "ReLU^2 backward"), not the gelu-square
  that the posted script has.
* `GPT.forward`: x = norm(wte(idx)); blocks; x = norm(x); logits = lm_head(x);
  logits = 15*tanh(logits/15); cross-entropy (mean over targets != -1) on float logits.
* tables (decoder-rtx, baseline 4): a bigram-table row is added to x0 (the stream entering
  block 0, after the embedding norm); a bigram-table row plus a projected frozen trigram row
  is added to the attention values in every layer.

Backward is the chain rule written out by hand; it is pinned by central finite differences.
The returned gradients are those of grad_scale * loss.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np


# ----------------------------------------------------------------------------- primitives

def rms_norm(x: np.ndarray, eps: float):
    """y = x / sqrt(mean(x^2) + eps) over the last dim; also returns r = 1/sqrt(...)."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1) + eps)
    return x * r[..., None], r


def rms_norm_bwd(y: np.ndarray, r: np.ndarray, dy: np.ndarray) -> np.ndarray:
    """d/dx of y = x*r(x):  dx = r * (dy - y * mean(dy * y))."""
    return r[..., None] * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def rope_tables(T: int, head_dim: int, base: float, dtype=np.float64):
    """cos/sin [T, Hd/2] of angle t * base^-(2i/Hd)."""
    inv_freq = base ** (-(np.arange(0, head_dim, 2, dtype=np.float64) / head_dim))
    ang = np.outer(np.arange(T, dtype=np.float64), inv_freq)
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x [B, T, H, Hd]; half-split rotation y1 = x1 c + x2 s, y2 = -x1 s + x2 c."""
    d = x.shape[-1] // 2
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    x1, x2 = x[..., :d], x[..., d:]
    return np.concatenate([x1 * c + x2 * s, -x1 * s + x2 * c], axis=-1)


def rope_bwd(dy: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Transpose of the rotation: dx1 = dy1 c - dy2 s, dx2 = dy1 s + dy2 c."""
    d = dy.shape[-1] // 2
    c, s = cos[None, :, None, :], sin[None, :, None, :]
    dy1, dy2 = dy[..., :d], dy[..., d:]
    return np.concatenate([dy1 * c - dy2 * s, dy1 * s + dy2 * c], axis=-1)


def causal_attention(q, k, v):
    """q, k, v [B, H, T, Hd] -> (o [B,H,T,Hd], p [B,H,T,T]); scale 1/sqrt(Hd), keys s <= t."""
    T, hd = q.shape[2], q.shape[3]
    s = (q @ np.swapaxes(k, -1, -2)) / math.sqrt(hd)
    mask = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(mask, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ v, p


def causal_attention_bwd(q, k, v, p, o, do):
    """Softmax-attention backward: dv = p^T do; dp = do v^T; ds = p (dp - rowsum(do*o));
    dq = ds k / sqrt(Hd); dk = ds^T q / sqrt(Hd)."""
    hd = q.shape[-1]
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    delta = np.sum(do * o, axis=-1, keepdims=True)
    ds = p * (dp - delta)
    scale = 1.0 / math.sqrt(hd)
    dq = (ds @ k) * scale
    dk = (np.swapaxes(ds, -1, -2) @ q) * scale
    return dq, dk, dv


def softcap_cross_entropy(z: np.ndarray, tgt: np.ndarray, cap: float):
    """Per-token loss of softcapped logits c = cap*tanh(z/cap) (cap 0 = no cap), and
    dloss_t/dz_t.  z [N, V] float, tgt [N] (-1 = ignored).  Ignored rows get loss 0, grad 0."""
    if cap > 0:
        th = np.tanh(z / cap)
        c = cap * th
        chain = 1.0 - th * th
    else:
        c = z
        chain = np.ones_like(z)
    m = c.max(axis=-1, keepdims=True)
    e = np.exp(c - m)
    se = e.sum(axis=-1, keepdims=True)
    lse = (m + np.log(se))[:, 0]
    valid = tgt >= 0
    t = np.where(valid, tgt, 0)
    loss = np.where(valid, lse - c[np.arange(len(t)), t], 0.0)
    g = e / se
    g[np.arange(len(t)), t] -= 1.0
    g *= chain
    g[~valid] = 0.0
    return loss, g


# ----------------------------------------------------------------------------- the step

class Result:
    def __init__(self):
        self.loss = None          # mean CE over valid targets (unscaled)
        self.loss_per_token = None
        self.grads: Dict[str, np.ndarray] = {}
        self.d_x0_add = None
        self.d_v_add = None
        self.logits = None        # softcapped logits [B, T, V] when requested


def _split_heads(x, B, T, H, hd):
    return x.reshape(B, T, H, hd)


def forward_backward(cfg, params: Dict[str, np.ndarray], tokens: np.ndarray,
                     x0_add: Optional[np.ndarray] = None, v_add: Optional[np.ndarray] = None,
                     tri_rows: Optional[np.ndarray] = None, grad_scale: float = 1.0,
                     want_grads: bool = True, want_logits: bool = False,
                     dtype=np.float64, targets: Optional[np.ndarray] = None) -> Result:
    """One training step of the decoder.

    tokens [B, T+1]: inputs tokens[:, :T], targets tokens[:, 1:] (unless `targets` [B, T] is
    given, where -1 marks an ignored position).  params: name -> array per the flat layout
    names (wte, h{l}.wqkv with q/k/v rows stacked, h{l}.wo, h{l}.wfc, h{l}.wpr, lm_head, wtri).
    x0_add, v_add, tri_rows: [B*T, D] per-token addends (gathered table rows) or None.
    Activations are recomputed per layer in backward (only each layer's input is kept).
    """
    B, T = tokens.shape[0], tokens.shape[1] - 1
    D, H, hd, V = cfg.d_model, cfg.n_head, cfg.head_dim, cfg.vocab
    L, eps, cap = cfg.n_layer, cfg.rms_eps, cfg.softcap
    N = B * T
    inp = tokens[:, :T].reshape(N).astype(np.int64)
    tgt = (tokens[:, 1:] if targets is None else targets).reshape(N).astype(np.int64)
    P = {k: np.asarray(v, dtype=dtype) for k, v in params.items()}
    cos, sin = rope_tables(T, hd, cfg.rope_base, dtype)

    # value addend u (same in every layer): bigram value row + trigram row projected by wtri
    u = None
    if v_add is not None:
        u = np.asarray(v_add, dtype=dtype).copy()
    if tri_rows is not None:
        tri = np.asarray(tri_rows, dtype=dtype)
        proj = tri @ P["wtri"].T
        u = proj if u is None else u + proj

    def layer_fwd(l, x, keep=False):
        wqkv = P[f"h{l}.wqkv"]
        wq, wk, wv = wqkv[:D], wqkv[D:2 * D], wqkv[2 * D:]
        a, ra = rms_norm(x, eps)
        q0, k0, v = a @ wq.T, a @ wk.T, a @ wv.T
        if u is not None:
            v = v + u
        q1 = rope(_split_heads(q0, B, T, H, hd), cos, sin)
        k1 = rope(_split_heads(k0, B, T, H, hd), cos, sin)
        if cfg.qk_norm:
            q2, rq = rms_norm(q1, eps)
            k2, rk = rms_norm(k1, eps)
        else:
            q2, rq, k2, rk = q1, None, k1, None
        qh, kh = q2.transpose(0, 2, 1, 3), k2.transpose(0, 2, 1, 3)
        vh = _split_heads(v, B, T, H, hd).transpose(0, 2, 1, 3)
        oh, p = causal_attention(qh, kh, vh)
        o = oh.transpose(0, 2, 1, 3).reshape(N, D)
        xm = x + o @ P[f"h{l}.wo"].T
        b, rb = rms_norm(xm, eps)
        hp = b @ P[f"h{l}.wfc"].T
        act = np.maximum(hp, 0.0) ** 2
        xo = xm + act @ P[f"h{l}.wpr"].T
        if not keep:
            return xo
        return xo, dict(a=a, ra=ra, q2=q2, rq=rq, k2=k2, rk=rk, qh=qh, kh=kh, vh=vh, oh=oh, p=p,
                        o=o, xm=xm, b=b, rb=rb, hp=hp, act=act)

    # forward
    e = P["wte"][inp]
    x, re = rms_norm(e, eps)
    x0_normed = x
    if x0_add is not None:
        x = x + np.asarray(x0_add, dtype=dtype)
    xs = []
    for l in range(L):
        xs.append(x)
        x = layer_fwd(l, x)
    f, rf = rms_norm(x, eps)
    z = f @ P["lm_head"].T
    loss_t, dz = softcap_cross_entropy(z, tgt, cap)
    n_valid = int(np.sum(tgt >= 0))
    res = Result()
    res.loss_per_token = loss_t
    res.loss = float(np.sum(loss_t) / max(n_valid, 1))
    if want_logits:
        c = cap * np.tanh(z / cap) if cap > 0 else z
        res.logits = c.reshape(B, T, V)
    if not want_grads:
        return res

    # backward
    G = {k: np.zeros_like(v) for k, v in P.items()}
    dz = dz * (grad_scale / max(n_valid, 1))
    G["lm_head"] = dz.T @ f
    df = dz @ P["lm_head"]
    dx = rms_norm_bwd(f, rf, df)
    du = np.zeros((N, D), dtype=dtype) if u is not None else None
    for l in reversed(range(L)):
        _, c_ = layer_fwd(l, xs[l], keep=True)
        wqkv = P[f"h{l}.wqkv"]
        # MLP: xo = xm + relu(b Wfc^T)^2 Wpr^T
        G[f"h{l}.wpr"] = dx.T @ c_["act"]
        dact = dx @ P[f"h{l}.wpr"]
        dhp = dact * 2.0 * np.maximum(c_["hp"], 0.0)
        G[f"h{l}.wfc"] = dhp.T @ c_["b"]
        db = dhp @ P[f"h{l}.wfc"]
        dxm = dx + rms_norm_bwd(c_["b"], c_["rb"], db)
        # attention: xm = x + o Wo^T
        G[f"h{l}.wo"] = dxm.T @ c_["o"]
        do = (dxm @ P[f"h{l}.wo"]).reshape(B, T, H, hd).transpose(0, 2, 1, 3)
        dqh, dkh, dvh = causal_attention_bwd(c_["qh"], c_["kh"], c_["vh"], c_["p"], c_["oh"], do)
        dq2, dk2 = dqh.transpose(0, 2, 1, 3), dkh.transpose(0, 2, 1, 3)
        dv = dvh.transpose(0, 2, 1, 3).reshape(N, D)
        if cfg.qk_norm:
            dq1 = rms_norm_bwd(c_["q2"], c_["rq"], dq2)
            dk1 = rms_norm_bwd(c_["k2"], c_["rk"], dk2)
        else:
            dq1, dk1 = dq2, dk2
        dq0 = rope_bwd(dq1, cos, sin).reshape(N, D)
        dk0 = rope_bwd(dk1, cos, sin).reshape(N, D)
        if du is not None:
            du += dv
        dqkv = np.concatenate([dq0, dk0, dv], axis=1)
        G[f"h{l}.wqkv"] = dqkv.T @ c_["a"]
        da = dqkv @ wqkv
        dx = dxm + rms_norm_bwd(c_["a"], c_["ra"], da)
    # embedding + x0 addend
    if x0_add is not None:
        res.d_x0_add = dx.copy()
    de = rms_norm_bwd(x0_normed, re, dx)
    np.add.at(G["wte"], inp, de)
    if du is not None:
        if v_add is not None:
            res.d_v_add = du
        if tri_rows is not None:
            G["wtri"] = du.T @ np.asarray(tri_rows, dtype=dtype)
    res.grads = G
    return res
