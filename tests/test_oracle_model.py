"""Pins of the CPU oracle's model step against things other than itself.

* central finite differences of the loss (fp64) for every parameter tensor and every addend,
  with a step small enough (1e-6) that the second-derivative kinks of ReLU^2 crossed by a step
  cost far less than the bar (observed errors <= 2e-7 against a bar of 1e-5);
* loss = ln V exactly when the LM head is zero (tanh(0) = 0, uniform softmax), and every
  other gradient exactly 0 then;
* causality: changing the token at position t leaves logits at positions < t unchanged;
* library routines of torch (rms_norm, scaled_dot_product_attention, cross_entropy) and
  closed forms for the primitives;
* a block with its residual branches zeroed reduces to the embedding/final-norm/head path; a
  block with a zero attention output, and a whole block at T = 1, reduce to closed forms of the
  MLP branch x + relu(norm(x) Wfc^T)^2 Wpr^T written with torch's rms_norm;
* rotary tables against hand-worked angles at frequency indices i >= 1.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as TF

from gpt_lm_step_amd import configs, inputs
from oracle import model as om
from oracle import tables as ot

TINY = configs.TINY


def _tiny_case(seed=7, tables=True, trigram=True, zero_head=False, std=0.02):
    cfg = TINY.replace(has_x0_add=int(tables), has_v_add=int(tables), has_trigram=int(trigram))
    params = inputs.model_params(cfg, seed=101, std=std, zero_head=zero_head)
    params = {k: v.astype(np.float64) for k, v in params.items()}
    tok = inputs.uniform_tokens(1, (cfg.batch, cfg.seq_len + 1), cfg.vocab)
    N, D = cfg.tokens, cfg.d_model
    x0 = inputs.addend(11, N, D, 0.02, False).astype(np.float64) if tables else None
    va = inputs.addend(12, N, D, 0.02, False).astype(np.float64) if tables else None
    tri = inputs.addend(13, N, D, 1.0, False).astype(np.float64) if trigram else None
    return cfg, params, tok, x0, va, tri


def _loss(cfg, params, tok, x0, va, tri, targets=None):
    return om.forward_backward(cfg, params, tok, x0, va, tri, want_grads=False,
                               targets=targets).loss


def test_finite_differences_every_tensor():
    cfg, params, tok, x0, va, tri = _tiny_case()
    res = om.forward_backward(cfg, params, tok, x0, va, tri)
    rng = np.random.default_rng(5)
    eps = 1e-6

    def fd_dir(get_set, d):
        base = get_set()
        get_set(base + eps * d)
        lp = _loss(cfg, params, tok, *addends)
        get_set(base - eps * d)
        lm = _loss(cfg, params, tok, *addends)
        get_set(base)
        return (lp - lm) / (2 * eps)

    addends = [x0, va, tri]
    checked = 0
    for name in list(params):
        def gs(new=None, name=name):
            if new is None:
                return params[name].copy()
            params[name] = new
        d = rng.standard_normal(params[name].shape)
        fd = fd_dir(gs, d)
        an = float(np.sum(res.grads[name] * d))
        assert abs(fd - an) <= 1e-5 * max(abs(an), 1e-6), (name, fd, an)
        # a few single coordinates too
        flat_idx = rng.integers(0, params[name].size, size=2)
        for fi in flat_idx:
            e = np.zeros(params[name].size)
            e[fi] = 1.0
            e = e.reshape(params[name].shape)
            fd = fd_dir(gs, e)
            an = float(res.grads[name].reshape(-1)[fi])
            # absolute floor: rounding of the two fp64 losses (|L| ~ 6.2) over the 2e-6 step,
            # 2 * 2^-52 * 6.2 / 2e-6 ~ 1.4e-9
            assert abs(fd - an) <= 1e-5 * abs(an) + 2e-9, (name, fi, fd, an)
        checked += 1
    for i, (nm, g) in enumerate([("x0_add", res.d_x0_add), ("v_add", res.d_v_add)]):
        def gs(new=None, i=i):
            if new is None:
                return addends[i].copy()
            addends[i] = new
        d = rng.standard_normal(addends[i].shape)
        fd = fd_dir(gs, d)
        an = float(np.sum(g * d))
        assert abs(fd - an) <= 1e-5 * max(abs(an), 1e-6), (nm, fd, an)
    assert checked == len(params)


def test_finite_differences_with_ignored_targets():
    cfg, params, tok, x0, va, tri = _tiny_case(tables=False, trigram=False)
    tgt = tok[:, 1:].copy()
    rng = np.random.default_rng(3)
    tgt[rng.random(tgt.shape) < 0.1] = -1
    res = om.forward_backward(cfg, params, tok, targets=tgt, grad_scale=0.25)
    eps = 1e-6
    for name in ["h1.wqkv", "lm_head", "wte"]:
        d = rng.standard_normal(params[name].shape)
        base = params[name].copy()
        params[name] = base + eps * d
        lp = _loss(cfg, params, tok, None, None, None, tgt)
        params[name] = base - eps * d
        lm = _loss(cfg, params, tok, None, None, None, tgt)
        params[name] = base
        fd = 0.25 * (lp - lm) / (2 * eps)
        an = float(np.sum(res.grads[name] * d))
        assert abs(fd - an) <= 1e-5 * abs(an), (name, fd, an)
    # the loss is the mean over valid targets only
    assert res.loss == pytest.approx(res.loss_per_token.sum() / np.sum(tgt >= 0), rel=1e-14)


def test_zero_head_gives_ln_vocab_and_zero_grads():
    cfg, params, tok, x0, va, tri = _tiny_case(zero_head=True)
    res = om.forward_backward(cfg, params, tok, x0, va, tri)
    assert res.loss == pytest.approx(6.238324625039508, abs=1e-12)   # ln 512
    assert math.log(512) == pytest.approx(6.238324625039508, abs=1e-15)
    for name, g in res.grads.items():
        if name != "lm_head":
            assert np.all(g == 0.0), name
    assert np.all(res.d_x0_add == 0.0) and np.all(res.d_v_add == 0.0)
    assert np.any(res.grads["lm_head"] != 0.0)


def test_causality_token_perturbation():
    """Changing input token t (and the table rows its hash selects) leaves logits < t fixed."""
    cfg = TINY.replace(has_x0_add=1, has_v_add=1)
    params = {k: v.astype(np.float64) for k, v in inputs.model_params(cfg, 101).items()}
    tx0 = inputs.normal(21, (4096, cfg.d_model), 0.02, False).astype(np.float64)
    tv = inputs.normal(22, (2048, cfg.d_model), 0.02, False).astype(np.float64)

    def run(tok):
        h = ot.hash_indices(tok[:, :cfg.seq_len], 2, cfg.vocab, 4096).reshape(-1)
        hv = ot.hash_indices(tok[:, :cfg.seq_len], 2, cfg.vocab, 2048).reshape(-1)
        return om.forward_backward(cfg, params, tok, tx0[h], tv[hv], None, want_grads=False,
                                   want_logits=True).logits

    tok = inputs.uniform_tokens(1, (cfg.batch, cfg.seq_len + 1), cfg.vocab)
    base = run(tok)
    for t in (0, 17, 40, 63):
        tok2 = tok.copy()
        tok2[:, t] = (tok2[:, t] + 123) % cfg.vocab
        out = run(tok2)
        assert np.array_equal(out[:, :t], base[:, :t]), t
        assert not np.allclose(out[:, t], base[:, t]), t


def test_residual_branches_zero_reduce_to_embedding_head_path():
    """With wo = wpr = 0 every block is the identity, so logits = cap*tanh(f Wh^T / cap) with
    f = rms(rms(wte[x]) + x0_add)."""
    cfg, params, tok, x0, va, tri = _tiny_case(trigram=False)
    for l in range(cfg.n_layer):
        params[f"h{l}.wo"][:] = 0
        params[f"h{l}.wpr"][:] = 0
    out = om.forward_backward(cfg, params, tok, x0, va, None, want_grads=False,
                              want_logits=True).logits.reshape(cfg.tokens, cfg.vocab)
    e = torch.tensor(params["wte"][tok[:, :cfg.seq_len].reshape(-1)])
    x = TF.rms_norm(e, (cfg.d_model,), eps=1e-6) + torch.tensor(x0)
    f = TF.rms_norm(x, (cfg.d_model,), eps=1e-6)
    z = f @ torch.tensor(params["lm_head"]).T
    ref = 15 * torch.tanh(z / 15)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_single_position_attention_is_value_path():
    """T = 1: softmax over one key is 1, so a layer with wfc = 0 gives
    x_out = x + (a Wv^T + u) Wo^T where a = rms(x)."""
    cfg = TINY.replace(seq_len=1, n_layer=1, has_v_add=1)
    params = {k: v.astype(np.float64) for k, v in inputs.model_params(cfg, 101).items()}
    params["h0.wfc"][:] = 0
    tok = inputs.uniform_tokens(3, (cfg.batch, 2), cfg.vocab)
    va = inputs.addend(12, cfg.tokens, cfg.d_model, 0.02, False).astype(np.float64)
    out = om.forward_backward(cfg, params, tok, None, va, None, want_grads=False,
                              want_logits=True).logits.reshape(cfg.tokens, cfg.vocab)
    D = cfg.d_model
    e = torch.tensor(params["wte"][tok[:, 0]])
    x = TF.rms_norm(e, (D,), eps=1e-6)
    a = TF.rms_norm(x, (D,), eps=1e-6)
    wv = torch.tensor(params["h0.wqkv"][2 * D:])
    x = x + (a @ wv.T + torch.tensor(va)) @ torch.tensor(params["h0.wo"]).T
    f = TF.rms_norm(x, (D,), eps=1e-6)
    ref = 15 * torch.tanh(f @ torch.tensor(params["lm_head"]).T / 15)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def _torch_mlp_branch(x, wfc, wpr):
    """Block.forward's second residual branch: x + mlp(norm(x)), mlp = relu(. Wfc^T)^2 Wpr^T."""
    b = TF.rms_norm(x, (x.shape[-1],), eps=1e-6)
    return x + torch.relu(b @ wfc.T).square() @ wpr.T


def test_zero_attention_output_reduces_block_to_mlp_branch():
    """One layer with wo = 0 over a full causal sequence: the attention branch adds nothing, so
    logits = cap*tanh(norm(x + relu(norm(x) Wfc^T)^2 Wpr^T) Wh^T / cap) with
    x = norm(wte[idx]) + x0_add.  The x0 addend is drawn with std 1 so that x is far from unit
    RMS, and wfc with std 0.2 so that the MLP moves x by tens of percents: feeding the MLP x
    instead of norm(x) (or dropping the branch) changes the logits at the first digit."""
    cfg = TINY.replace(n_layer=1, has_x0_add=1)
    params = {k: v.astype(np.float64) for k, v in inputs.model_params(cfg, 101).items()}
    params["h0.wo"][:] = 0
    params["h0.wfc"] *= 10.0
    tok = inputs.uniform_tokens(1, (cfg.batch, cfg.seq_len + 1), cfg.vocab)
    x0 = inputs.addend(11, cfg.tokens, cfg.d_model, 1.0, False).astype(np.float64)
    out = om.forward_backward(cfg, params, tok, x0, None, None, want_grads=False,
                              want_logits=True).logits.reshape(cfg.tokens, cfg.vocab)
    D = cfg.d_model
    e = torch.tensor(params["wte"][tok[:, :cfg.seq_len].reshape(-1)])
    x = TF.rms_norm(e, (D,), eps=1e-6) + torch.tensor(x0)
    x = _torch_mlp_branch(x, torch.tensor(params["h0.wfc"]), torch.tensor(params["h0.wpr"]))
    f = TF.rms_norm(x, (D,), eps=1e-6)
    ref = 15 * torch.tanh(f @ torch.tensor(params["lm_head"]).T / 15)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_single_position_block_closed_form():
    """T = 1, one full layer: x_mid = x + (a Wv^T + u) Wo^T with a = norm(x) (softmax over one
    key is 1), then x_out = x_mid + relu(norm(x_mid) Wfc^T)^2 Wpr^T.  wo (std 0.2) makes x_mid
    far from x, so an MLP fed norm(x) rather than norm(x_mid) fails."""
    cfg = TINY.replace(seq_len=1, n_layer=1, has_v_add=1)
    params = {k: v.astype(np.float64) for k, v in inputs.model_params(cfg, 101).items()}
    params["h0.wo"] *= 10.0
    params["h0.wfc"] *= 10.0
    tok = inputs.uniform_tokens(3, (cfg.batch, 2), cfg.vocab)
    va = inputs.addend(12, cfg.tokens, cfg.d_model, 1.0, False).astype(np.float64)
    out = om.forward_backward(cfg, params, tok, None, va, None, want_grads=False,
                              want_logits=True).logits.reshape(cfg.tokens, cfg.vocab)
    D = cfg.d_model
    e = torch.tensor(params["wte"][tok[:, 0]])
    x = TF.rms_norm(e, (D,), eps=1e-6)
    a = TF.rms_norm(x, (D,), eps=1e-6)
    wv = torch.tensor(params["h0.wqkv"][2 * D:])
    xm = x + (a @ wv.T + torch.tensor(va)) @ torch.tensor(params["h0.wo"]).T
    xo = _torch_mlp_branch(xm, torch.tensor(params["h0.wfc"]), torch.tensor(params["h0.wpr"]))
    f = TF.rms_norm(xo, (D,), eps=1e-6)
    ref = 15 * torch.tanh(f @ torch.tensor(params["lm_head"]).T / 15)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)
    # the MLP branch is not negligible here (it moves the residual stream by > 10%)
    assert float(torch.linalg.norm(xo - xm) / torch.linalg.norm(xm)) > 0.1


# ----------------------------------------------------------------------------- primitives

def test_rms_norm_against_torch_and_closed_form():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 7, 96)) * 3
    y, r = om.rms_norm(x, 1e-6)
    ref = TF.rms_norm(torch.tensor(x), (96,), eps=1e-6).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13)
    ms = np.mean(x * x, -1)
    np.testing.assert_allclose(np.mean(y * y, -1), ms / (ms + 1e-6), rtol=1e-13)
    # eps = 0: y is scale invariant and x . dx = 0 for any dy
    y0, r0 = om.rms_norm(x, 0.0)
    dy = rng.standard_normal(x.shape)
    dx = om.rms_norm_bwd(y0, r0, dy)
    np.testing.assert_allclose(np.sum(x * dx, -1), 0.0, atol=1e-10)


def test_rope_properties_and_worked_value():
    T, hd = 16, 32
    cos, sin = om.rope_tables(T, hd, 10000.0)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, T, 3, hd))
    y = om.rope(x, cos, sin)
    np.testing.assert_allclose(y[:, 0], x[:, 0], rtol=0, atol=0)          # position 0
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # <R_m q, R_n k> depends only on m - n
    q = np.broadcast_to(rng.standard_normal(hd), (1, T, 1, hd))
    k = np.broadcast_to(rng.standard_normal(hd), (1, T, 1, hd))
    rq, rk = om.rope(q, cos, sin)[0, :, 0], om.rope(k, cos, sin)[0, :, 0]
    assert np.dot(rq[5], rk[2]) == pytest.approx(np.dot(rq[12], rk[9]), rel=1e-12)
    # worked value from apply_rotary_emb: x2[0] = 1 at position 1 -> y1[0] = sin(1), y2[0] = cos(1)
    e = np.zeros((1, T, 1, hd))
    e[0, 1, 0, hd // 2] = 1.0
    ye = om.rope(e, cos, sin)[0, 1, 0]
    assert ye[0] == pytest.approx(0.8414709848078965, abs=1e-15)
    assert ye[hd // 2] == pytest.approx(0.5403023058681397, abs=1e-15)
    # backward is the transpose: <rope(x), dy> = <x, rope_bwd(dy)>
    dy = rng.standard_normal(x.shape)
    assert np.sum(y * dy) == pytest.approx(np.sum(x * om.rope_bwd(dy, cos, sin)), rel=1e-12)


def test_rope_worked_values_at_higher_frequency_indices():
    """The angle of pair i at position t is t * base^(-2i/Hd) (_precompute_rotary_embeddings:
    inv_freq = 1/base^(arange(0, Hd, 2)/Hd)).  Hand-worked at base 10000:
      Hd = 32, i = 8:  10000^(-16/32) = 0.01, position 3 -> angle 0.03,
        cos 0.03 = 1 - 0.03^2/2 + 0.03^4/24 - ... = 0.99955003374898754...,
        sin 0.03 = 0.03 - 0.03^3/6 + 0.03^5/120 - ... = 0.029995500202495660...
      Hd = 32, i = 4:  10000^(-8/32) = 0.1, position 5 -> angle 0.5 (cos 0.87758256189037276,
        sin 0.47942553860420301);
      Hd = 64, i = 16: 10000^(-32/64) = 0.01 again, position 3 -> angle 0.03.
    A base of 1e5, or an exponent of -i/Hd or -4i/Hd, gives other angles at all three."""
    c03, s03 = 0.99955003374898754, 0.029995500202495660
    c05, s05 = 0.87758256189037276, 0.47942553860420301
    cos, sin = om.rope_tables(8, 32, 10000.0)
    assert cos[3, 8] == pytest.approx(c03, abs=1e-15) and sin[3, 8] == pytest.approx(s03, abs=1e-15)
    assert cos[5, 4] == pytest.approx(c05, abs=1e-15) and sin[5, 4] == pytest.approx(s05, abs=1e-15)
    cos64, sin64 = om.rope_tables(8, 64, 10000.0)
    assert cos64[3, 16] == pytest.approx(c03, abs=1e-15)
    assert sin64[3, 16] == pytest.approx(s03, abs=1e-15)
    # through apply_rotary_emb: x1[i] = 1 at position t -> y1[i] = cos, y2[i] = -sin
    for hd, i, t, c, s_ in ((32, 8, 3, c03, s03), (32, 4, 5, c05, s05), (64, 16, 3, c03, s03)):
        co, si = om.rope_tables(8, hd, 10000.0)
        e = np.zeros((1, 8, 1, hd))
        e[0, t, 0, i] = 1.0
        y = om.rope(e, co, si)[0, t, 0]
        assert y[i] == pytest.approx(c, abs=1e-15) and y[hd // 2 + i] == pytest.approx(-s_, abs=1e-15)
        assert np.count_nonzero(y) == 2


def test_attention_against_torch_sdpa_and_special_cases():
    rng = np.random.default_rng(2)
    B, H, T, hd = 2, 3, 33, 16
    q, k, v = (rng.standard_normal((B, H, T, hd)) for _ in range(3))
    o, p = om.causal_attention(q, k, v)
    ref = TF.scaled_dot_product_attention(torch.tensor(q), torch.tensor(k), torch.tensor(v),
                                          is_causal=True).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    # T = 1 gives o = v
    o1, _ = om.causal_attention(q[:, :, :1], k[:, :, :1], v[:, :, :1])
    np.testing.assert_allclose(o1, v[:, :, :1], rtol=1e-15)
    # constant keys: o_t = mean_{s<=t} v_s
    kc = np.broadcast_to(k[:, :, :1], k.shape).copy()
    oc, _ = om.causal_attention(q, kc, v)
    cm = np.cumsum(v, axis=2) / np.arange(1, T + 1)[None, None, :, None]
    np.testing.assert_allclose(oc, cm, rtol=1e-12, atol=1e-13)
    # backward against torch autograd of SDPA
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    do = rng.standard_normal(o.shape)
    TF.scaled_dot_product_attention(tq, tk, tv, is_causal=True).backward(torch.tensor(do))
    dq, dk, dv = om.causal_attention_bwd(q, k, v, p, o, do)
    for a, b in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(a, b.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_softcap_cross_entropy_against_torch():
    rng = np.random.default_rng(4)
    N, V = 40, 97
    z = rng.standard_normal((N, V)) * 20
    tgt = rng.integers(0, V, N)
    tgt[::7] = -1
    loss, g = om.softcap_cross_entropy(z, tgt, 15.0)
    tz = torch.tensor(z, requires_grad=True)
    c = 15 * torch.tanh(tz / 15)
    ref = TF.cross_entropy(c, torch.tensor(tgt), ignore_index=-1, reduction="sum")
    assert loss.sum() == pytest.approx(ref.item(), rel=1e-13)
    ref.backward()
    np.testing.assert_allclose(g, tz.grad.numpy(), rtol=1e-10, atol=1e-14)
    # without the cap the per-row gradient sums to zero (softmax - onehot)
    _, g0 = om.softcap_cross_entropy(z, tgt, 0.0)
    np.testing.assert_allclose(g0.sum(-1), 0.0, atol=1e-13)


def test_param_and_flop_counts_match_the_d32_log():
    golden = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", "nanochat_d32.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                golden[k] = float(v)
    assert configs.n_params(configs.D32) == int(golden["n_params"])
    assert configs.flops_per_token(configs.D32) == pytest.approx(golden["flops_per_token"],
                                                                 rel=5e-7)


def test_qk_norm_makes_scores_invariant_to_query_key_scale():
    """norm(q), norm(k) per head (CausalSelfAttention.forward): scaling Wq, Wk by any c > 0
    leaves the logits unchanged up to the eps inside the norm; without the QK-norm the same
    scaling sharpens every softmax and moves the logits by percents."""
    cfg, params, tok, x0, va, tri = _tiny_case(trigram=False)
    D = cfg.d_model
    p2 = {k: v.copy() for k, v in params.items()}
    p2["h0.wqkv"][:2 * D] *= 9.0

    def logits(c, p):
        return om.forward_backward(c, p, tok, x0, va, None, want_grads=False,
                                   want_logits=True).logits

    def rel(a, b):
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    # mean(q^2) is about 0.05 here, so eps = 1e-6 moves the normalized q, k by ~1e-5 relative
    on = rel(logits(cfg, p2), logits(cfg, params))
    assert on <= 1e-5, on
    off = cfg.replace(qk_norm=0)
    moved = rel(logits(off, p2), logits(off, params))
    assert moved >= 1e-2, moved          # observed 3.5e-2: 1e5 times the invariant case


def test_relu_squared_is_degree_two_homogeneous():
    """relu(s*h)^2 = s^2 relu(h)^2 for s > 0: Wfc*s with Wpr/s^2 gives the same loss (a gelu or
    plain relu activation would not)."""
    cfg, params, tok, x0, va, tri = _tiny_case(trigram=False)
    base = _loss(cfg, params, tok, x0, va, None)
    p2 = {k: v.copy() for k, v in params.items()}
    p2["h1.wfc"] *= 3.0
    p2["h1.wpr"] /= 9.0
    assert _loss(cfg, p2, tok, x0, va, None) == pytest.approx(base, rel=1e-12)
    p3 = {k: v.copy() for k, v in params.items()}
    p3["h1.wfc"] *= 3.0
    p3["h1.wpr"] /= 3.0
    assert abs(_loss(cfg, p3, tok, x0, va, None) - base) > 1e-6
