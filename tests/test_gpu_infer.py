"""GPU parity of inference with a key/value cache (gpt_infer_*) and of gpt_sample against the
oracle (oracle/infer.py, oracle/model.py).

Logits: fp32 path rel-L2 <= 1e-5 and max |diff| <= 1e-4 against the fp64 oracle; bf16 path
rel-L2 <= 3e-2 and cosine >= 0.999 (the training step's bf16 gradient bar).  Sampling: the argmax
is exact; a draw is the id whose cumulative-probability cell holds u, up to 2e-5 at a cell edge
(fp32 sums on the device), and always an id the top-k rule keeps; away from the edges it is the
oracle's id exactly.
"""
import numpy as np
import pytest
import torch

from gpt_lm_step_amd import binding as B
from gpt_lm_step_amd import configs, inputs
from oracle import infer as oi
from oracle import model as om

from gpu_util import cosine, dev, host, rel_l2

pytestmark = pytest.mark.gpu

BF16_SMALL = configs.TINY.replace(n_layer=2, d_model=256, n_head=4, head_dim=64, d_mlp=1024,
                                  vocab=960, dtype=configs.BF16, name="small-bf16")
BF16_HD128 = BF16_SMALL.replace(n_head=2, head_dim=128, name="small-bf16-hd128")


def _model(cfg, seed):
    params = inputs.model_params(cfg, seed)
    dt = torch.bfloat16 if cfg.dtype == configs.BF16 else torch.float32
    return params, dev(inputs.flatten_params(cfg, params), dt)


def _run_chunks(cfg, flat, tok, chunks, max_seq):
    """Feeds tok [B, sum(chunks)] chunk by chunk; returns [(position after the chunk, logits)]."""
    ctx = B.gpt_infer_init(cfg, tok.shape[0], max_seq)
    logits = torch.full((tok.shape[0], cfg.vocab), float("nan"), device="cuda")
    out, p = [], 0
    for n in chunks:
        B.gpt_infer_forward(ctx, flat, dev(np.ascontiguousarray(tok[:, p:p + n]).astype(np.int32)),
                            logits)
        torch.cuda.synchronize()
        p += n
        assert B.gpt_infer_position(ctx) == p
        out.append((p, host(logits).copy()))
    return out


def _check_logits(got, want, bf16):
    if bf16:
        assert rel_l2(got, want) <= 3e-2, rel_l2(got, want)
        assert cosine(got, want) >= 0.999
    else:
        assert rel_l2(got, want) <= 1e-5, rel_l2(got, want)
        assert np.max(np.abs(got - want)) <= 1e-4


@pytest.mark.parametrize("cfg,chunks", [
    (configs.TINY, [10, 1, 1, 1, 7, 1, 19]),        # cache path throughout
    (configs.TINY, [64, 1, 1, 3]),                   # full causal prefill, then the cache
    (BF16_SMALL, [128, 1, 1, 2, 1]),
    (BF16_SMALL, [37, 1, 26]),
    (BF16_HD128, [64, 1, 5, 1]),
    (BF16_SMALL, [320, 1, 3, 1]),                    # decode over two key splits
    (configs.TINY, [64, 200, 1, 16]),                # long chunk after a prefix, then splits
    (configs.TINY, [45, 3, 1]),                      # first chunk not a multiple of 32
    (BF16_SMALL, [40, 8, 10]),                       # 24 and 30 token rows on the decode GEMM
], ids=["fp32-chunks", "fp32-prefill64", "bf16-prefill128", "bf16-ragged", "bf16-hd128",
        "bf16-two-splits", "fp32-long-chunk", "fp32-ragged-prefill", "bf16-wide-decode"])
def test_chunked_inference_matches_the_full_forward(cfg, chunks):
    """Logits after every chunk equal the oracle's full forward over the whole prefix: one
    oracle pass gives every position's logits (causality is pinned in the oracle's tests).  The
    chunks cover each attention path: the causal kernel of training (first chunks of more than 16
    tokens, including lengths that are not a multiple of 32) and the key-split kernel (first
    chunks of up to 16 tokens, every later chunk in groups of 16 queries, one or more splits of
    128 keys); bf16 chunks of up to 32 tokens in all take the decode GEMM."""
    params, flat = _model(cfg, 201)
    n = sum(chunks)
    tok = inputs.uniform_tokens(7, (3, n + 1), cfg.vocab)
    got = _run_chunks(cfg, flat, tok, chunks, max_seq=n + 8)
    full = om.forward_backward(cfg.replace(batch=3, seq_len=n), params, tok, want_grads=False,
                               want_logits=True).logits
    for p, lg in got:
        _check_logits(lg, full[:, p - 1], cfg.dtype == configs.BF16)


def test_next_logits_after_a_single_token():
    """A one-token prompt (no cache yet) and a batch of one."""
    cfg = configs.TINY
    params, flat = _model(cfg, 202)
    tok = inputs.uniform_tokens(8, (1, 1), cfg.vocab)
    (_, got), = _run_chunks(cfg, flat, tok, [1], max_seq=1)
    _check_logits(got, oi.next_logits(cfg, params, tok), False)


def test_out_of_range_ids_are_clamped_and_reported():
    """An id >= vocab (or < 0) is read as the nearest valid id, flagged, and the flag clears on
    reading; the logits equal those of the clamped ids."""
    cfg = configs.TINY
    params, flat = _model(cfg, 205)
    ctx = B.gpt_infer_init(cfg, 2, 8)
    assert B.gpt_infer_check_errors(ctx) == 0
    tok = inputs.uniform_tokens(13, (2, 4), cfg.vocab)
    bad = tok.copy()
    bad[0, 1], bad[1, 3] = cfg.vocab + 5, -3
    logits = torch.empty(2, cfg.vocab, device="cuda")
    B.gpt_infer_forward(ctx, flat, dev(bad), logits)
    assert B.gpt_infer_check_errors(ctx) == 1
    assert B.gpt_infer_check_errors(ctx) == 0
    clamped = np.clip(bad, 0, cfg.vocab - 1)
    _check_logits(host(logits), oi.next_logits(cfg, params, clamped), False)
    ctx.close()


def test_reset_position_and_batch_rules():
    cfg = configs.TINY
    _, flat = _model(cfg, 203)
    ctx = B.gpt_infer_init(cfg, 4, 16)
    logits = torch.empty(4, cfg.vocab, device="cuda")
    t3 = dev(inputs.uniform_tokens(9, (3, 10), cfg.vocab))
    B.gpt_infer_forward(ctx, flat, t3, logits[:3])
    assert B.gpt_infer_position(ctx) == 10
    with pytest.raises(B.GptError) as e:                 # batch fixed until reset
        B.gpt_infer_forward(ctx, flat, dev(inputs.uniform_tokens(9, (4, 1), cfg.vocab)), logits)
    assert e.value.status == B.GPT_ESHAPE
    with pytest.raises(B.GptError) as e:                 # 10 + 7 > 16
        B.gpt_infer_forward(ctx, flat, t3[:, :7].contiguous(), logits[:3])
    assert e.value.status == B.GPT_ERANGE
    assert B.gpt_infer_position(ctx) == 10
    B.gpt_infer_forward(ctx, flat, t3[:, :6].contiguous(), logits[:3])
    assert B.gpt_infer_position(ctx) == 16
    B.gpt_infer_reset(ctx)
    assert B.gpt_infer_position(ctx) == 0
    t4 = dev(inputs.uniform_tokens(10, (4, 16), cfg.vocab))
    B.gpt_infer_forward(ctx, flat, t4, logits)           # new batch size after reset
    torch.cuda.synchronize()
    assert np.isfinite(host(logits)).all()
    ctx.close()


def test_d32_full_size_prefill_then_decode_sampled():
    """The d32 model (32 layers, d2048, 16 heads x 128, V=65536, device-drawn N(0, 0.02) bf16
    weights), batch 8: a 256-token prefill of Zipf tokens, then two single-token decode steps;
    sequences 0 and 5 are checked against one oracle pass over their 258 tokens."""
    cfg = configs.D32
    P, picks = 256, (0, 5)
    flat = inputs.device_params(cfg, 103)
    tok = inputs.zipf_tokens(11, (cfg.batch, P + 3), cfg.vocab)
    got = _run_chunks(cfg, flat, tok, [P, 1, 1], max_seq=512)
    params = inputs.unflatten(cfg, flat.float().cpu().numpy())
    del flat
    torch.cuda.empty_cache()
    sel = tok[list(picks)]
    full = om.forward_backward(cfg.replace(batch=len(picks), seq_len=P + 2), params, sel,
                               want_grads=False, want_logits=True).logits
    for p, lg in got:
        for i, b in enumerate(picks):
            _check_logits(lg[b], full[i, p - 1], True)


# ---------------------------------------------------------------- sampling

def _sample(logits, temperature, top_k, u):
    out = torch.full((logits.shape[0],), -7, dtype=torch.int32, device="cuda")
    B.gpt_sample(dev(logits.astype(np.float32)), temperature, top_k,
                 None if u is None else dev(u.astype(np.float32)), out)
    torch.cuda.synchronize()
    return host(out)


@pytest.mark.parametrize("V", [512, 1000, 16384, 16385, 50304, 65536])
def test_argmax_is_exact_with_ties(V):
    rng = np.random.default_rng(V)
    z = rng.standard_normal((6, V)).astype(np.float32)
    z[1, V // 3] = z[1].max()            # a tie later than the first maximum ...
    z[2, :] = 0.25                       # ... all equal ...
    z[3, V - 1] = 100.0                  # ... the last column ...
    z[4, :] = -np.inf
    z[4, 5] = -1e30                      # ... one finite value
    want = oi.sample(z.astype(np.float64), 0.0, 0, np.zeros(6))
    np.testing.assert_array_equal(_sample(z, 0.0, 0, None), want)
    # top_k 1 keeps every copy of the maximum (rows 1 and 2 draw among them); the cumulative sums
    # of equal kept terms are exact in fp32, and u V is far from a cell edge for these V
    u = np.full(6, 0.3719)
    np.testing.assert_array_equal(_sample(z, 0.7, 1, u), oi.sample(z.astype(np.float64), 0.7, 1, u))


@pytest.mark.parametrize("V", [512, 16384, 16385, 65536])
@pytest.mark.parametrize("temperature,top_k", [(1.0, 0), (0.7, 50), (1.3, 7), (0.9, 10**6)])
def test_draws_follow_the_inverse_cdf(V, temperature, top_k):
    rng = np.random.default_rng(V + top_k)
    rows = 64
    z = (rng.standard_normal((rows, V)) * 3).astype(np.float32)
    z[::4] = np.round(z[::4] * 2) / 2          # many equal logits: ties at the top-k threshold
    u = rng.random(rows).astype(np.float32)
    got = _sample(z, temperature, top_k, u)
    want = oi.sample(z.astype(np.float64), temperature, top_k, u.astype(np.float64))
    edge = 0
    for r in range(rows):
        row = z[r].astype(np.float64)
        if 0 < top_k < V:
            kth = np.sort(row)[::-1][top_k - 1]
            row = np.where(row >= kth, row, -np.inf)
        p = np.exp(row / temperature - np.max(row / temperature))
        p /= p.sum()
        c = np.cumsum(p)
        g = int(got[r])
        assert 0 <= g < V and p[g] > 0, (r, g)
        lo = c[g - 1] if g > 0 else 0.0
        assert lo - 2e-5 <= u[r] <= c[g] + 2e-5, (r, g, lo, c[g], u[r])
        near = min(abs(u[r] - lo), abs(u[r] - c[g])) <= 2e-5
        edge += near
        if not near:
            assert g == want[r], (r, g, want[r])
    assert rows - edge >= rows // 2     # most draws are decided exactly


def test_inference_profile_stages():
    """gpt_infer_profile brackets every launch of a decode step: each per-layer stage appears
    once per layer with positive time and work, and reading clears the record."""
    cfg = BF16_SMALL
    _, flat = _model(cfg, 204)
    tok = inputs.uniform_tokens(12, (2, 9), cfg.vocab)
    ctx = B.gpt_infer_init(cfg, 2, 16)
    logits = torch.empty(2, cfg.vocab, device="cuda")
    B.gpt_infer_forward(ctx, flat, dev(tok[:, :8]), logits)
    B.gpt_infer_profile(ctx, True)
    B.gpt_infer_forward(ctx, flat, dev(tok[:, 8:9]), logits)
    B.gpt_infer_profile(ctx, False)
    stages = {n: (c, ms, f, b) for n, c, ms, f, b in B.gpt_infer_profile_read(ctx)}
    L = cfg.n_layer
    per_layer = ("qkv", "rope_append", "attn_split", "attn_combine", "out", "out_resid_norm", "up",
                 "down", "down_resid_norm")
    for name in per_layer:
        calls, ms, flops, nbytes = stages[name]
        assert calls == L and ms > 0 and nbytes > 0, (name, stages[name])
    for name in ("embed", "rmsnorm", "gather_last", "final_norm", "head", "softcap"):
        assert stages[name][0] == 1, name
    assert stages["qkv"][2] == 2.0 * 2 * 3 * cfg.d_model * cfg.d_model * L
    assert B.gpt_infer_profile_read(ctx) == []
    ctx.close()
