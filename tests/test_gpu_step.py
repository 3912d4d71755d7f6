"""GPU parity of the whole training step (gpt_fwd_bwd) against the oracle.

Tolerances: fp32 path loss rel err <= 1e-5 and per-tensor gradient rel-L2 <= 1e-4; bf16 path
loss rel err <= 1e-2, per-tensor gradient rel-L2 <= 3e-2 and cosine >= 0.999.

At full launch sizes the oracle cannot run the whole batch, so only a sample of sequences
carries targets (the rest are -1): sequences are independent and ignored targets contribute
nothing, so the step's loss and every gradient equal the oracle's on those sequences alone.
"""
import math

import numpy as np
import pytest
import torch

from gpt_lm_step_amd import binding as B
from gpt_lm_step_amd import configs, inputs
from oracle import model as om
from oracle import tables as ot

from gpu_util import cosine, dev, host, rel_l2

pytestmark = pytest.mark.gpu


class Step:
    """Device buffers + context for one config."""

    def __init__(self, cfg, params):
        self.cfg = cfg
        self.dtype = torch.bfloat16 if cfg.dtype == configs.BF16 else torch.float32
        self.ctx = B.gpt_init(cfg)
        self.params = dev(inputs.flatten_params(cfg, params), self.dtype)
        self.grads = torch.full((configs.param_elems(cfg),), float("nan"), device="cuda")
        self.loss = torch.zeros(1, device="cuda")
        N, D = cfg.tokens, cfg.d_model
        self.d_x0 = torch.full((N, D), float("nan"), device="cuda", dtype=self.dtype)
        self.d_v = torch.full((N, D), float("nan"), device="cuda", dtype=self.dtype)

    def run(self, tokens, targets, x0=None, va=None, tri=None, grad_scale=1.0, accumulate=0):
        c = self.cfg
        T = c.seq_len
        t_in = dev(np.ascontiguousarray(tokens[:, :T]).astype(np.int32))
        t_tg = dev(np.ascontiguousarray(targets).astype(np.int32))
        add = lambda a: None if a is None else dev(a, self.dtype)
        B.gpt_fwd_bwd(self.ctx, t_in, t_tg, self.params, self.grads, self.loss, grad_scale,
                      accumulate, add(x0), add(va), add(tri),
                      self.d_x0 if c.has_x0_add else None,
                      self.d_v if (c.has_v_add or c.has_trigram) else None)
        torch.cuda.synchronize()
        return float(self.loss.item())

    def grad_dict(self):
        return inputs.unflatten(self.cfg, host(self.grads))


def _compare(cfg, res, step, loss, tol_loss, tol_g, cos_min=None, extra=()):
    assert abs(loss - res.loss) <= tol_loss * abs(res.loss), (loss, res.loss)
    got = step.grad_dict()
    worst = {}
    for name, want in res.grads.items():
        e = rel_l2(got[name], want)
        worst[name] = e
        assert e <= tol_g, (name, e)
        if cos_min is not None:
            assert cosine(got[name], want) >= cos_min, name
    for name, g, want in extra:
        e = rel_l2(g, want)
        assert e <= tol_g, (name, e)
        if cos_min is not None:
            assert cosine(g, want) >= cos_min, name
    return worst


def _tiny(tables, trigram, seed=101):
    cfg = configs.TINY.replace(has_x0_add=int(tables), has_v_add=int(tables),
                               has_trigram=int(trigram))
    params = inputs.model_params(cfg, seed)
    tok = inputs.uniform_tokens(1, (cfg.batch, cfg.seq_len + 1), cfg.vocab)
    N, D = cfg.tokens, cfg.d_model
    x0 = inputs.addend(11, N, D, 0.02, False) if tables else None
    va = inputs.addend(12, N, D, 0.02, False) if tables else None
    tri = inputs.addend(13, N, D, 1.0, False) if trigram else None
    return cfg, params, tok, x0, va, tri


@pytest.mark.parametrize("tables,trigram", [(False, False), (True, False), (True, True)])
def test_tiny_fp32_step_matches_oracle(tables, trigram):
    cfg, params, tok, x0, va, tri = _tiny(tables, trigram)
    step = Step(cfg, params)
    loss = step.run(tok, tok[:, 1:], x0, va, tri)
    res = om.forward_backward(cfg, params, tok, x0, va, tri)
    extra = []
    if tables:
        extra.append(("d_x0_add", host(step.d_x0), res.d_x0_add))
        extra.append(("d_v_add", host(step.d_v), res.d_v_add))
    _compare(cfg, res, step, loss, 1e-5, 1e-4, extra=extra)


def test_tiny_fp32_ignored_targets_scale_and_accumulation():
    cfg, params, tok, _, _, _ = _tiny(False, False)
    tgt = tok[:, 1:].copy()
    tgt[np.random.default_rng(3).random(tgt.shape) < 0.1] = -1
    step = Step(cfg, params)
    loss = step.run(tok, tgt, grad_scale=0.25)
    res = om.forward_backward(cfg, params, tok, targets=tgt, grad_scale=0.25)
    _compare(cfg, res, step, loss, 1e-5, 1e-4)
    # accumulate a second micro-batch with other tokens
    tok2 = inputs.uniform_tokens(2, tok.shape, cfg.vocab)
    step.run(tok2, tok2[:, 1:], grad_scale=0.25, accumulate=1)
    res2 = om.forward_backward(cfg, params, tok2, grad_scale=0.25)
    got = step.grad_dict()
    for name in res.grads:
        assert rel_l2(got[name], res.grads[name] + res2.grads[name]) <= 1e-4, name


def test_tiny_zero_head_loss_is_ln_vocab_and_other_grads_vanish():
    cfg = configs.TINY
    params = inputs.model_params(cfg, 101, zero_head=True)
    tok = inputs.uniform_tokens(1, (cfg.batch, cfg.seq_len + 1), cfg.vocab)
    step = Step(cfg, params)
    loss = step.run(tok, tok[:, 1:])
    assert loss == pytest.approx(math.log(cfg.vocab), rel=1e-6)
    g = step.grad_dict()
    for name, v in g.items():
        if name != "lm_head":
            assert np.all(v == 0.0), name


def test_step_is_bitwise_deterministic():
    cfg, params, tok, x0, va, tri = _tiny(True, True)
    step = Step(cfg, params)
    step.run(tok, tok[:, 1:], x0, va, tri)
    g1, d1 = step.grads.clone(), step.d_v.clone()
    step.run(tok, tok[:, 1:], x0, va, tri)
    assert torch.equal(g1, step.grads) and torch.equal(d1, step.d_v)


def test_workspace_guards_report_an_overwrite():
    """Every buffer of the step's workspace is followed by 256 guard bytes; after a step they are
    intact, and a byte changed in the last guard (the workspace's final 256 bytes) is reported as
    bit 4 by gpt_check_errors, then cleared."""
    cfg, params, tok, x0, va, tri = _tiny(True, True)
    step = Step(cfg, params)
    step.run(tok, tok[:, 1:], x0, va, tri)
    assert B.gpt_check_errors(step.ctx) == 0
    n = B.gpt_workspace_bytes(cfg)
    ws = step.ctx.workspace
    ws[n - 3] = ws[n - 3] ^ 0x40                   # inside the last guard region
    torch.cuda.synchronize()
    assert B.gpt_check_errors(step.ctx) == 4
    ws[n - 3] = ws[n - 3] ^ 0x40
    torch.cuda.synchronize()
    assert B.gpt_check_errors(step.ctx) == 0


def test_out_of_range_ids_are_flagged_not_faulting():
    cfg, params, tok, _, _, _ = _tiny(False, False)
    step = Step(cfg, params)
    bad = tok.copy()
    bad[0, 3] = cfg.vocab + 7
    bad[1, 5] = -4
    tgt = bad[:, 1:].copy()
    tgt[2, 2] = cfg.vocab
    loss = step.run(bad, tgt)
    assert math.isfinite(loss)
    assert B.gpt_check_errors(step.ctx) == 3
    assert B.gpt_check_errors(step.ctx) == 0


def _sampled_targets(tok, T, keep):
    tgt = np.full((tok.shape[0], T), -1, np.int32)
    for b in keep:
        tgt[b] = tok[b, 1:]
    return tgt


def test_gpt2_small_bf16_full_launch_sampled_sequences():
    """GPT-2-small shape at its full launch size (B=8, T=1024, V=50304), Zipf tokens; sequences
    0 and 5 carry targets and are recomputed by the oracle."""
    cfg = configs.GPT2_SMALL
    params = inputs.model_params(cfg, 102)
    tok = inputs.step_tokens(cfg, 2)
    keep = [0, 5]
    step = Step(cfg, params)
    loss = step.run(tok, _sampled_targets(tok, cfg.seq_len, keep))
    sub = cfg.replace(batch=len(keep))
    res = om.forward_backward(sub, params, tok[keep])
    _compare(cfg, res, step, loss, 1e-2, 3e-2, cos_min=0.999)
    assert B.gpt_check_errors(step.ctx) == 0        # no kernel wrote past its buffer


@pytest.mark.parametrize("base", ["speedrun-bf16", "d32-small-batch", "small-chunked"])
def test_weight_gradient_stream_changes_no_bit(base):
    """The blocks' weight-gradient products on a stream of their own give bitwise the results of
    the same step on the caller's stream alone: two micro-batches (overwrite, then accumulate
    with grad_scale 1/2), loss, every gradient and the addend gradients compared bit for bit.
    Shapes: the speedrun micro-batch (GPT-2-small with both table addends and the trigram
    projection, full 8 x 1024 launch), the d32 layer shapes with 4 layers and 2 x 2048 tokens,
    and a small model whose LM head and cross-entropy run in four chunks (the last ragged)."""
    if base == "speedrun-bf16":
        cfg = configs.SPEEDRUN
    elif base == "d32-small-batch":
        cfg = configs.D32.replace(n_layer=4, batch=2)
    else:
        cfg = configs.GPTConfig(n_layer=2, d_model=256, n_head=4, head_dim=64, d_mlp=1024,
                                vocab=4096, seq_len=128, batch=5, dtype=configs.BF16,
                                ce_chunk_tokens=192, has_v_add=1)
    params = inputs.model_params(cfg, 106)
    N, D = cfg.tokens, cfg.d_model
    vadd = cfg.has_v_add or cfg.has_trigram
    adds = [inputs.addend(21 + i, N, D, s, True) if on else None
            for i, (on, s) in enumerate(((cfg.has_x0_add, 0.02), (cfg.has_v_add, 0.02),
                                         (cfg.has_trigram, 1.0)))]
    steps = [Step(cfg.replace(wgrad_stream=w), params) for w in (1, -1)]
    for mb in range(2):
        tok = inputs.step_tokens(cfg, 30 + mb)
        for st in steps:
            st.loss_v = st.run(tok, tok[:, 1:], *adds, grad_scale=0.5, accumulate=mb)
        a, b = steps
        assert a.loss_v == b.loss_v, mb
        assert torch.equal(a.grads, b.grads), mb
        if cfg.has_x0_add:
            assert torch.equal(a.d_x0, b.d_x0), mb
        if vadd:
            assert torch.equal(a.d_v, b.d_v), mb
    assert torch.isfinite(steps[0].grads).all()
    # accumulating a micro-batch onto its own gradient doubles it exactly (x + x is exact in
    # fp32, and every kernel repeats its arithmetic bit for bit): the accumulate epilogues, the
    # paired launch's included, add the stored value once.  A chunked LM head sums its chunks'
    # weight gradients into the stored one, so there the doubling holds to rounding only.
    st = steps[0]
    tok = inputs.step_tokens(cfg, 40)
    st.run(tok, tok[:, 1:], *adds, grad_scale=0.5, accumulate=0)
    once = st.grad_dict()
    st.run(tok, tok[:, 1:], *adds, grad_scale=0.5, accumulate=1)
    twice = st.grad_dict()
    chunked = 0 < cfg.ce_chunk_tokens < cfg.tokens
    for name, g in once.items():
        if chunked and name == "lm_head":
            assert rel_l2(twice[name], 2 * g) <= 1e-6, name
        else:
            assert np.array_equal(twice[name], 2 * g), name


@pytest.mark.timeout(900)
def test_d32_bf16_full_launch_one_full_sequence():
    """The d32 step at the size the bench times (B=8, T=2048, V=65536, 32 layers, device-drawn
    N(0,0.02) bf16 weights, Zipf tokens) with targets on all 2048 positions of one sequence and
    none elsewhere: the loss and every gradient equal the oracle's on that sequence alone.  The
    oracle runs in fp32 storage (its error, ~1e-6 relative, is far below the bf16 bar) so that
    it finishes in about a minute on 16 host cores."""
    cfg = configs.D32
    T, b0 = cfg.seq_len, 5
    flat = inputs.device_params(cfg, 103)
    tok = inputs.step_tokens(cfg, 3)
    tgt = np.full((cfg.batch, T), -1, np.int32)
    tgt[b0] = tok[b0, 1:]
    ctx = B.gpt_init(cfg)
    grads = torch.full((configs.param_elems(cfg),), float("nan"), device="cuda")
    loss_t = torch.zeros(1, device="cuda")
    B.gpt_fwd_bwd(ctx, dev(np.ascontiguousarray(tok[:, :T]).astype(np.int32)), dev(tgt), flat,
                  grads, loss_t, 1.0, 0, None, None, None, None, None)
    torch.cuda.synchronize()
    assert B.gpt_check_errors(ctx) == 0             # no kernel wrote past its buffer
    loss = float(loss_t.item())
    got = inputs.unflatten(cfg, host(grads))
    del grads
    params = inputs.unflatten(cfg, flat.float().cpu().numpy())
    del flat, ctx
    torch.cuda.empty_cache()
    res = om.forward_backward(cfg.replace(batch=1), params, tok[b0:b0 + 1], dtype=np.float32)
    assert abs(loss - res.loss) <= 1e-2 * abs(res.loss), (loss, res.loss)
    for name, want in res.grads.items():
        e = rel_l2(got[name], want)
        assert e <= 3e-2, (name, e)
        assert cosine(got[name], want) >= 0.999, name


def test_tiny_bf16_step_with_tables_matches_oracle():
    """The tiny decoder on the bf16 path (the kernels the bf16 workloads run: DMA-staged GEMMs,
    the pipelined attention backward, bf16 norms and cross-entropy) with all three table
    addends, against the fp64 oracle on the same bf16-rounded inputs."""
    cfg = configs.TINY.replace(dtype=configs.BF16, has_x0_add=1, has_v_add=1, has_trigram=1)
    params = inputs.model_params(cfg, 101)
    tok = inputs.uniform_tokens(1, (cfg.batch, cfg.seq_len + 1), cfg.vocab)
    N, D = cfg.tokens, cfg.d_model
    x0 = inputs.addend(11, N, D, 0.02, True)
    va = inputs.addend(12, N, D, 0.02, True)
    tri = inputs.addend(13, N, D, 1.0, True)
    step = Step(cfg, params)
    loss = step.run(tok, tok[:, 1:], x0, va, tri)
    res = om.forward_backward(cfg, params, tok, x0, va, tri)
    extra = [("d_x0_add", host(step.d_x0), res.d_x0_add), ("d_v_add", host(step.d_v), res.d_v_add)]
    _compare(cfg, res, step, loss, 1e-2, 3e-2, cos_min=0.999, extra=extra)


@pytest.mark.parametrize("accumulate", [0, 1])
def test_tiny_fp32_chunked_head_and_cross_entropy(accumulate):
    """Five sequences (320 tokens) with 128-token LM-head / cross-entropy chunks: chunks of 128,
    128 and a ragged 64, so later chunks add into the head's weight gradient and read targets
    and write losses at their offsets.  Against the oracle (fp32 bar), with ignored targets and
    a grad scale, overwriting and accumulating; against the unchunked step, the loss and every
    gradient but the head's are bit-identical (rows are independent)."""
    cfg = configs.TINY.replace(batch=5, ce_chunk_tokens=128)
    params = inputs.model_params(cfg, 101)
    tok = inputs.uniform_tokens(7, (cfg.batch, cfg.seq_len + 1), cfg.vocab)
    tgt = tok[:, 1:].copy()
    tgt[np.random.default_rng(8).random(tgt.shape) < 0.1] = -1
    step = Step(cfg, params)
    if accumulate:
        step.grads.fill_(0.5)
    loss = step.run(tok, tgt, grad_scale=0.5, accumulate=accumulate)
    res = om.forward_backward(cfg, params, tok, targets=tgt, grad_scale=0.5)
    if accumulate:
        res.grads = {k: v + 0.5 for k, v in res.grads.items()}
    _compare(cfg, res, step, loss, 1e-5, 1e-4)
    whole = Step(cfg.replace(ce_chunk_tokens=0), params)
    if accumulate:
        whole.grads.fill_(0.5)
    loss_w = whole.run(tok, tgt, grad_scale=0.5, accumulate=accumulate)
    assert loss_w == loss
    g_c, g_w = step.grad_dict(), whole.grad_dict()
    for name in g_c:
        if name != "lm_head":
            assert np.array_equal(g_c[name], g_w[name]), name


def test_small_bf16_chunked_head_and_cross_entropy():
    """A small bf16 model (2 layers, d256, 4 heads x 64, vocab 4096, 5 x 128 tokens) with
    192-token chunks: 192, 192, 192 and a ragged 64, against the oracle at the bf16 bar."""
    cfg = configs.GPTConfig(n_layer=2, d_model=256, n_head=4, head_dim=64, d_mlp=1024,
                            vocab=4096, seq_len=128, batch=5, dtype=configs.BF16,
                            ce_chunk_tokens=192)
    params = inputs.model_params(cfg, 111)
    tok = inputs.step_tokens(cfg, 12)
    step = Step(cfg, params)
    loss = step.run(tok, tok[:, 1:])
    res = om.forward_backward(cfg, params, tok)
    _compare(cfg, res, step, loss, 1e-2, 3e-2, cos_min=0.999)


def test_speedrun_microbatch_with_tables_sampled():
    """Speedrun shape: GPT-2-small model + x0 bigram (2^21 rows), value bigram (2^20 rows) and
    the frozen trigram table (2^21 rows, N(0,1)) projected by wtri, one 8 x 1024 micro-batch;
    the addends come from bigram_fwd, the oracle rebuilds them from the same tables."""
    cfg = configs.SPEEDRUN
    tc = configs.TABLES
    params = inputs.model_params(cfg, 102)
    tok = inputs.step_tokens(cfg, 5)
    keep = [3]
    T, N, D = cfg.seq_len, cfg.tokens, cfg.d_model
    g = torch.Generator(device="cuda").manual_seed(104)
    tx0 = (torch.randn(tc.x0_rows, D, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    tv = (torch.randn(tc.v_rows, D, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    ttri = torch.randn(tc.tri_rows, D, device="cuda", generator=g).to(torch.bfloat16)
    t_in = dev(np.ascontiguousarray(tok[:, :T]).astype(np.int32))
    adds = []
    for table, order in ((tx0, 2), (tv, 2), (ttri, 3)):
        y = torch.zeros(N, D, device="cuda", dtype=torch.bfloat16)
        B.bigram_fwd(t_in, order, cfg.vocab, table, y)
        adds.append(y)
    step = Step(cfg, params)
    c = cfg
    B.gpt_fwd_bwd(step.ctx, t_in, dev(_sampled_targets(tok, T, keep)), step.params, step.grads,
                  step.loss, 1.0, 0, adds[0], adds[1], adds[2], step.d_x0, step.d_v)
    torch.cuda.synchronize()
    loss = float(step.loss.item())
    # oracle addends for the kept sequence, from the same tables
    sel = tok[keep, :T]
    rows = []
    for table, order, R in ((tx0, 2, tc.x0_rows), (tv, 2, tc.v_rows), (ttri, 3, tc.tri_rows)):
        h = ot.hash_indices(sel, order, cfg.vocab, R).reshape(-1)
        rows.append(host(table[torch.from_numpy(h).cuda()]))
    sub = cfg.replace(batch=len(keep))
    res = om.forward_backward(sub, params, tok[keep], rows[0], rows[1], rows[2])
    tsl = slice(keep[0] * T, (keep[0] + 1) * T)
    extra = [("d_x0_add", host(step.d_x0)[tsl], res.d_x0_add),
             ("d_v_add", host(step.d_v)[tsl], res.d_v_add)]
    _compare(cfg, res, step, loss, 1e-2, 3e-2, cos_min=0.999, extra=extra)
    # tokens of the other sequences get exactly zero addend gradients
    other = np.ones(N, bool)
    other[tsl] = False
    assert np.all(host(step.d_x0)[other] == 0) and np.all(host(step.d_v)[other] == 0)
