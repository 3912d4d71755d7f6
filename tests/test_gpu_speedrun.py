"""GPU parity of the speedrun-shaped optimizer step, end to end, against the oracle.

The decoder-rtx posts train a GPT-2-small-shaped model with two hashed bigram tables (rows added
to x0 and to the attention values) and a frozen trigram table projected into the values, on a
large batch made of several micro-batches, with the tables' sparse optimizer inlined in the
backward pass.  Here: MB micro-batches of 8 x 1024 tokens, each three bigram_fwd gathers into
zeroed addend buffers and one gpt_fwd_bwd with grad_scale = 1/MB accumulating into the same
dense gradients (accumulate = 1 after the first), the per-token addend gradients staged into
[MB * 8192, 768] bf16 slabs, then one bigram_bwd_update per table over every token of the step.

In each micro-batch one sequence carries targets (the others are -1), so the oracle recomputes
only those sequences; every other token's addend gradient is exactly zero, and a table row hit
only by such tokens keeps its weights and its zero second moment.  bf16 bar: loss rel <= 1e-2,
every dense gradient, both addend-gradient slabs, both tables' updates (new minus old weights of
the touched rows) and their second moments rel-L2 <= 3e-2 with cosine >= 0.999.
"""
import numpy as np
import pytest
import torch

from gpt_lm_step_amd import binding as B
from gpt_lm_step_amd import configs, inputs
from oracle import model as om
from oracle import tables as ot

from gpu_util import cosine, dev, host, rel_l2

pytestmark = pytest.mark.gpu

BF = torch.bfloat16


def _close(name, got, want, tol=3e-2, cos_min=0.999):
    e = rel_l2(got, want)
    assert e <= tol, (name, e)
    assert cosine(got, want) >= cos_min, (name, cosine(got, want))


@pytest.mark.timeout(600)
def test_speedrun_accumulated_step_with_table_updates():
    cfg = configs.SPEEDRUN
    tc = configs.TABLES
    MB = 3
    keep = [3, 6, 1]                      # the sequence of each micro-batch that has targets
    T, N, D, V = cfg.seq_len, cfg.tokens, cfg.d_model, cfg.vocab
    params = inputs.model_params(cfg, 102)
    toks = [inputs.step_tokens(cfg, 50 + m) for m in range(MB)]
    g = torch.Generator(device="cuda").manual_seed(104)
    tx0 = (torch.randn(tc.x0_rows, D, device="cuda", generator=g) * 0.02).to(BF)
    tv = (torch.randn(tc.v_rows, D, device="cuda", generator=g) * 0.02).to(BF)
    ttri = torch.randn(tc.tri_rows, D, device="cuda", generator=g).to(BF)
    tx0_0, tv_0 = tx0.clone(), tv.clone()
    vx0 = torch.zeros(tc.x0_rows, device="cuda")
    vv = torch.zeros(tc.v_rows, device="cuda")

    ctx = B.gpt_init(cfg)
    flat = dev(inputs.flatten_params(cfg, params), BF)
    grads = torch.full((configs.param_elems(cfg),), float("nan"), device="cuda")
    loss_t = torch.zeros(1, device="cuda")
    slab_x0 = torch.full((MB * N, D), float("nan"), device="cuda", dtype=BF)
    slab_v = torch.full((MB * N, D), float("nan"), device="cuda", dtype=BF)
    h_x0 = torch.full((MB * N,), -1, device="cuda", dtype=torch.int32)
    h_v = torch.full((MB * N,), -1, device="cuda", dtype=torch.int32)
    losses = []
    for m in range(MB):
        tok = toks[m]
        t_in = dev(np.ascontiguousarray(tok[:, :T]).astype(np.int32))
        tgt = np.full((cfg.batch, T), -1, np.int32)
        tgt[keep[m]] = tok[keep[m], 1:]
        adds = []
        for table, order, h_out in ((tx0, 2, h_x0[m * N:(m + 1) * N]),
                                    (tv, 2, h_v[m * N:(m + 1) * N]), (ttri, 3, None)):
            y = torch.zeros(N, D, device="cuda", dtype=BF)
            B.bigram_fwd(t_in, order, V, table, y, h_out)
            adds.append(y)
        B.gpt_fwd_bwd(ctx, t_in, dev(tgt), flat, grads, loss_t, 1.0 / MB, int(m > 0),
                      adds[0], adds[1], adds[2], slab_x0[m * N:(m + 1) * N],
                      slab_v[m * N:(m + 1) * N])
        torch.cuda.synchronize()
        losses.append(float(loss_t.item()))
    B.bigram_bwd_update(h_x0, slab_x0, tx0, vx0, tc.lr)
    B.bigram_bwd_update(h_v, slab_v, tv, vv, tc.lr)
    torch.cuda.synchronize()
    assert B.gpt_check_errors(ctx) == 0             # no kernel wrote past its buffer

    # ---- oracle: the kept sequences, their addends rebuilt from the same (initial) tables
    want_g = None
    d_x0_all = np.zeros((MB * N, D))
    d_v_all = np.zeros((MB * N, D))
    for m in range(MB):
        b = keep[m]
        sel = toks[m][b:b + 1]
        rows = []
        for table, order, R in ((tx0_0, 2, tc.x0_rows), (tv_0, 2, tc.v_rows),
                                (ttri, 3, tc.tri_rows)):
            h = ot.hash_indices(sel[:, :T], order, V, R).reshape(-1)
            rows.append(host(table[torch.from_numpy(h).cuda()]))
        res = om.forward_backward(cfg.replace(batch=1), params, sel, rows[0], rows[1], rows[2],
                                  grad_scale=1.0 / MB)
        assert abs(losses[m] - res.loss) <= 1e-2 * abs(res.loss), (m, losses[m], res.loss)
        want_g = res.grads if want_g is None else {k: want_g[k] + res.grads[k] for k in want_g}
        tsl = slice(m * N + b * T, m * N + (b + 1) * T)
        d_x0_all[tsl] = res.d_x0_add
        d_v_all[tsl] = res.d_v_add
        print(f"micro-batch {m}: loss {losses[m]:.5f} (oracle {res.loss:.5f})", flush=True)

    got_g = inputs.unflatten(cfg, host(grads))
    for name, want in want_g.items():
        _close(name, got_g[name], want)
    got_x0, got_v = host(slab_x0), host(slab_v)
    live = np.zeros(MB * N, bool)
    for m in range(MB):
        live[m * N + keep[m] * T:m * N + (keep[m] + 1) * T] = True
    _close("d_x0_add", got_x0[live], d_x0_all[live])
    _close("d_v_add", got_v[live], d_v_all[live])
    assert np.all(got_x0[~live] == 0) and np.all(got_v[~live] == 0)

    # ---- both table updates over every token of the step (rows are independent)
    all_tok = np.concatenate([t[:, :T] for t in toks], axis=0)
    for name, t0, t1, v1, R, dy in (("x0", tx0_0, tx0, vx0, tc.x0_rows, d_x0_all),
                                    ("value", tv_0, tv, vv, tc.v_rows, d_v_all)):
        h = ot.hash_indices(all_tok, 2, V, R).reshape(-1)
        assert np.array_equal(host(h_x0 if name == "x0" else h_v).astype(np.int64), h), name
        rows, inv = np.unique(h, return_inverse=True)
        t_rows = torch.from_numpy(rows).cuda()
        w0 = host(t0[t_rows]).astype(np.float64)
        w_want, v_want, _ = ot.sparse_row_update(w0, np.zeros(len(rows)), inv, dy, tc.lr)
        w_got = host(t1[t_rows]).astype(np.float64)
        v_got = host(v1[t_rows]).astype(np.float64)
        hit = np.zeros(len(rows), bool)
        hit[np.unique(inv[live])] = True           # rows some kept token reached
        _close(f"{name} table update", (w_got - w0)[hit], (w_want - w0)[hit])
        _close(f"{name} second moment", v_got[hit], v_want[hit])
        # rows reached only by tokens without targets: zero gradient, nothing moves
        assert np.array_equal(w_got[~hit], w0[~hit]) and np.all(v_got[~hit] == 0), name
        mask = torch.ones(R, dtype=torch.bool, device="cuda")
        mask[t_rows] = False
        assert torch.equal(t1[mask], t0[mask]) and torch.count_nonzero(v1[mask]) == 0, name
