"""GPU parity of the hashed n-gram tables (bigram_fwd, bigram_bwd_update) against the oracle."""
import numpy as np
import pytest
import torch

from gpt_lm_step_amd import binding as B
from gpt_lm_step_amd import configs, inputs
from oracle import tables as ot

from gpu_util import (bf16_bits, bf16_bits_to_f64, bf16_ulp_distance, dev, host,
                      oracle_bf16_bits, table_update_bound)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("order,rows,dtype", [(2, 4096, torch.bfloat16), (2, 5003, torch.bfloat16),
                                              (3, 4096, torch.bfloat16), (3, 7919, torch.float32)])
def test_bigram_fwd_hash_and_pure_gather_bit_exact(order, rows, dtype):
    Bn, T, V, D = 3, 100, 1000, 64
    tok = inputs.uniform_tokens(31, (Bn, T), V)
    table = inputs.normal(32, (rows, D), 0.02, dtype == torch.bfloat16)
    t_tok, t_tab = dev(tok), dev(table, dtype)
    y = torch.zeros(Bn * T, D, device="cuda", dtype=dtype)
    h = torch.full((Bn * T,), -7, device="cuda", dtype=torch.int32)
    B.bigram_fwd(t_tok, order, V, t_tab, y, h)
    torch.cuda.synchronize()
    want_h = ot.hash_indices(tok, order, V, rows).reshape(-1)
    assert np.array_equal(host(h).astype(np.int64), want_h)
    # y = 0 + row: a pure gather, bit for bit
    assert torch.equal(y, t_tab[torch.from_numpy(want_h).cuda()])


def test_bigram_fwd_adds_into_y_within_one_ulp():
    Bn, T, V, D, R = 2, 64, 300, 128, 1 << 12
    tok = inputs.uniform_tokens(33, (Bn, T), V)
    table = inputs.normal(34, (R, D), 0.02, True)
    y0 = inputs.normal(35, (Bn * T, D), 1.0, True)
    y = dev(y0, torch.bfloat16)
    B.bigram_fwd(dev(tok), 2, V, dev(table, torch.bfloat16), y)
    h = ot.hash_indices(tok, 2, V, R).reshape(-1)
    want = ot.gather_add(y0, table, h)
    assert bf16_ulp_distance(bf16_bits(y), oracle_bf16_bits(want)).max() <= 1


def test_bigram_fwd_tables_workload_sampled():
    """196,608 Zipf(1.1) tokens (192 x 1024) over V = 50304, the 2^21 x 768 bf16 table."""
    tc = configs.TABLES
    tok = inputs.zipf_tokens(4, (tc.n_tokens // tc.seq_len, tc.seq_len), tc.vocab)
    g = torch.Generator(device="cuda").manual_seed(104)
    table = (torch.randn(tc.x0_rows, tc.dim, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    y = torch.zeros(tc.n_tokens, tc.dim, device="cuda", dtype=torch.bfloat16)
    h = torch.empty(tc.n_tokens, device="cuda", dtype=torch.int32)
    B.bigram_fwd(dev(tok), 2, tc.vocab, table, y, h)
    want_h = ot.hash_indices(tok, 2, tc.vocab, tc.x0_rows).reshape(-1)
    assert np.array_equal(host(h).astype(np.int64), want_h)
    sample = np.random.default_rng(0).choice(tc.n_tokens, 4096, replace=False)
    rows = bf16_bits(table[torch.from_numpy(want_h[sample]).cuda()])
    assert np.array_equal(bf16_bits(y[torch.from_numpy(sample).cuda()]), rows)


def _oracle_update(table_np, v_np, h, dy_np, lr):
    """Oracle update restricted to the rows h touches (rows are independent)."""
    valid = (h >= 0) & (h < table_np.shape[0])
    rows, inv = np.unique(h[valid], return_inverse=True)
    w_sub, v_sub, _ = ot.sparse_row_update(table_np[rows], v_np[rows], inv, dy_np[valid], lr)
    return rows, w_sub, v_sub


def _check_rows(got_bits, w0, want, v_want, dy, h, lr):
    """Updated bf16 rows within the fp32 error bound of the oracle (see table_update_bound);
    most elements are identical."""
    valid = (h >= 0) & (h < np.iinfo(np.int32).max)
    rows, h_local = np.unique(h[valid], return_inverse=True)
    step = lr / (np.sqrt(v_want) + 1e-8)
    bound = table_update_bound(w0, want, dy[valid], h_local, step)
    err = np.abs(bf16_bits_to_f64(got_bits) - want)
    assert np.all(err <= bound), float(np.max(err / bound))
    assert np.mean(bf16_ulp_distance(got_bits, oracle_bf16_bits(want)) == 0) > 0.99


def _run_update(table, v, h, dy, lr):
    B.bigram_bwd_update(h, dy, table, v, lr)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 64), (torch.bfloat16, 768), (torch.float32, 136)])
def test_bwd_update_matches_oracle(dtype, D):
    rng = np.random.default_rng(40)
    R, n = 5003, 3000
    h = rng.integers(0, 400, n).astype(np.int32)
    h[:700] = 17                 # one segment far longer than a chunk (several partials)
    h[700:740] = 4999            # a segment of 40 tokens (two chunks)
    rng.shuffle(h)
    bf = dtype == torch.bfloat16
    table0 = inputs.normal(41, (R, D), 0.02, bf)
    v0 = np.abs(rng.standard_normal(R)).astype(np.float32) * 0.01
    dy0 = inputs.normal(42, (n, D), 1.0, bf)
    table, v = dev(table0, dtype), dev(v0)
    _run_update(table, v, dev(h), dev(dy0, dtype), lr=1e-2)
    rows, w_want, v_want = _oracle_update(table0.astype(np.float64), v0.astype(np.float64), h,
                                          dy0.astype(np.float64), 1e-2)
    v_got = host(v)
    np.testing.assert_allclose(v_got[rows], v_want, rtol=1e-5)
    untouched = np.setdiff1d(np.arange(R), rows)
    assert np.array_equal(v_got[untouched], v0[untouched])
    if bf:
        got_bits = bf16_bits(table)
        _check_rows(got_bits[rows], table0[rows].astype(np.float64), w_want, v_want,
                    dy0.astype(np.float64), h, 1e-2)
        assert np.array_equal(got_bits[untouched], inputs.f32_to_bf16_bits(table0[untouched]))
    else:
        got = host(table)
        np.testing.assert_allclose(got[rows], w_want, rtol=1e-5, atol=1e-7)
        assert np.array_equal(got[untouched], table0[untouched])


def test_bwd_update_skips_out_of_range_rows_and_is_deterministic():
    rng = np.random.default_rng(43)
    R, D, n = 1000, 64, 2000
    h = rng.integers(-5, R + 5, n).astype(np.int32)
    h[::50] = 3
    table0 = inputs.normal(44, (R, D), 0.02, True)
    dy0 = inputs.normal(45, (n, D), 1.0, True)
    outs = []
    for _ in range(2):
        table, v = dev(table0, torch.bfloat16), torch.zeros(R, device="cuda")
        _run_update(table, v, dev(h), dev(dy0, torch.bfloat16), lr=3e-2)
        outs.append((bf16_bits(table), host(v)))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    rows, w_want, v_want = _oracle_update(table0.astype(np.float64), np.zeros(R), h,
                                          dy0.astype(np.float64), 3e-2)
    np.testing.assert_allclose(outs[0][1][rows], v_want, rtol=1e-5)
    hv = np.where((h >= 0) & (h < R), h, -1)
    keep = hv >= 0
    _check_rows(outs[0][0][rows], table0[rows].astype(np.float64), w_want, v_want,
                dy0[keep].astype(np.float64), hv[keep], 3e-2)


def test_bwd_update_empty_is_noop():
    table = torch.ones(10, 64, device="cuda", dtype=torch.bfloat16)
    v = torch.zeros(10, device="cuda")
    e = torch.empty(0, device="cuda", dtype=torch.int32)
    B.bigram_bwd_update(e, torch.empty(0, 64, device="cuda", dtype=torch.bfloat16), table, v, 0.1)
    torch.cuda.synchronize()
    assert torch.all(table == 1) and torch.all(v == 0)


@pytest.mark.parametrize("which", ["x0", "value"])
def test_bwd_update_tables_workload(which):
    """Tables workload: 196,608 Zipf tokens hashed into the 2^21-row x0 table or the 2^20-row
    value table, dy ~ N(0,1) bf16, lr 1e-2; every touched row checked against the oracle,
    untouched rows bitwise unchanged."""
    tc = configs.TABLES
    R = tc.x0_rows if which == "x0" else tc.v_rows
    tok = inputs.zipf_tokens(4, (tc.n_tokens // tc.seq_len, tc.seq_len), tc.vocab)
    h = ot.hash_indices(tok, 2, tc.vocab, R).reshape(-1).astype(np.int32)
    dy0 = inputs.normal(204 if which == "x0" else 205, (tc.n_tokens, tc.dim), 1.0, True)
    g = torch.Generator(device="cuda").manual_seed(104 if which == "x0" else 106)
    table = (torch.randn(R, tc.dim, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    before = table.clone()
    v = torch.zeros(R, device="cuda")
    _run_update(table, v, dev(h), dev(dy0, torch.bfloat16), tc.lr)
    rows = np.unique(h)
    t_rows = torch.from_numpy(rows).cuda()
    w0 = host(before[t_rows]).astype(np.float64)
    r2, w_want, v_want = _oracle_update(w0, np.zeros(len(rows)),
                                        np.searchsorted(rows, h), dy0.astype(np.float64), tc.lr)
    assert np.array_equal(r2, np.arange(len(rows)))
    np.testing.assert_allclose(host(v[t_rows]), v_want, rtol=1e-5)
    _check_rows(bf16_bits(table[t_rows]), w0, w_want, v_want, dy0.astype(np.float64), h, tc.lr)
    mask = torch.ones(R, dtype=torch.bool, device="cuda")
    mask[t_rows] = False
    assert torch.equal(table[mask], before[mask])
    assert torch.count_nonzero(v[mask]) == 0
