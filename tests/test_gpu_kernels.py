"""GPU parity of each stage of the step (GEMM layouts, RMSNorm, rotary + QK-norm, attention,
softcapped cross-entropy) against the oracle's primitives, through the per-kernel C ABI."""
import math

import numpy as np
import pytest
import torch

from gpt_lm_step_amd import binding as B
from gpt_lm_step_amd import inputs
from oracle import model as om

from gpu_util import dev, host, rel_l2

pytestmark = pytest.mark.gpu

BF, F32 = torch.bfloat16, torch.float32


def _operand(rng_seed, rows, K, kc, dtype):
    """Random (rows x K) logical operand and its device storage in the requested layout."""
    a = inputs.normal(rng_seed, (rows, K), 1.0, dtype == BF)
    stored = a if kc else np.ascontiguousarray(a.T)
    return a, dev(stored, dtype)


@pytest.mark.parametrize("dtype", [BF, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("a_kc,b_kc", [(1, 1), (1, 0), (0, 0), (0, 1)])
@pytest.mark.parametrize("M,N,K", [(256, 384, 128), (200, 136, 72), (8, 8, 8), (392, 520, 1032)])
def test_gemm_layouts(dtype, a_kc, b_kc, M, N, K):
    a, ta = _operand(1, M, K, a_kc, dtype)
    b, tb = _operand(2, N, K, b_kc, dtype)
    lda = K if a_kc else M
    ldb = K if b_kc else N
    c = torch.full((M, N), float("nan"), device="cuda")
    B.gptk_gemm(a_kc, b_kc, M, N, K, ta, lda, tb, ldb, c, N, beta=0)
    want = a.astype(np.float64) @ b.astype(np.float64).T
    tol = 1e-5
    assert rel_l2(host(c), want) < tol
    # beta = 1 accumulates
    B.gptk_gemm(a_kc, b_kc, M, N, K, ta, lda, tb, ldb, c, N, beta=1)
    assert rel_l2(host(c), 2 * want) < tol


@pytest.mark.parametrize("a_kc,b_kc", [(1, 1), (1, 0), (0, 0), (0, 1)])
def test_gemm_big_tile_ragged(a_kc, b_kc):
    """A tiling that selects the large-tile kernel (255 tiles of 256 x 256 fill one round), with
    ragged M, N and K tails."""
    M, N, K = 4104, 3592, 264
    a, ta = _operand(21, M, K, a_kc, BF)
    b, tb = _operand(22, N, K, b_kc, BF)
    c = torch.full((M, N), float("nan"), device="cuda")
    B.gptk_gemm(a_kc, b_kc, M, N, K, ta, K if a_kc else M, tb, K if b_kc else N, c, N)
    want = a.astype(np.float64) @ b.astype(np.float64).T
    assert rel_l2(host(c), want) < 1e-5


def test_gemm_large_square_bf16():
    M = N = K = 2048
    a, ta = _operand(3, M, K, 1, BF)
    b, tb = _operand(4, N, K, 1, BF)
    c = torch.empty(M, N, device="cuda")
    B.gptk_gemm(1, 1, M, N, K, ta, K, tb, K, c, N)
    want = a.astype(np.float64) @ b.astype(np.float64).T
    assert rel_l2(host(c), want) < 2e-6


@pytest.mark.parametrize("a_kc,b_kc,M,N,K,splits", [
    (0, 0, 768, 768, 8192, 4),      # measured plan: 128 tiles, 4 splits (GPT-2-small out proj.)
    (0, 0, 2304, 768, 8192, 4),     # measured plan: 128 tiles, 4 splits (GPT-2-small q/k/v)
    (0, 0, 2048, 2048, 16384, 4),   # measured plan: 256 tiles, 4 splits (d32 out proj.)
    (0, 0, 640, 640, 8192, 16),     # general rule: 128 tiles, 16 splits
    (0, 0, 2560, 1536, 16384, 8),   # general rule: 256 tiles, 8 splits
    (1, 0, 392, 520, 4104, 8),      # ragged M, N and a last split shorter than the others
    (0, 1, 264, 136, 2056, 4),
    (1, 1, 256, 384, 128, 1),       # too short to split
])
def test_gemm_wgrad_split_k(a_kc, b_kc, M, N, K, splits):
    """Split-K weight-gradient GEMM against fp64, overwrite then accumulate; the plan's split
    count is the one the step uses for such shapes."""
    need = B.gptk_gemm_wgrad_ws_floats(M, N, K)
    assert need == (splits * M * N if splits > 1 else 0)
    a, ta = _operand(41, M, K, a_kc, BF)
    b, tb = _operand(42, N, K, b_kc, BF)
    lda, ldb = (K if a_kc else M), (K if b_kc else N)
    ws = torch.full((max(need, 4),), float("nan"), device="cuda")
    c = torch.full((M, N), float("nan"), device="cuda")
    B.gptk_gemm_wgrad(a_kc, b_kc, M, N, K, ta, lda, tb, ldb, c, N, beta=0, ws=ws)
    want = a.astype(np.float64) @ b.astype(np.float64).T
    assert rel_l2(host(c), want) < 1e-5
    B.gptk_gemm_wgrad(a_kc, b_kc, M, N, K, ta, lda, tb, ldb, c, N, beta=1, ws=ws)
    assert rel_l2(host(c), 2 * want) < 1e-5
    if need:
        small = torch.empty(need - 4, device="cuda")
        with pytest.raises(B.GptError):
            B.gptk_gemm_wgrad(a_kc, b_kc, M, N, K, ta, lda, tb, ldb, c, N, ws=small)


@pytest.mark.parametrize("dtype", [BF, F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128, 768, 2048])
def test_rmsnorm_fwd_bwd(dtype, D):
    N = 300
    x = inputs.normal(5, (N, D), 2.0, False)
    dy = inputs.normal(6, (N, D), 1.0, False)
    dres = inputs.normal(7, (N, D), 1.0, False)
    tx = dev(x)
    y = torch.empty(N, D, device="cuda", dtype=dtype)
    r = torch.empty(N, device="cuda")
    B.gptk_rmsnorm_fwd(tx, y, r, 1e-6)
    y_want, r_want = om.rms_norm(x.astype(np.float64), 1e-6)
    np.testing.assert_allclose(host(r), r_want, rtol=2e-6)
    assert rel_l2(host(y), y_want) < (3e-3 if dtype == BF else 1e-6)
    dx = dev(dres)
    dx_t = torch.empty(N, D, device="cuda", dtype=dtype)
    B.gptk_rmsnorm_bwd(tx, dev(r_want.astype(np.float32)), dev(dy), dx, dx, dx_t)
    want = dres + om.rms_norm_bwd(y_want, r_want, dy.astype(np.float64))
    assert rel_l2(host(dx), want) < 1e-6
    assert rel_l2(host(dx_t), want) < (3e-3 if dtype == BF else 1e-6)


@pytest.mark.parametrize("dtype,hd", [(BF, 64), (BF, 128), (F32, 32), (BF, 32)])
def test_rope_qknorm_fwd_bwd(dtype, hd):
    Bn, T, H = 2, 128, 3
    D, N = H * hd, 2 * 128
    bf = dtype == BF
    qkv0 = inputs.normal(8, (N, 3 * D), 1.0, bf)
    cos = torch.empty(T, hd // 2, device="cuda", dtype=dtype)
    sin = torch.empty_like(cos)
    B.gptk_rope_table(cos, sin, T, hd, 10000.0)
    c64, s64 = om.rope_tables(T, hd, 10000.0)
    # the tables the kernels use: fp64 values rounded once to the storage type
    cq = (inputs.round_bf16(c64.astype(np.float32)) if bf else c64.astype(np.float32))
    sq = (inputs.round_bf16(s64.astype(np.float32)) if bf else s64.astype(np.float32))
    assert np.array_equal(host(cos), cq) and np.array_equal(host(sin), sq)
    cq, sq = cq.astype(np.float64), sq.astype(np.float64)
    qkv = dev(qkv0, dtype)
    rstd = torch.empty(N, 2 * H, device="cuda")
    B.gptk_rope_qknorm_fwd(qkv, cos, sin, rstd, T, H, hd, 1, 1e-6)
    x = qkv0.astype(np.float64)
    q = x[:, :D].reshape(Bn, T, H, hd)
    k = x[:, D:2 * D].reshape(Bn, T, H, hd)
    qn, rq = om.rms_norm(om.rope(q, cq, sq), 1e-6)
    kn, rk = om.rms_norm(om.rope(k, cq, sq), 1e-6)
    got = host(qkv)
    tol = 4e-3 if bf else 1e-6
    assert rel_l2(got[:, :D], qn.reshape(N, D)) < tol
    assert rel_l2(got[:, D:2 * D], kn.reshape(N, D)) < tol
    assert np.array_equal(got[:, 2 * D:], qkv0[:, 2 * D:])        # v untouched
    np.testing.assert_allclose(host(rstd)[:, :H], rq.reshape(N, H), rtol=1e-5)
    np.testing.assert_allclose(host(rstd)[:, H:], rk.reshape(N, H), rtol=1e-5)
    # backward, fed with the oracle's forward results (saved normalized q/k and their rstd)
    saved = qkv0.copy()
    saved[:, :D] = qn.reshape(N, D)
    saved[:, D:2 * D] = kn.reshape(N, D)
    if bf:
        saved = inputs.round_bf16(saved.astype(np.float32))
    r = np.concatenate([rq.reshape(N, H), rk.reshape(N, H)], 1).astype(np.float32)
    dq = inputs.normal(9, (N, 3 * D), 1.0, bf)
    tdq = dev(dq, dtype)
    B.gptk_rope_qknorm_bwd(tdq, dev(saved, dtype), cos, sin, dev(r), T, H, hd, 1)
    y = saved.astype(np.float64)
    for blk in (0, 1):
        yy = y[:, blk * D:(blk + 1) * D].reshape(Bn, T, H, hd)
        rr = r[:, blk * H:(blk + 1) * H].astype(np.float64).reshape(Bn, T, H)
        dd = dq[:, blk * D:(blk + 1) * D].astype(np.float64).reshape(Bn, T, H, hd)
        want = om.rope_bwd(om.rms_norm_bwd(yy, rr, dd), cq, sq).reshape(N, D)
        assert rel_l2(host(tdq)[:, blk * D:(blk + 1) * D], want) < tol


@pytest.mark.parametrize("dtype", [BF, F32], ids=["bf16", "f32"])
def test_rope_table_worked_values(dtype):
    """gptk_rope_table at frequency indices i >= 1 against hand-worked angles t * 10000^(-2i/hd):
    hd 32, i 8 -> 0.01 per position (t 3: angle 0.03); hd 32, i 4 -> 0.1 (t 5: 0.5); hd 64,
    i 16 -> 0.01 (t 3: 0.03); each value rounded once to the storage type."""
    cases = [(32, 8, 3, 0.99955003374898754, 0.029995500202495660),
             (32, 4, 5, 0.87758256189037276, 0.47942553860420301),
             (64, 16, 3, 0.99955003374898754, 0.029995500202495660)]
    for hd, i, t, c, s in cases:
        cos = torch.empty(8, hd // 2, device="cuda", dtype=dtype)
        sin = torch.empty_like(cos)
        B.gptk_rope_table(cos, sin, 8, hd, 10000.0)
        if dtype == BF:
            rnd = lambda x: inputs.round_bf16(np.array([x], np.float32))[0]
        else:
            rnd = np.float32
        assert host(cos)[t, i] == rnd(c), (hd, i, t)
        assert host(sin)[t, i] == rnd(s), (hd, i, t)


def _attn_case(dtype, Bn, T, H, hd, seed):
    D = H * hd
    bf = dtype == BF
    qkv = inputs.normal(seed, (Bn * T, 3 * D), 1.0, bf)
    # QK-normed q and k have unit RMS; scale like that so softmax is not saturated
    return qkv


def _heads(x, Bn, T, H, hd, blk):
    D = H * hd
    return x[:, blk * D:(blk + 1) * D].reshape(Bn, T, H, hd).transpose(0, 2, 1, 3)


def _check_attention(dtype, hd, T, Bn, H, qkv0):
    """Forward (out, LSE) and backward (dq, dk, dv) of the kernels against the oracle on the
    same stored inputs; the backward is fed the oracle's forward results, not the GPU's."""
    D, N = H * hd, Bn * T
    bf = dtype == BF
    tq = dev(qkv0, dtype)
    out = torch.empty(N, D, device="cuda", dtype=dtype)
    lse2 = torch.empty(Bn, H, T, device="cuda")
    B.gptk_attention_fwd(tq, out, lse2, Bn, T, H, hd)
    x = qkv0.astype(np.float64)
    q, k, v = (_heads(x, Bn, T, H, hd, i) for i in range(3))
    o, p = om.causal_attention(q, k, v)
    o_tok = o.transpose(0, 2, 1, 3).reshape(N, D)
    tol = 1e-2 if bf else 1e-5
    assert rel_l2(host(out), o_tok) < tol
    s = (q @ k.transpose(0, 1, 3, 2)) / math.sqrt(hd)
    s = np.where(np.triu(np.ones((T, T), bool), 1), -np.inf, s)
    m = s.max(-1)
    lse = m + np.log(np.exp(s - m[..., None]).sum(-1))
    np.testing.assert_allclose(host(lse2) * math.log(2), lse, rtol=0, atol=(2e-3 if bf else 1e-5))
    # backward, fed with the oracle's forward results (O rounded to the storage type, LSE)
    do = inputs.normal(11, (N, D), 1.0, bf)
    o_in = inputs.round_bf16(o_tok.astype(np.float32)) if bf else o_tok.astype(np.float32)
    dqkv = torch.full((N, 3 * D), float("nan"), device="cuda", dtype=dtype)
    scratch = torch.empty(Bn * H * T, device="cuda")
    B.gptk_attention_bwd(tq, dev(o_in, dtype), dev(do, dtype),
                         dev((lse / math.log(2)).astype(np.float32)), scratch, dqkv, Bn, T, H, hd)
    o_h = o_in.astype(np.float64).reshape(Bn, T, H, hd).transpose(0, 2, 1, 3)
    do_h = do.astype(np.float64).reshape(Bn, T, H, hd).transpose(0, 2, 1, 3)
    dq, dk, dv = om.causal_attention_bwd(q, k, v, p, o_h, do_h)
    got = host(dqkv)
    for i, want in enumerate((dq, dk, dv)):
        w = want.transpose(0, 2, 1, 3).reshape(N, D)
        assert rel_l2(got[:, i * D:(i + 1) * D], w) < (2e-2 if bf else 1e-5), i
    return s


@pytest.mark.parametrize("dtype,hd,T,Bn,H", [(BF, 64, 256, 2, 3), (BF, 128, 192, 2, 3),
                                              (BF, 32, 64, 2, 3), (F32, 32, 128, 2, 3),
                                              (F32, 64, 64, 2, 3),
                                              # >= 512 workgroups: 64 queries per wave
                                              (BF, 128, 512, 16, 16),
                                              # the d32 sequence length and head size
                                              (BF, 128, 2048, 1, 2)])
def test_attention_fwd_bwd(dtype, hd, T, Bn, H):
    _check_attention(dtype, hd, T, Bn, H, _attn_case(dtype, Bn, T, H, hd, 10))


@pytest.mark.parametrize("dtype,hd,T", [(BF, 128, 512), (BF, 64, 512), (BF, 128, 1024),
                                        (F32, 64, 256), (F32, 32, 256)])
def test_attention_scores_rising_along_the_sequence(dtype, hd, T):
    """Keys whose scores rise by ~6 log2 units per 64-key tile: every row's running maximum
    keeps growing, so the forward's softmax reference maximum (which lags the true maximum
    until a row's weights would exceed 2^8) must be raised again after the first tile, with a
    rescale factor strictly between 0 and 1, several times per row at T >= 512.  q_t[0] = 4 and
    k_s[0] = kappa * s on top of N(0, 1) entries, kappa = 6 sqrt(hd) / (64 * 4 * log2 e)."""
    Bn, H = 2, 2
    D = H * hd
    bf = dtype == BF
    qkv0 = inputs.normal(15, (Bn * T, 3 * D), 1.0, False)
    kappa = 6.0 * math.sqrt(hd) / (64 * 4.0 * math.log2(math.e))
    pos = np.tile(np.arange(T), Bn).astype(np.float64)
    for h in range(H):
        qkv0[:, h * hd] = 4.0
        qkv0[:, D + h * hd] = kappa * pos
    if bf:
        qkv0 = inputs.round_bf16(qkv0)
    s = _check_attention(dtype, hd, T, Bn, H, qkv0)
    # the inputs do what they are meant to: from the fourth tile on, every query's running
    # maximum exceeds its maximum over the first tile by more than 8 log2 units (so every wave
    # rescales after its first tile), and the last rows by more than 3 * 8 when T >= 512
    l2e = math.log2(math.e)
    for t in range(192, T, 7):
        grow = (s[..., t, :t + 1].max(-1) - s[..., t, :64].max(-1)) * l2e
        assert np.all(grow > 8.0), t
    if T >= 512:
        assert np.all((s[..., -1, :].max(-1) - s[..., -1, :64].max(-1)) * l2e > 24.0)


def test_attention_single_key_rows_and_constant_keys():
    """The first position attends only to itself (o_0 = v_0), and with identical keys
    o_t = mean_{s<=t} v_s (closed forms that hold at any size)."""
    Bn, T, H, hd = 1, 128, 2, 64
    D, N = H * hd, T
    qkv0 = inputs.normal(12, (N, 3 * D), 1.0, False)
    qkv0[:, D:2 * D] = qkv0[0, D:2 * D]                      # constant keys
    out = torch.empty(N, D, device="cuda")
    lse2 = torch.empty(Bn, H, T, device="cuda")
    B.gptk_attention_fwd(dev(qkv0), out, lse2, Bn, T, H, hd)
    v = qkv0[:, 2 * D:].astype(np.float64)
    want = np.cumsum(v, 0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(host(out), want, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("dtype,V", [(BF, 50304), (BF, 65536), (F32, 512), (BF, 512)])
def test_softcap_cross_entropy(dtype, V):
    rows = 37
    bf = dtype == BF
    z0 = inputs.normal(13, (rows, V), 3.0, bf)
    z0[0, :] = 0.0                                    # uniform row: loss = ln V
    z0[1, 5] = 400.0                                  # saturated softcap
    tgt = np.random.default_rng(14).integers(0, V, rows).astype(np.int32)
    tgt[2] = -1
    tgt[3] = V - 1
    nv = int(np.sum(tgt >= 0))
    tz = dev(z0, dtype)
    loss = torch.empty(rows, device="cuda")
    B.gptk_softcap_ce(tz, dev(tgt), torch.tensor([nv], dtype=torch.int32, device="cuda"), loss,
                      cap=15.0, grad_scale=0.5)
    l_want, g_want = om.softcap_cross_entropy(z0.astype(np.float64), tgt.astype(np.int64), 15.0)
    np.testing.assert_allclose(host(loss), l_want, rtol=(1e-5 if not bf else 2e-5), atol=1e-5)
    assert host(loss)[0] == pytest.approx(math.log(V), rel=1e-5)
    assert host(loss)[2] == 0.0
    g = host(tz)
    assert rel_l2(g, g_want * 0.5 / nv) < (5e-3 if bf else 1e-5)
    assert np.all(g[2] == 0)


@pytest.mark.parametrize("dtype,V,rows,cap", [(BF, 65536, 600, 15.0), (BF, 50304, 700, 15.0),
                                              (BF, 2048, 2300, 15.0), (BF, 4096, 1500, 0.0),
                                              (F32, 512, 3000, 15.0)])
def test_cross_entropy_rows_per_workgroup(dtype, V, rows, cap):
    """More rows than workgroups that fit the GPU at once, so each workgroup walks several rows
    (loads of the next row in flight during the current one); rows of only negative logits,
    saturated logits of both signs and ignored targets throughout."""
    bf = dtype == BF
    z0 = inputs.normal(21, (rows, V), 3.0, bf)
    z0[1::7] = -np.abs(z0[1::7]) - 1.0                 # every logit negative
    z0[2::11, 3] = 400.0                               # saturated above
    z0[3::13, :] = -400.0                              # saturated below everywhere: uniform
    if bf:
        z0 = inputs.round_bf16(z0)                     # both sides see the same logits
    tgt = np.random.default_rng(22).integers(0, V, rows).astype(np.int32)
    tgt[::17] = -1
    nv = int(np.sum(tgt >= 0))
    tz = dev(z0, dtype)
    loss = torch.empty(rows, device="cuda")
    B.gptk_softcap_ce(tz, dev(tgt), torch.tensor([nv], dtype=torch.int32, device="cuda"), loss,
                      cap=cap, grad_scale=1.0)
    l_want, g_want = om.softcap_cross_entropy(z0.astype(np.float64), tgt.astype(np.int64), cap)
    np.testing.assert_allclose(host(loss), l_want, rtol=(2e-5 if bf else 1e-5), atol=1e-5)
    g = host(tz)
    assert rel_l2(g, g_want / nv) < (5e-3 if bf else 1e-5)
    # row by row too (a wrong row hides in the norm of 1000)
    per_row = np.linalg.norm(g - g_want / nv, axis=1) / np.maximum(np.linalg.norm(g_want / nv, axis=1), 1e-30)
    assert np.max(per_row[tgt >= 0]) < (2e-2 if bf else 1e-4)
    assert np.all(g[tgt < 0] == 0)


@pytest.mark.parametrize("hd,H,T,Bn,qk_norm,vadd", [(128, 2, 64, 5, 1, False),   # 128x128 tiles, ragged M
                                                   (64, 4, 128, 3, 0, True),
                                                   (32, 4, 64, 4, 1, True),
                                                   (128, 16, 64, 37, 1, False)])  # 256x256, ragged M
def test_qkv_projection_with_fused_rotary_qknorm(hd, H, T, Bn, qk_norm, vadd):
    """The bf16 q/k/v projection with rotary + QK-norm in the GEMM epilogue against the oracle:
    q = x Wq^T etc. in fp64, the half-split rotation with the stored (bf16) tables, RMSNorm per
    head; rstd per (token, head); the value block plus its addend."""
    D = H * hd
    N = Bn * T
    x = inputs.normal(16, (N, D), 1.0, True)
    w = inputs.normal(17, (3 * D, D), 0.05, True)
    u = inputs.normal(18, (N, D), 0.5, False) if vadd else None
    cos = torch.empty(T, hd // 2, device="cuda", dtype=BF)
    sin = torch.empty_like(cos)
    B.gptk_rope_table(cos, sin, T, hd, 10000.0)
    qkv = torch.full((N, 3 * D), float("nan"), device="cuda", dtype=BF)
    rstd = torch.full((N, 2 * H), float("nan"), device="cuda")
    B.gptk_qkv_rope_fwd(dev(x, BF), dev(w, BF), qkv, cos, sin, rstd, None if u is None else dev(u),
                        T, H, hd, qk_norm, 1e-6)
    torch.cuda.synchronize()
    y = x.astype(np.float64) @ w.astype(np.float64).T
    cq, sq = host(cos).astype(np.float64), host(sin).astype(np.float64)
    got = host(qkv)
    for blk in (0, 1):
        z = om.rope(y[:, blk * D:(blk + 1) * D].reshape(Bn, T, H, hd), cq, sq)
        if qk_norm:
            z, r = om.rms_norm(z, 1e-6)
            np.testing.assert_allclose(host(rstd)[:, blk * H:(blk + 1) * H], r.reshape(N, H),
                                       rtol=1e-4)
        assert rel_l2(got[:, blk * D:(blk + 1) * D], z.reshape(N, D)) < 4e-3, blk
    v = y[:, 2 * D:] + (u.astype(np.float64) if vadd else 0.0)
    assert rel_l2(got[:, 2 * D:], v) < 4e-3
