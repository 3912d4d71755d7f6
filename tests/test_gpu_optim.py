"""GPU parity of the dense optimizer step (gpt_opt_step) against the oracle (oracle/optim.py).

Tolerances (derived from the arithmetic): Adam tensors and every state buffer are fp32 on both
sides: relative L2 error of the update <= 1e-5.  Muon updates go through five bf16 Newton-Schulz
steps on both sides with one rounding per new matrix; the GPU accumulates in fp32 where the
oracle is exact, so a product near a bf16 rounding boundary can round the other way (2^-8
relative) and the iteration carries it on: relative L2 error of the update <= 2e-2, cosine
>= 0.999.  The bf16 copy of the weights must equal the round-to-nearest-even of the new fp32
weights bit for bit."""
import math

import numpy as np
import pytest
import torch

from gpt_lm_step_amd import binding as B
from gpt_lm_step_amd import configs
from oracle import optim as oo

from gpu_util import cosine, rel_l2

pytestmark = pytest.mark.gpu

HP = dict(lr_matrix=0.02, lr_embedding=0.2, lr_unembedding=0.004, beta1=0.8, beta2=0.95,
          eps=1e-10, weight_decay=0.0, grad_clip=1.0, num_iterations=1000, warmup_ratio=0.0,
          warmdown_ratio=0.2, final_lr_frac=0.0, nesterov=1, ns_steps=5)


def _hparams(it, t):
    return dict(lr_matrix=HP["lr_matrix"], lr_embedding=HP["lr_embedding"],
                lr_unembedding=HP["lr_unembedding"],
                lr_mult=B.gpt_lr_multiplier(it, HP["num_iterations"], HP["warmup_ratio"],
                                            HP["warmdown_ratio"], HP["final_lr_frac"]),
                momentum=B.gpt_muon_momentum(it), beta1=HP["beta1"], beta2=HP["beta2"],
                eps=HP["eps"], weight_decay=HP["weight_decay"], grad_clip=HP["grad_clip"],
                nesterov=1, ns_steps=5, adam_step=t)


def _tensors(cfg, flat):
    return {n: flat[o:o + s[0] * s[1]].reshape(s) for n, o, s in configs.param_layout(cfg)}


def _state_dict(cfg, state):
    """The oracle's view of the flat state: 'mom.<matrix>' per Muon matrix, 'm.'/'v.' for Adam."""
    T = _tensors(cfg, state[:configs.param_elems(cfg)])
    vd = cfg.vocab * cfg.d_model
    v0 = configs.param_elems(cfg)
    va = (vd + 63) // 64 * 64
    out = {"m.wte": T["wte"], "m.lm_head": T["lm_head"],
           "v.wte": state[v0:v0 + vd].reshape(cfg.vocab, cfg.d_model),
           "v.lm_head": state[v0 + va:v0 + va + vd].reshape(cfg.vocab, cfg.d_model)}
    for mname, tensor, rows in oo.muon_matrices(cfg):
        out[f"mom.{mname}"] = T[tensor][rows]
    return out


def _run_steps(cfg, steps, seed):
    rng = np.random.default_rng(seed)
    n = configs.param_elems(cfg)
    master0 = (rng.standard_normal(n) * 0.02).astype(np.float32)
    bf16 = cfg.dtype == configs.BF16
    master = torch.from_numpy(master0.copy()).cuda()
    params = torch.empty(n, dtype=torch.bfloat16, device="cuda") if bf16 else None
    state = torch.zeros(B.gpt_opt_state_elems(cfg), device="cuda")
    ws = torch.empty(B.gpt_opt_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    gnorm = torch.zeros(1, device="cuda")
    o_master = _tensors(cfg, master0.astype(np.float64))
    o_state = {}
    for k in range(steps):
        g = (rng.standard_normal(n) * 0.05).astype(np.float32)
        g[: cfg.vocab * cfg.d_model] *= 0.01                       # a smaller embedding gradient
        grads = torch.from_numpy(g).cuda()
        before = master.cpu().numpy().astype(np.float64)
        B.gpt_opt_step(cfg, master, params, grads, state, _hparams(k, k + 1), ws, gnorm)
        torch.cuda.synchronize()
        o_before = {kk: v.copy() for kk, v in o_master.items()}
        o_master, o_state, o_norm = oo.optimizer_step(cfg, o_master, _tensors(cfg, g.astype(np.float64)),
                                                      o_state, it=k, t=k + 1, hp=HP, bf16=True)
        got = master.cpu().numpy().astype(np.float64)
        assert float(gnorm.item()) == pytest.approx(o_norm, rel=1e-5)
        G = _tensors(cfg, got - before)
        W = {kk: o_master[kk] - o_before[kk] for kk in o_master}
        for name in G:
            e = rel_l2(G[name], W[name])
            if name in ("wte", "lm_head"):
                assert e <= 1e-5, (k, name, e)
            else:
                assert e <= 2e-2, (k, name, e)
                assert cosine(G[name], W[name]) >= 0.999, (k, name)
        # keep both sides on the same weights and state (the GPU's) for the next step
        o_master = _tensors(cfg, got)
        S = _state_dict(cfg, state.cpu().numpy().astype(np.float64))
        for key, want in o_state.items():
            assert rel_l2(S[key], want) <= 1e-5, (k, key)
        o_state = S
        if bf16:
            np.testing.assert_array_equal(params.view(torch.int16).cpu().numpy(),
                                          master.to(torch.bfloat16).view(torch.int16).cpu().numpy())


def test_optimizer_step_small_bf16_model_two_steps():
    cfg = configs.TINY.replace(n_layer=2, d_model=256, n_head=4, head_dim=64, d_mlp=1024,
                               vocab=512, dtype=configs.BF16)
    _run_steps(cfg, 2, 31)


def test_optimizer_step_tiny_fp32_in_place():
    _run_steps(configs.TINY, 2, 32)


def test_optimizer_step_d32_full_size_sampled():
    """The d32 step's optimizer at full size (1.88e9 parameters, every Muon batch at its real
    shape); the oracle recomputes the global norm, both Adam tensors and three Muon matrices
    (layer 0's q block, a tall MLP up and a wide MLP down projection)."""
    cfg = configs.D32
    n = configs.param_elems(cfg)
    g = torch.Generator(device="cuda").manual_seed(41)
    master = torch.randn(n, device="cuda", generator=g) * 0.02
    grads = torch.randn(n, device="cuda", generator=g) * 0.05
    params = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    state = torch.zeros(B.gpt_opt_state_elems(cfg), device="cuda")
    ws = torch.empty(B.gpt_opt_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    gnorm = torch.zeros(1, device="cuda")
    lay = {name: (o, s) for name, o, s in configs.param_layout(cfg)}

    def host_t(buf, name, rows=slice(None)):
        o, s = lay[name]
        return buf[o:o + s[0] * s[1]].view(s[0], s[1])[rows].cpu().numpy().astype(np.float64)

    D = cfg.d_model
    picks = [("h0.q", "h0.wqkv", slice(0, D)), ("h17.wfc", "h17.wfc", slice(None)),
             ("h31.wpr", "h31.wpr", slice(None))]
    before = {name: host_t(master, name) for name in ("wte", "lm_head")}
    before.update({m: host_t(master, t, r) for m, t, r in picks})
    gh = {name: host_t(grads, name) for name in ("wte", "lm_head")}
    gh.update({m: host_t(grads, t, r) for m, t, r in picks})
    norm = float(torch.linalg.vector_norm(grads.double()).item())
    B.gpt_opt_step(cfg, master, params, grads, state, _hparams(0, 1), ws, gnorm)
    torch.cuda.synchronize()
    assert float(gnorm.item()) == pytest.approx(norm, rel=1e-5)
    f = min(1.0, HP["grad_clip"] / (norm + 1e-6))
    scale = (D / 768) ** -0.5
    for name, lr in (("wte", HP["lr_embedding"] * scale), ("lm_head", HP["lr_unembedding"] * scale)):
        want, _, _ = oo.adam_update(before[name], f * gh[name], 0.0, 0.0, 1, lr, HP["beta1"],
                                    HP["beta2"], HP["eps"], 0.0)
        e = rel_l2(host_t(master, name) - before[name], want - before[name])
        assert e <= 1e-5, (name, e)
    for m, t, r in picks:
        want, _ = oo.muon_update(before[m], f * gh[m], np.zeros_like(gh[m]), HP["lr_matrix"],
                                 oo.muon_momentum(0), True, 5, bf16=True)
        got = host_t(master, t, r)
        e = rel_l2(got - before[m], want - before[m])
        assert e <= 2e-2, (m, e)
        assert cosine(got - before[m], want - before[m]) >= 0.999, m
    np.testing.assert_array_equal(params[:1 << 20].view(torch.int16).cpu().numpy(),
                                  master[:1 << 20].to(torch.bfloat16).view(torch.int16).cpu().numpy())
