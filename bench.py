#!/usr/bin/env python3
"""Throughput of one decoder training step (forward + hand-written backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload d32|gpt2|tiny]

Prints ONE JSON line: tokens/s of the whole fwd+bwd step (inputs already in HBM), MFU against
the bf16 dense MFMA peak using the nanochat estimate_flops convention
(6*(params - embedding) + 12*L*H*Hd*T per token), the roofline of the dominant kernel
(timed live with HIP events around each launch of an instrumented pass), and the CPU oracle
timed on a bounded sample of the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

from gpt_lm_step_amd import configs, inputs

PEAK_BF16 = 2.5e15       # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP32 = 157.3e12     # MI355X fp32 (matrix and vector), FLOP/s
PEAK_HBM = 8.0e12        # MI355X HBM3E, B/s
METRIC = "train tokens/sec (fwd+bwd) on 1 MI355X + MFU vs bf16 MFMA peak"
WORKLOADS = {"d32": configs.D32, "gpt2": configs.GPT2_SMALL, "tiny": configs.TINY}
# Stages made of several kernels (their time is not one kernel's launch duration).
MULTI_KERNEL = {"wte_segsum"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="d32", choices=sorted(WORKLOADS))
    ap.add_argument("--profile-steps", type=int, default=2)
    ap.add_argument("--cpu-tokens", type=int, default=384,
                    help="tokens of the CPU-oracle sample (one sequence)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def cpu_baseline(cfg, flat_dev, tokens, n_tok):
    """The oracle (fp64 numpy, as it stands) on one sequence of n_tok tokens of the same model."""
    import torch
    from threadpoolctl import threadpool_limits
    from oracle import model as om
    cores = len(os.sched_getaffinity(0))
    flat = flat_dev.float().cpu().numpy()
    params = inputs.unflatten(cfg, flat)
    sub = cfg.replace(batch=1, seq_len=n_tok)
    tok = np.ascontiguousarray(tokens[:1, :n_tok + 1])
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        res = om.forward_backward(sub, params, tok)
        dt = time.perf_counter() - t0
    assert np.isfinite(res.loss)
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"1 sequence x {n_tok} tokens of the {cfg.name} step (same layers and "
                      f"vocab, fp64 numpy fwd+bwd), {dt:.1f} s"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the step has no multi-GPU path (got --gpus {a.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from gpt_lm_step_amd import binding as B
    if not os.path.exists(B._LIB_PATH):
        from gpt_lm_step_amd import build
        build.build()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    cfg = WORKLOADS[a.workload]
    seeds = inputs.seeds_for(cfg.name)
    bf16 = cfg.dtype == configs.BF16
    tokens = inputs.step_tokens(cfg, seeds["tokens"], zipf=bf16)
    T = cfg.seq_len
    t_in = torch.from_numpy(np.ascontiguousarray(tokens[:, :T])).cuda()
    t_tg = torch.from_numpy(np.ascontiguousarray(tokens[:, 1:])).cuda()
    params = inputs.device_params(cfg, seeds["weights"])
    grads = torch.empty(configs.param_elems(cfg), device="cuda")
    loss = torch.zeros(1, device="cuda")
    ctx = B.gpt_init(cfg)

    def step():
        B.gpt_fwd_bwd(ctx, t_in, t_tg, params, grads, loss)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(a.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / a.steps
    lval = float(loss.item())
    assert np.isfinite(lval), lval

    # instrumented pass: every launch bracketed by events on the step's stream
    B.gpt_profile(ctx, True)
    for _ in range(a.profile_steps):
        step()
    B.gpt_profile(ctx, False)
    stages = B.gpt_profile_read(ctx)
    torch.cuda.synchronize()
    ps = max(a.profile_steps, 1)
    stage_ms = {n: round(m / ps, 3) for n, c, m, f, b in stages}
    single = [s for s in stages if s[0] not in MULTI_KERNEL]
    name, calls, tot_ms, flops, nbytes = max(single, key=lambda s: s[2])
    per_launch_s = tot_ms / calls / 1e3
    if flops > 0:
        peak = PEAK_BF16 if bf16 else PEAK_FP32
        achieved = flops / calls / per_launch_s
        roof = {"bound": "mfma", "kernel": name, "achieved": round(achieved / 1e12, 1),
                "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None, "launches_per_step": calls // ps,
                "avg_launch_ms": round(per_launch_s * 1e3, 4),
                "algorithmic_per_launch": flops / calls}
    else:
        achieved = nbytes / calls / per_launch_s
        roof = {"bound": "hbm", "kernel": name, "achieved": round(achieved / 1e9, 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(achieved / PEAK_HBM, 4),
                "traffic": None, "launches_per_step": calls // ps,
                "avg_launch_ms": round(per_launch_s * 1e3, 4),
                "algorithmic_per_launch": nbytes / calls}

    tok_s = cfg.tokens / (ms / 1e3)
    fpt = configs.flops_per_token(cfg)
    peak = PEAK_BF16 if bf16 else PEAK_FP32
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32", "data": "synthetic (seeded Zipf tokens, N(0,0.02) weights)",
        "config": {"workload": f"{cfg.name} fwd+bwd step", "layers": cfg.n_layer,
                   "d_model": cfg.d_model, "heads": cfg.n_head, "head_dim": cfg.head_dim,
                   "d_mlp": cfg.d_mlp, "vocab": cfg.vocab, "seq_len": cfg.seq_len,
                   "batch": cfg.batch, "tokens_per_step": cfg.tokens, "parallelism": "none (1 GPU)"},
        "mfu": round(fpt * tok_s / peak, 4),
        "hw_mfu": round(configs.hardware_flops_per_step(cfg) / (ms / 1e3) / peak, 4),
        "flops_per_token": fpt, "loss": round(lval, 5), "wall_s": round(wall, 3),
        "roofline": roof, "stage_ms_per_step": stage_ms,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, params, tokens, min(a.cpu_tokens, cfg.seq_len))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
