#!/usr/bin/env python3
"""Throughput of one decoder training step (forward + hand-written backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload d32|gpt2|tiny|tables|speedrun|opt]

Prints ONE JSON line.  Dense workloads (d32 default, gpt2, tiny): tokens/s of the whole fwd+bwd
step (inputs already in HBM), MFU against the bf16 dense MFMA peak using the nanochat
estimate_flops convention (6*(params - embedding) + 12*L*H*Hd*T per token), the roofline of the
dominant kernel and of every stage (timed live with HIP events around each launch of an
instrumented pass), and the CPU oracle timed on a bounded sample of the same workload on this
host's cores.  `tables`: the hashed-bigram gather and the fused scatter-reduce + per-row update
of both tables over 196,608 tokens.  `speedrun`: one optimizer step of the GPT-2-small model
with both bigram tables and the trigram table, 24 accumulated micro-batches of 8 x 1024 tokens,
then one in-place update per table.  `opt`: the dense optimizer step of the d32 model.
`decode`: batched generation with the key/value cache on the d32 model (batch 8, 1024-token
prompt, then one token per sequence per step: cached forward + top-k sampling).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

from gpt_lm_step_amd import configs, inputs

PEAK_BF16 = 2.5e15       # MI355X dense bf16 MFMA, FLOP/s
PEAK_FP32 = 157.3e12     # MI355X fp32 (matrix and vector), FLOP/s
PEAK_HBM = 8.0e12        # MI355X HBM3E, B/s
METRIC = "train tokens/sec (fwd+bwd) on 1 MI355X + MFU vs bf16 MFMA peak"
DENSE = {"d32": configs.D32, "gpt2": configs.GPT2_SMALL, "tiny": configs.TINY}
WORKLOADS = sorted(list(DENSE) + ["tables", "speedrun", "copy", "opt", "decode", "gemm_ref"])
# Stages made of several kernels (their time is not one kernel's launch duration); the weight-
# gradient stages join them when their shape is split over K (see split_stages).
MULTI_KERNEL = {"wte_segsum"}


def split_stages(B, cfg):
    """Weight-gradient stages whose GEMM runs split over K (partials + a reduce kernel)."""
    if cfg.dtype != configs.BF16:
        return set()
    D, F, N, V = cfg.d_model, cfg.d_mlp, cfg.tokens, cfg.vocab
    shapes = {"head_wgrad": (V, D, N), "down_wgrad": (D, F, N), "up_wgrad": (F, D, N),
              "out_wgrad": (D, D, N), "qkv_wgrad": (3 * D, D, N), "tri_wgrad": (D, D, N)}
    return {k for k, s in shapes.items() if B.gptk_gemm_wgrad_ws_floats(*s) > 0}


def multi_stages(B, cfg):
    """Stages that launch more than one kernel for this configuration."""
    # the fp32 attention backward computes rowsum(dO*O) in a kernel of its own before dQ
    extra = set() if cfg.dtype == configs.BF16 else {"attn_bwd_dq"}
    return split_stages(B, cfg) | extra


# Kernels whose HBM traffic has been measured with rocprofv3 counters (profiles/traffic.json): the
# stage name, substrings of the kernel symbol ('|'-separated alternatives: mangled or demangled)
# that identify it in the counter output, the source file the measurement belongs to, and the
# workloads whose runs measure it (a symbol pattern names that stage's kernel only there: the
# decode workload's prefill launches the training GEMMs too).
TRAINING = ("d32", "gpt2", "speedrun")
TRAFFIC_KERNELS = {
    "down_dgrad": ("EpiDRelu2", "gemm.h", TRAINING),
    "up_fwd": ("EpiRelu2", "gemm.h", TRAINING),
    "down_fwd": ("EpiResidELi4E|EpiResid, 4>", "gemm.h", TRAINING),
    "attn_bwd_dkdv": ("attn_bwd_dkdv_pipe_kernel", "attn.hip", TRAINING),
    "softcap_ce": ("9ce_kernelI|::ce_kernel<", "ce.hip", TRAINING),
    "bigram_fwd (hash + gather-add, x0 table)": ("bigram_gather_kernel", "tables.hip", ("tables",)),
    "attn_split": ("attn_split_kernel", "infer.hip", ("decode",)),
}
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "gpt_lm_step_amd", "csrc")


def _source_sha(name):
    import hashlib
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()[:16]


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from the stored counter measurement, or None when there is
    none or the kernel's source has changed since it was taken."""
    try:
        entries = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    for e in entries:
        if e["workload"] == workload and e["stage"] == stage:
            if e["source_sha"] != _source_sha(e["source"]):
                return None
            return e["hbm_bytes_per_launch"]
    return None


def _counter_per_dispatch(out_dir, counter, pattern):
    """Mean of `counter` (summed over instances) per dispatch of the kernels matching `pattern`."""
    import csv
    import glob
    import collections
    f = glob.glob(os.path.join(out_dir, "*counter_collection.csv"))[0]
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(f)):
        if r["Counter_Name"] == counter and any(p in r["Kernel_Name"] for p in pattern.split("|")):
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
    assert per, f"no {counter} rows for {pattern} in {out_dir}"
    return sum(per.values()) / len(per)


def record_traffic(a):
    """Write profiles/traffic.json entries for this workload from four rocprofv3 --pmc output
    directories: FETCH_SIZE and WRITE_SIZE over the workload, and the same over `--workload copy`
    (a device copy of COPY_BYTES, read once and written once), which scales each counter."""
    fetch_dir, write_dir, copy_fetch_dir, copy_write_dir = a.record_traffic
    copy_pat = "copyBuffer"
    fs = COPY_BYTES / (1024.0 * _counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE", copy_pat))
    ws = COPY_BYTES / (1024.0 * _counter_per_dispatch(copy_write_dir, "WRITE_SIZE", copy_pat))
    try:
        entries = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        entries = []
    for stage, (pattern, source, workloads) in TRAFFIC_KERNELS.items():
        if a.workload not in workloads:
            continue
        try:
            fk = _counter_per_dispatch(fetch_dir, "FETCH_SIZE", pattern)
            wk = _counter_per_dispatch(write_dir, "WRITE_SIZE", pattern)
        except AssertionError:
            continue
        entries = [e for e in entries if not (e["workload"] == a.workload and e["stage"] == stage)]
        entries.append({"workload": a.workload, "stage": stage, "kernel_pattern": pattern,
                        "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
                        "copy_fetch_scale": round(fs, 4), "copy_write_scale": round(ws, 4),
                        "hbm_bytes_per_launch": round(fk * 1024 * fs + wk * 1024 * ws),
                        "source": source, "source_sha": _source_sha(source)})
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(entries, f, indent=1)
    print(json.dumps(entries, indent=1))


COPY_BYTES = 1 << 30


def bench_copy(a):
    """Calibration: a plain device-to-device copy of COPY_BYTES (read once, written once)."""
    import torch
    x = torch.ones(COPY_BYTES // 4, device="cuda")
    y = torch.empty_like(x)
    for _ in range(a.warmup):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(a.steps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps
    return {"metric": "device copy bytes/s (counter calibration)", "value": 2 * COPY_BYTES / ms / 1e6,
            "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
            "higher_is_better": True, "config": {"workload": "copy", "bytes": COPY_BYTES}}


GEMM_REF_SHAPES = [  # (name, M, N, K): the step's forward products (tokens x out x in)
    ("d32 q/k/v", 16384, 6144, 2048), ("d32 out", 16384, 2048, 2048),
    ("d32 MLP up", 16384, 8192, 2048), ("d32 MLP down", 16384, 2048, 8192),
    ("d32 LM head", 16384, 65536, 2048),
    ("GPT-2 q/k/v", 8192, 2304, 768), ("GPT-2 out", 8192, 768, 768),
    ("GPT-2 MLP up", 8192, 3072, 768), ("GPT-2 MLP down", 8192, 768, 3072),
    ("GPT-2 LM head", 8192, 50304, 768),
]


def bench_gemm_ref(a, B):
    """Context for the GEMM figures: this library's bf16 product (gptk_gemm, fp32 output, tile
    size by its own rule) and hipBLASLt through torch.mm (bf16 output) on the step's product
    shapes, the same operand layouts (A [M, K] K-contiguous, B stored [K, N]), each timed with
    events over a.steps launches after a.warmup.  value = geometric mean of the library's
    rate over hipBLASLt's."""
    import torch
    rows, ratios = [], []
    g = torch.Generator(device="cuda").manual_seed(7)
    for name, M, N, K in GEMM_REF_SHAPES:
        x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
        w = torch.randn(K, N, device="cuda", generator=g).to(torch.bfloat16)
        c = torch.empty(M, N, device="cuda")

        def ours():
            B.gptk_gemm(1, 0, M, N, K, x, K, w, N, c, N)

        def lib():
            return torch.mm(x, w)

        def timed(f):
            for _ in range(a.warmup):
                f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(a.steps):
                f()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / a.steps
        t_ours, t_lib = timed(ours), timed(lib)
        fl = 2.0 * M * N * K
        rows.append({"product": name, "M": M, "N": N, "K": K,
                     "ours_ms": round(t_ours, 4), "ours_tflops": round(fl / t_ours / 1e9, 1),
                     "hipblaslt_ms": round(t_lib, 4), "hipblaslt_tflops": round(fl / t_lib / 1e9, 1)})
        ratios.append(t_lib / t_ours)
        print(f"{name:16s} {M:6d} {N:6d} {K:5d}  ours {rows[-1]['ours_tflops']:7.1f} TFLOP/s  "
              f"hipBLASLt {rows[-1]['hipblaslt_tflops']:7.1f} TFLOP/s", file=sys.stderr, flush=True)
        del x, w, c
        torch.cuda.empty_cache()
    gm = math.exp(sum(math.log(r) for r in ratios) / len(ratios))
    return {"metric": "bf16 GEMM rate relative to hipBLASLt (geometric mean over the step's products)",
            "value": round(gm, 4), "unit": "ratio", "n_gpus": 1, "steps": a.steps,
            "warmup": a.warmup, "higher_is_better": True, "dtype": "bf16",
            "config": {"workload": "gemm_ref", "products": rows}}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="d32", choices=WORKLOADS)
    ap.add_argument("--profile-steps", type=int, default=2)
    ap.add_argument("--cpu-tokens", type=int, default=384,
                    help="tokens of the CPU-oracle sample (one sequence)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--record-traffic", nargs=4, metavar="DIR",
                    help="write profiles/traffic.json from rocprofv3 --pmc output directories: "
                         "FETCH_SIZE and WRITE_SIZE of the workload, then of --workload copy")
    return ap.parse_args()


def _cores():
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, flat_dev, tokens, n_tok, addends=None):
    """The oracle (fp64 numpy, as it stands) on one sequence of n_tok tokens of the same model.
    `addends`: optional callable (tokens [1, n_tok+1]) -> (x0_add, v_add, tri_rows) on the host."""
    from threadpoolctl import threadpool_limits
    from oracle import model as om
    cores = _cores()
    flat = flat_dev.float().cpu().numpy()
    params = inputs.unflatten(cfg, flat)
    sub = cfg.replace(batch=1, seq_len=n_tok)
    tok = np.ascontiguousarray(tokens[:1, :n_tok + 1])
    adds = addends(tok) if addends else (None, None, None)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        res = om.forward_backward(sub, params, tok, *adds)
        dt = time.perf_counter() - t0
    assert np.isfinite(res.loss)
    return {"value": n_tok / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"1 sequence x {n_tok} tokens of the {cfg.name} step (same layers and "
                      f"vocab, fp64 numpy fwd+bwd), {dt:.1f} s"}


def _roof_entry(name, calls, tot_ms, flops, nbytes, bf16):
    """Roofline of one stage: algorithmic work per launch / average launch duration."""
    per_launch_s = tot_ms / calls / 1e3
    if flops > 0:
        peak = PEAK_BF16 if bf16 else PEAK_FP32
        ach = flops / calls / per_launch_s
        return {"bound": "mfma", "kernel": name, "achieved": round(ach / 1e12, 1),
                "peak": peak / 1e12, "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                "avg_launch_ms": round(per_launch_s * 1e3, 4), "algorithmic_per_launch": flops / calls}
    ach = nbytes / calls / per_launch_s
    return {"bound": "hbm", "kernel": name, "achieved": round(ach / 1e9, 1),
            "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(ach / PEAK_HBM, 4),
            "avg_launch_ms": round(per_launch_s * 1e3, 4), "algorithmic_per_launch": nbytes / calls}


def _roof_entry_by_intensity(name, calls, tot_ms, flops, nbytes):
    """Roofline of a bf16 stage bound by whichever resource its arithmetic intensity selects:
    the matrix cores above the ridge (peak FLOP/s / peak bytes/s), HBM below it."""
    if flops > 0 and flops / max(nbytes, 1.0) >= PEAK_BF16 / PEAK_HBM:
        return _roof_entry(name, calls, tot_ms, flops, nbytes, True)
    return _roof_entry(name, calls, tot_ms, 0.0, nbytes, True)


def profile_stages(B, ctx, step, n_steps, bf16, multi=frozenset(), workload=None):
    """Instrumented pass: every launch bracketed by events on the step's stream.  Returns the
    dominant single-kernel stage's roofline and a per-stage table."""
    import torch
    B.gpt_profile(ctx, True)
    for _ in range(n_steps):
        step()
    B.gpt_profile(ctx, False)
    stages = B.gpt_profile_read(ctx)
    torch.cuda.synchronize()
    ps = max(n_steps, 1)
    parts = {}
    for n, c, m, f, b in stages:
        e = _roof_entry(n, c, m, f, b, bf16)
        parts[n] = {"ms_per_step": round(m / ps, 3), "launches": c // ps,
                    "achieved": e["achieved"], "unit": e["unit"], "frac": e["frac"]}
    single = [s for s in stages if s[0] not in MULTI_KERNEL and s[0] not in multi]
    name, calls, tot_ms, flops, nbytes = max(single, key=lambda s: s[2])
    roof = _roof_entry(name, calls, tot_ms, flops, nbytes, bf16)
    roof["traffic"] = measured_traffic(workload, name)
    roof["launches_per_step"] = calls // ps
    return roof, parts


def time_steps(step, steps, warmup):
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, time.perf_counter() - w0


def bench_dense(a, B):
    import torch
    cfg = DENSE[a.workload]
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

    ms, wall = time_steps(step, a.steps, a.warmup)
    lval = float(loss.item())
    assert np.isfinite(lval), lval
    roof, parts = profile_stages(B, ctx, step, a.profile_steps, bf16, multi_stages(B, cfg),
                                 a.workload)

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
        "roofline": roof, "parts": parts,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, params, tokens, min(a.cpu_tokens, cfg.seq_len))
    return out


def _tables(tc, seed, tri_seed=None):
    """Device tables: x0 (2^21 rows) and value (2^20 rows) N(0, 0.02), trigram N(0, 1); bf16."""
    import torch
    g = torch.Generator(device="cuda").manual_seed(seed)
    tx0 = (torch.randn(tc.x0_rows, tc.dim, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    tv = (torch.randn(tc.v_rows, tc.dim, device="cuda", generator=g) * 0.02).to(torch.bfloat16)
    ttri = None
    if tri_seed is not None:
        g.manual_seed(tri_seed)
        ttri = torch.randn(tc.tri_rows, tc.dim, device="cuda", generator=g).to(torch.bfloat16)
    return tx0, tv, ttri


def gather_bytes(n, dim, unique):
    """Algorithmic bytes of one gather-add: tokens + h (4 B each), each distinct row read once,
    y read and written (bf16)."""
    return n * 8 + unique * dim * 2 + 2 * n * dim * 2


def update_bytes(n, dim, unique):
    """Algorithmic bytes of one scatter-reduce + update: h, dy once, each touched row read and
    written, plus its fp32 second moment read and written."""
    return n * 4 + n * dim * 2 + unique * (2 * dim * 2 + 8)


def _timed(fn, evs):
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    evs.append((e0, e1))


def cpu_tables_baseline(tc, n_seq=32, rows_log2=18):
    """The oracle's hash + gather-add + sparse row update (fp64 numpy, as it stands) on the
    first n_seq sequences, tables of 2^rows_log2 rows (the oracle copies whole tables in fp64)."""
    from threadpoolctl import threadpool_limits
    from oracle import tables as ot
    cores = _cores()
    seeds = inputs.seeds_for("tables")
    tok = inputs.zipf_tokens(seeds["tokens"], (tc.n_tokens // tc.seq_len, tc.seq_len), tc.vocab)[:n_seq]
    R = 1 << rows_log2
    table = inputs.normal(seeds["weights"], (R, tc.dim), 0.02, True)
    dy = inputs.normal(seeds["dy"], (tok.size, tc.dim), 1.0, True)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        h = ot.hash_indices(tok, 2, tc.vocab, R)
        y = ot.gather_add(np.zeros((tok.size, tc.dim), np.float32), table, h)
        ot.sparse_row_update(table, np.zeros(R), h, dy, tc.lr, tc.beta2, tc.eps)
        dt = time.perf_counter() - t0
    assert np.isfinite(y).all()
    return {"value": tok.size / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_seq} sequences x {tc.seq_len} tokens, one table of 2^{rows_log2} x "
                      f"{tc.dim} rows: hash + gather-add + sparse update in fp64 numpy, {dt:.1f} s"}


def bench_tables(a, B):
    import torch
    tc = configs.TABLES
    seeds = inputs.seeds_for("tables")
    n_seq = tc.n_tokens // tc.seq_len
    tok = torch.from_numpy(inputs.zipf_tokens(seeds["tokens"], (n_seq, tc.seq_len), tc.vocab)).cuda()
    N, D = tc.n_tokens, tc.dim
    tx0, tv, _ = _tables(tc, seeds["weights"])
    g = torch.Generator(device="cuda").manual_seed(seeds["dy"])
    dy = torch.randn(N, D, device="cuda", generator=g).to(torch.bfloat16)
    v_x0 = torch.zeros(tc.x0_rows, device="cuda")
    v_v = torch.zeros(tc.v_rows, device="cuda")
    y_x0 = torch.zeros(N, D, device="cuda", dtype=torch.bfloat16)
    y_v = torch.zeros(N, D, device="cuda", dtype=torch.bfloat16)
    h_x0 = torch.empty(N, device="cuda", dtype=torch.int32)
    h_v = torch.empty(N, device="cuda", dtype=torch.int32)
    ws = torch.empty(B.bigram_workspace_bytes(N, D), dtype=torch.uint8, device="cuda")
    ws_v = torch.empty(B.bigram_workspace_bytes(N, D), dtype=torch.uint8, device="cuda")
    parts = [("gather_x0", lambda: B.bigram_fwd(tok, 2, tc.vocab, tx0, y_x0, h_x0)),
             ("gather_v", lambda: B.bigram_fwd(tok, 2, tc.vocab, tv, y_v, h_v)),
             ("update_x0", lambda: B.bigram_bwd_update(h_x0, dy, tx0, v_x0, tc.lr, tc.beta2, tc.eps, ws)),
             ("update_v", lambda: B.bigram_bwd_update(h_v, dy, tv, v_v, tc.lr, tc.beta2, tc.eps, ws_v))]
    # the two tables are independent: the value table's gather and update run on a second
    # stream (default priority, its own workspace), joined at the end of the step, so the short
    # launches of the two updates (sort passes, edge finish) overlap
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()

    def step():
        side.wait_stream(main)
        parts[0][1]()
        with torch.cuda.stream(side):
            parts[1][1]()
        parts[2][1]()
        with torch.cuda.stream(side):
            parts[3][1]()
        main.wait_stream(side)

    ms, wall = time_steps(step, a.steps, a.warmup)
    # per-part event timing over the same number of steps
    evs = {n: [] for n, _ in parts}
    for _ in range(a.steps):
        for n, fn in parts:
            _timed(fn, evs[n])
    torch.cuda.synchronize()
    part_ms = {n: sum(e0.elapsed_time(e1) for e0, e1 in v) / len(v) for n, v in evs.items()}
    u_x0 = int(torch.unique(h_x0).numel())
    u_v = int(torch.unique(h_v).numel())
    seg = torch.unique(h_x0, return_counts=True)[1]
    edges = [1, 4, 16, 64, 256, 1 << 62]
    hist = {(f"{lo}-{hi - 1}" if hi < edges[-1] else f">={lo}"): int(((seg >= lo) & (seg < hi)).sum())
            for lo, hi in zip(edges[:-1], edges[1:])}
    alg = {"gather_x0": gather_bytes(N, D, u_x0), "gather_v": gather_bytes(N, D, u_v),
           "update_x0": update_bytes(N, D, u_x0), "update_v": update_bytes(N, D, u_v)}
    table = {}
    for n in part_ms:
        gbs = alg[n] / (part_ms[n] / 1e3) / 1e9
        table[n] = {"ms": round(part_ms[n], 4), "algorithmic_bytes": alg[n],
                    "achieved": round(gbs, 1), "unit": "GB/s", "frac": round(gbs * 1e9 / PEAK_HBM, 4)}
    # the roofline part is the slowest entry point of the step (the x0 table's update: its sort
    # passes, segmented sums and edge finish are timed together as one call)
    names = {"gather_x0": "bigram_fwd (hash + gather-add, x0 table)",
             "gather_v": "bigram_fwd (hash + gather-add, value table)",
             "update_x0": "bigram_bwd_update (sort + segmented sums + row update, x0 table)",
             "update_v": "bigram_bwd_update (sort + segmented sums + row update, value table)"}
    dom = max(table, key=lambda n: table[n]["ms"])
    roof = {"bound": "hbm", "kernel": names[dom],
            "achieved": table[dom]["achieved"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
            "frac": table[dom]["frac"],
            "traffic": measured_traffic("tables", names[dom]),
            "launches_per_step": 1,
            "avg_launch_ms": table[dom]["ms"], "algorithmic_per_launch": alg[dom]}
    out = {
        "metric": "hashed-table tokens/sec (gather fwd + scatter-reduce/update bwd, 2 tables) on 1 MI355X",
        "value": round(N / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf(1.1) tokens, N(0,0.02) tables, N(0,1) upstream grads)",
        "config": {"workload": "hashed bigram tables: x0 2^21x768 + value 2^20x768 bf16, 196608 tokens",
                   "tokens": N, "dim": D, "x0_rows": tc.x0_rows, "v_rows": tc.v_rows,
                   "unique_rows_x0": u_x0, "unique_rows_v": u_v, "largest_segment": int(seg.max()),
                   "segment_hist_x0": hist, "parallelism": "none (1 GPU)"},
        "wall_s": round(wall, 3), "roofline": roof, "parts": table,
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_tables_baseline(tc)
    return out


def bench_speedrun(a, B):
    import torch
    cfg = configs.SPEEDRUN
    tc = configs.TABLES
    MB = configs.SPEEDRUN_MICRO_BATCHES
    seeds = inputs.seeds_for(cfg.name)
    T, N, D, V = cfg.seq_len, cfg.tokens, cfg.d_model, cfg.vocab
    tokens = inputs.zipf_tokens(seeds["tokens"], (MB * cfg.batch, T + 1), V)
    t_in = torch.from_numpy(np.ascontiguousarray(tokens[:, :T])).cuda().view(MB, cfg.batch, T)
    t_tg = torch.from_numpy(np.ascontiguousarray(tokens[:, 1:])).cuda().view(MB, cfg.batch, T)
    params = inputs.device_params(cfg, seeds["weights"])
    grads = torch.empty(configs.param_elems(cfg), device="cuda")
    loss = torch.zeros(1, device="cuda")
    ctx = B.gpt_init(cfg)
    tx0, tv, ttri = _tables(tc, seeds["tables"], seeds["trigram"])
    v_x0 = torch.zeros(tc.x0_rows, device="cuda")
    v_v = torch.zeros(tc.v_rows, device="cuda")
    bf = torch.bfloat16
    add_x0 = torch.empty(N, D, device="cuda", dtype=bf)
    add_v = torch.empty(N, D, device="cuda", dtype=bf)
    add_tri = torch.empty(N, D, device="cuda", dtype=bf)
    d_x0 = torch.empty(MB * N, D, device="cuda", dtype=bf)   # per-token addend grads, staged
    d_v = torch.empty(MB * N, D, device="cuda", dtype=bf)
    h_x0 = torch.empty(MB * N, device="cuda", dtype=torch.int32)
    h_v = torch.empty(MB * N, device="cuda", dtype=torch.int32)
    ws = torch.empty(B.bigram_workspace_bytes(MB * N, D), dtype=torch.uint8, device="cuda")

    def step():
        for i in range(MB):
            sl = slice(i * N, (i + 1) * N)
            add_x0.zero_()
            add_v.zero_()
            add_tri.zero_()
            B.bigram_fwd(t_in[i], 2, V, tx0, add_x0, h_x0[sl])
            B.bigram_fwd(t_in[i], 2, V, tv, add_v, h_v[sl])
            B.bigram_fwd(t_in[i], 3, V, ttri, add_tri)
            B.gpt_fwd_bwd(ctx, t_in[i], t_tg[i], params, grads, loss, 1.0 / MB, int(i > 0),
                          add_x0, add_v, add_tri, d_x0[sl], d_v[sl])
        B.bigram_bwd_update(h_x0, d_x0, tx0, v_x0, tc.lr, tc.beta2, tc.eps, ws)
        B.bigram_bwd_update(h_v, d_v, tv, v_v, tc.lr, tc.beta2, tc.eps, ws)

    ms, wall = time_steps(step, a.steps, a.warmup)
    lval = float(loss.item())
    assert np.isfinite(lval), lval
    # stages of the dense micro-batch step
    roof, parts = profile_stages(B, ctx, lambda: B.gpt_fwd_bwd(
        ctx, t_in[0], t_tg[0], params, grads, loss, 1.0 / MB, 1, add_x0, add_v, add_tri,
        d_x0[:N], d_v[:N]), a.profile_steps, True, multi_stages(B, cfg), a.workload)
    n_tok = MB * N
    tok_s = n_tok / (ms / 1e3)
    fpt = configs.flops_per_token(cfg)
    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Zipf tokens, N(0,0.02) weights and tables, N(0,1) trigram rows)",
        "config": {"workload": "speedrun-shaped optimizer step: gpt2-small + x0/value bigram "
                               "tables + frozen trigram, 24 x 8 x 1024 tokens",
                   "micro_batches": MB, "tokens_per_step": n_tok, "layers": cfg.n_layer,
                   "d_model": D, "vocab": V, "parallelism": "none (1 GPU)"},
        "mfu": round(fpt * tok_s / PEAK_BF16, 4), "flops_per_token": fpt,
        "loss_last_micro_batch": round(lval, 5), "wall_s": round(wall, 3),
        "roofline": roof, "parts_micro_batch": parts,
    }
    if not a.no_cpu_baseline:
        from oracle import tables as ot

        def addends(tok):
            rows = []
            for table, order, R in ((tx0, 2, tc.x0_rows), (tv, 2, tc.v_rows), (ttri, 3, tc.tri_rows)):
                h = ot.hash_indices(tok[:, :-1], order, V, R).reshape(-1)
                rows.append(table[torch.from_numpy(h).cuda()].float().cpu().numpy())
            return tuple(rows)
        out["cpu_baseline"] = cpu_baseline(cfg, params, tokens, min(a.cpu_tokens, T), addends)
    return out


def ns_groups(cfg):
    """(count, rows, cols) of every batch of Muon matrices (q/k/v/o blocks, MLP up, MLP down,
    trigram projection)."""
    D, F, L = cfg.d_model, cfg.d_mlp, cfg.n_layer
    g = [(4 * L, D, D), (L, F, D), (L, D, F)]
    if cfg.has_trigram:
        g.append((1, D, D))
    return g


def ns_work(cfg, steps=5, symmetric=True):
    """Newton-Schulz GEMM flops of one optimizer step and its launches (3 per step and batch):
    X X^T (2 S^2 L), c A A + b A (2 S^3), B X + a X (2 R C S), S = min(R, C), L = max(R, C).
    The first two results are symmetric and only their upper-triangle tiles are computed: a share
    (T + 1) / 2T of their flops for T = S / 256 tiles per side."""
    flops, launches = 0.0, 0
    for count, R, C in ns_groups(cfg):
        S, L = min(R, C), max(R, C)
        T = -(-S // 256)
        tri = (T + 1) / (2.0 * T) if symmetric else 1.0
        flops += count * steps * (tri * (2.0 * S * S * L + 2.0 * S ** 3) + 2.0 * R * C * S)
        launches += 3 * steps
    return flops, launches


def opt_bytes(cfg):
    """Algorithmic bytes of the optimizer's memory-bound kernels per step: the norm pass reads
    the gradients; the update reads them again with the fp32 weights and first moments (written
    back) and writes the bf16 copy; Adam also reads and writes its second moments; Muon writes
    its bf16 input, which the scaling reads and writes and the final update reads."""
    n = configs.param_elems(cfg)
    vd = cfg.vocab * cfg.d_model
    nm = sum(c * r * k for c, r, k in ns_groups(cfg))
    return 4 * n + (4 + 8 + 8 + 2) * n + 8 * 2 * vd + (2 + 4 + 2) * nm


def bench_opt(a, B):
    import torch
    cfg = configs.D32
    n = configs.param_elems(cfg)
    g = torch.Generator(device="cuda").manual_seed(inputs.seeds_for(cfg.name)["weights"])
    master = torch.randn(n, device="cuda", generator=g) * 0.02
    params = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    grads = torch.randn(n, device="cuda", generator=g) * 0.05
    state = torch.zeros(B.gpt_opt_state_elems(cfg), device="cuda")
    ws = torch.empty(B.gpt_opt_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    gnorm = torch.zeros(1, device="cuda")
    count = [0]

    def hp(ns_steps):
        count[0] += 1
        return dict(lr_matrix=0.02, lr_embedding=0.2, lr_unembedding=0.004,
                    lr_mult=B.gpt_lr_multiplier(0, 1000, 0.0, 0.2, 0.0),
                    momentum=B.gpt_muon_momentum(0), beta1=0.8, beta2=0.95, eps=1e-10,
                    weight_decay=0.0, grad_clip=1.0, nesterov=1, ns_steps=ns_steps,
                    adam_step=count[0])

    ms, wall = time_steps(lambda: B.gpt_opt_step(cfg, master, params, grads, state, hp(5), ws, gnorm),
                          a.steps, a.warmup)
    ms0, _ = time_steps(lambda: B.gpt_opt_step(cfg, master, params, grads, state, hp(0), ws, gnorm),
                        a.steps, a.warmup)
    assert np.isfinite(float(gnorm.item()))
    flops, launches = ns_work(cfg)
    ns_ms = max(ms - ms0, 1e-6)
    ach = flops / (ns_ms / 1e3)
    roof = {"bound": "mfma", "kernel": "Newton-Schulz batched GEMMs (gemm_dma_kernel, NS sites)",
            "achieved": round(ach / 1e12, 1), "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16, 4), "avg_launch_ms": round(ns_ms / launches, 4),
            "algorithmic_per_launch": flops / launches, "traffic": None,
            "launches_per_step": launches,
            "timing": "HIP events: the step with 5 Newton-Schulz steps minus the step with none"}
    nbytes = opt_bytes(cfg)
    parts = {"newton_schulz": {"ms_per_step": round(ns_ms, 3), "launches": launches,
                               "achieved": round(ach / 1e12, 1), "unit": "TFLOP/s",
                               "frac": round(ach / PEAK_BF16, 4)},
             "elementwise (clip, Adam, momentum, scaling, update)": {
                 "ms_per_step": round(ms0, 3), "achieved": round(nbytes / (ms0 / 1e3) / 1e9, 1),
                 "unit": "GB/s", "frac": round(nbytes / (ms0 / 1e3) / PEAK_HBM, 4)}}
    out = {"metric": "dense optimizer step time (clip + Adam + Muon with 5 bf16 Newton-Schulz steps)",
           "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
           "ms_per_step": round(ms, 3), "higher_is_better": False, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (N(0,0.02) weights, N(0,0.05) gradients)",
           "config": {"workload": f"{cfg.name} optimizer step", "params": n,
                      "muon_matrices": sum(c for c, _, _ in ns_groups(cfg))},
           "wall_s": round(wall, 3), "roofline": roof, "parts": parts}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_opt(cfg)
    return out


def cpu_baseline_opt(cfg):
    """The oracle's Muon update (fp64 numpy, bf16 Newton-Schulz) of one D x D matrix, scaled to
    the whole step by Newton-Schulz flops."""
    from threadpoolctl import threadpool_limits
    from oracle import optim as oo
    cores = _cores()
    rng = np.random.default_rng(5)
    D = cfg.d_model
    p = rng.standard_normal((D, D)) * 0.02
    g = rng.standard_normal((D, D)) * 0.05
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        oo.muon_update(p, g, np.zeros_like(g), 0.02, 0.85, True, 5, bf16=True)
        dt = time.perf_counter() - t0
    flops, _ = ns_work(cfg, symmetric=False)  # the oracle computes every product in full
    one = 5 * (2.0 * D ** 3 * 3)
    return {"value": round(dt * flops / one * 1e3, 1), "unit": "ms", "cores": cores, "kind": "oracle",
            "sample": f"one {D} x {D} Muon update with 5 bf16 Newton-Schulz steps (fp64 numpy), "
                      f"{dt:.1f} s, scaled to the step's Newton-Schulz flops"}


def decode_bytes(cfg, batch, p_first, steps):
    """Algorithmic HBM bytes per decode step, averaged over `steps` steps whose new tokens sit at
    positions p_first, p_first + 1, ...: every weight matrix and the LM head read once (bf16), one
    embedding row per sequence, the cached keys and values of every attended position read and
    the new ones written, the fp32 logits written and read back by the sampler."""
    D, F, L, V = cfg.d_model, cfg.d_mlp, cfg.n_layer, cfg.vocab
    kv_row = 2 * D * 2                              # one position's key + value, one layer, bf16
    weights = L * (4 * D * D + 2 * D * F) * 2 + V * D * 2
    total = 0.0
    for s in range(steps):
        attended = p_first + s + 1
        total += (weights + batch * D * 2 + L * batch * kv_row * (attended + 1)
                  + batch * V * 4 * 2)
    return total / steps


def bench_decode(a, B):
    import torch
    cfg = configs.D32
    batch, prompt, top_k, temperature = 8, 1024, 50, 1.0
    seeds = inputs.seeds_for(cfg.name)
    flat = inputs.device_params(cfg, seeds["weights"])
    prof_steps = max(a.profile_steps, 1)
    max_seq = prompt + a.warmup + a.steps + prof_steps
    ctx = B.gpt_infer_init(cfg, batch, max_seq)
    g = torch.Generator(device="cuda").manual_seed(seeds["tokens"])
    u = torch.rand(a.warmup + a.steps + prof_steps + 1, batch, device="cuda", generator=g)
    tok = torch.from_numpy(inputs.zipf_tokens(seeds["tokens"], (batch, prompt), cfg.vocab)).cuda()
    logits = torch.empty(batch, cfg.vocab, device="cuda")
    nxt = torch.empty(batch, 1, dtype=torch.int32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    B.gpt_infer_forward(ctx, flat, tok, logits)
    e1.record()
    B.gpt_sample(logits, temperature, top_k, u[0], nxt.view(-1))
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    i = [1]

    def step():
        B.gpt_infer_forward(ctx, flat, nxt, logits)
        B.gpt_sample(logits, temperature, top_k, u[i[0]], nxt.view(-1))
        i[0] += 1

    ms, wall = time_steps(step, a.steps, a.warmup)
    ids = nxt.view(-1).cpu().numpy()
    assert ((ids >= 0) & (ids < cfg.vocab)).all() and np.isfinite(logits.cpu().numpy()).all()
    nbytes = decode_bytes(cfg, batch, prompt + a.warmup, a.steps)
    ach = nbytes / (ms / 1e3)
    step_roof = {"bound": "hbm", "kernel": "decode step (all kernels)", "achieved": round(ach / 1e9, 1),
                 "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": round(ach / PEAK_HBM, 4),
                 "algorithmic_per_step": nbytes}
    # instrumented pass: every launch of a few more steps bracketed by events on the stream
    B.gpt_infer_profile(ctx, True)
    for _ in range(prof_steps):
        step()
    B.gpt_infer_profile(ctx, False)
    stages = B.gpt_infer_profile_read(ctx)
    torch.cuda.synchronize()
    parts = {}
    for n, c, m, f, b in stages:
        e = _roof_entry_by_intensity(n, c, m, f, b)
        parts[n] = {"ms_per_step": round(m / prof_steps, 4), "launches": c // prof_steps,
                    "achieved": e["achieved"], "unit": e["unit"], "frac": e["frac"]}
    name, calls, tot_ms, flops, nb = max(stages, key=lambda x: x[2])
    roof = _roof_entry_by_intensity(name, calls, tot_ms, flops, nb)
    roof["traffic"] = measured_traffic("decode", name)
    roof["launches_per_step"] = calls // prof_steps
    out = {"metric": "decode tokens/sec (KV-cached forward + top-k sampling) on 1 MI355X",
           "value": round(batch / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (device-drawn N(0,0.02) weights, Zipf prompt tokens)",
           "config": {"workload": f"{cfg.name} decode", "batch": batch, "prompt": prompt,
                      "top_k": top_k, "temperature": temperature},
           "prefill_ms": round(prefill_ms, 3),
           "prefill_tokens_per_s": round(batch * prompt / (prefill_ms / 1e3), 1),
           "wall_s": round(wall, 3), "roofline": roof, "step_roofline": step_roof, "parts": parts}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(cfg, flat, tok.cpu().numpy())
    return out


def cpu_baseline_decode(cfg, flat_dev, tokens, n_tok=96):
    """The oracle (fp64 numpy, no cache: the full forward over the prefix) producing one next-token
    distribution for one sequence of n_tok tokens."""
    from threadpoolctl import threadpool_limits
    from oracle import infer as oinf
    cores = _cores()
    params = inputs.unflatten(cfg, flat_dev.float().cpu().numpy())
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        z = oinf.next_logits(cfg, params, tokens[:1, :n_tok])
        dt = time.perf_counter() - t0
    assert np.isfinite(z).all()
    return {"value": round(1.0 / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"next-token logits of 1 sequence after {n_tok} tokens of the {cfg.name} "
                      f"model (fp64 numpy full forward, as the oracle has no cache), {dt:.1f} s"}


def main():
    a = parse()
    if a.record_traffic:
        record_traffic(a)
        return
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
    if a.workload == "copy":
        out = bench_copy(a)
    elif a.workload == "gemm_ref":
        out = bench_gemm_ref(a, B)
    elif a.workload == "tables":
        out = bench_tables(a, B)
    elif a.workload == "speedrun":
        out = bench_speedrun(a, B)
    elif a.workload == "opt":
        out = bench_opt(a, B)
    elif a.workload == "decode":
        out = bench_decode(a, B)
    else:
        out = bench_dense(a, B)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
