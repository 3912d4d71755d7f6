"""The C-ABI library loads, exports every declared symbol, and its host-side logic (layout,
workspace sizing, argument validation) works without a GPU.  No kernel is launched here."""
import ctypes as C
import os
import re

import pytest

from gpt_lm_step_amd import binding as B
from gpt_lm_step_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in ("gpt.h", "gpt_kernels.h"):
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M):
            if m.group(1) not in ("if", "return", "sizeof"):
                names.add(m.group(1))
    return names


def test_library_exports_every_declared_symbol():
    declared = _declared_functions()
    assert set(B.EXPORTS) | set(B.KERNEL_EXPORTS) == declared
    lib = B.lib()
    for name in sorted(declared):
        assert hasattr(lib, name), name


@pytest.mark.parametrize("cfg", list(configs.PRESETS.values()), ids=list(configs.PRESETS))
def test_param_layout_matches_python_layout(cfg):
    got, total = B.gpt_param_layout(cfg)
    want = configs.param_layout(cfg)
    assert [(n, o, tuple(s)) for n, o, s in got] == [(n, o, tuple(s)) for n, o, s in want]
    assert total == configs.param_elems(cfg)


def test_d32_layout_counts_the_page_parameters():
    got, _ = B.gpt_param_layout(configs.D32)
    assert sum(s[0] * s[1] for _, _, s in got) == 1_879_048_192


def test_workspace_sizes_are_plausible():
    small = B.gpt_workspace_bytes(configs.TINY)
    big = B.gpt_workspace_bytes(configs.D32)
    assert 0 < small < 64 << 20
    # d32 stashes ~1.2 GB of activations per layer plus 2 GB of bf16 logits
    assert 30e9 < big < 80e9


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 48, B.GPT_ESHAPE), ("n_kv_head", 2, B.GPT_ESHAPE), ("vocab", 500, B.GPT_ESHAPE),
    ("seq_len", 100, B.GPT_ESHAPE), ("dtype", 7, B.GPT_EINVAL), ("n_layer", 0, B.GPT_ESHAPE),
    ("vocab", 65536 + 64, B.GPT_ESHAPE), ("d_model", 4096, B.GPT_ESHAPE),
    ("ce_chunk_tokens", 100, B.GPT_ESHAPE), ("ce_chunk_tokens", -64, B.GPT_ESHAPE),
    ("wgrad_stream", 2, B.GPT_EINVAL), ("wgrad_stream", -2, B.GPT_EINVAL),
])
def test_invalid_configs_are_rejected(field, value, status):
    c = B.make_config(configs.TINY)
    setattr(c, field, value)
    if field == "head_dim":
        c.n_head = 1
        c.d_model = 48 * 1
    b = C.c_size_t(0)
    assert B.lib().gpt_workspace_bytes(C.byref(c), C.byref(b)) == status
    assert len(B.lib().gpt_last_error()) > 0


def _splitk_bytes(cfg, rows):
    """Split-K scratch of a bf16 step: the largest partial set of its fp32-output products (the
    four weight gradients of a block, the LM head's weight and input gradients over `rows`)."""
    n, d, f, V = cfg.tokens, cfg.d_model, cfg.d_mlp, cfg.vocab
    ws = B.gptk_gemm_wgrad_ws_floats
    return 4 * max(ws(3 * d, d, n), ws(d, d, n), ws(d, f, n), ws(f, d, n), ws(V, d, rows),
                   ws(rows, d, V))


def test_cross_entropy_chunk_shrinks_the_workspace_by_its_logits():
    """A chunk of C tokens keeps a [C, vocab] logits buffer instead of [N, vocab]; everything
    else in the workspace is the same (d32: 2 GiB of bf16 logits at the default) except the
    split-K scratch, which follows the LM head's products over C rows."""
    cfg = configs.D32
    whole = B.gpt_workspace_bytes(cfg)
    chunked = B.gpt_workspace_bytes(cfg.replace(ce_chunk_tokens=4096))
    V, N = cfg.vocab, cfg.tokens
    diff = whole - chunked
    want = (N - 4096) * V * 2 + _splitk_bytes(cfg, N) - _splitk_bytes(cfg, 4096)
    assert abs(diff - want) <= 4096, (diff, want)
    # a chunk larger than the batch is the whole batch
    assert B.gpt_workspace_bytes(configs.TINY.replace(ce_chunk_tokens=1 << 20)) == \
        B.gpt_workspace_bytes(configs.TINY)


def test_init_rejects_missing_or_small_workspace():
    c = B.make_config(configs.TINY)
    h = C.c_void_p()
    assert B.lib().gpt_init(C.byref(c), None, 0, None, C.byref(h)) == B.GPT_EWORKSPACE
    # a fake, aligned, too-small "workspace" address: rejected before any use
    assert B.lib().gpt_init(C.byref(c), 1 << 20, 1024, None, C.byref(h)) == B.GPT_EWORKSPACE
    assert B.lib().gpt_init(C.byref(c), (1 << 20) + 8, 1 << 40, None, C.byref(h)) == B.GPT_EINVAL


def test_fp32_path_rejects_head_dim_128():
    cfg = configs.TINY.replace(n_head=1, head_dim=128)
    c = B.make_config(cfg)
    h = C.c_void_p()
    n = B.gpt_workspace_bytes(cfg)
    assert B.lib().gpt_init(C.byref(c), 1 << 20, n, None, C.byref(h)) == B.GPT_ESHAPE


def test_fwd_bwd_argument_checks_without_gpu():
    L = B.lib()
    assert L.gpt_fwd_bwd(None, 1, 1, 1, 1, 1.0, 0, None, None, None, None, None, 1, None) == B.GPT_EINVAL


def test_table_entry_point_validation():
    L = B.lib()
    # bigram_fwd: bad order, bad dim, bad rows, null pointers
    assert L.bigram_fwd(16, 2, 4, 4, 100, 16, 1000, 64, B.BF16, 16, None, None) == B.GPT_EINVAL
    assert L.bigram_fwd(16, 2, 4, 2, 100, 16, 1000, 60, B.BF16, 16, None, None) == B.GPT_ESHAPE
    assert L.bigram_fwd(16, 2, 4, 2, 100, 16, 0, 64, B.BF16, 16, None, None) == B.GPT_ERANGE
    assert L.bigram_fwd(None, 2, 4, 2, 100, 16, 1000, 64, B.BF16, 16, None, None) == B.GPT_EINVAL
    assert L.bigram_fwd(None, 0, 4, 2, 100, None, 1000, 64, B.BF16, None, None, None) == B.GPT_OK
    # bigram_bwd_update: n = 0 is a no-op; too little workspace is refused
    assert L.bigram_bwd_update(None, None, 0, 64, B.BF16, None, None, 10, 0.1, 0.95, 1e-8, None, 0, None) == B.GPT_OK
    need = L.bigram_workspace_bytes(1000, 64)
    assert need > 1000 * 16
    assert L.bigram_bwd_update(16, 16, 1000, 64, B.BF16, 16, 16, 1 << 20, 0.1, 0.95, 1e-8, 256,
                               need - 1, None) == B.GPT_EWORKSPACE
    assert L.bigram_bwd_update(16, 16, 1000, 4096, B.BF16, 16, 16, 1 << 20, 0.1, 0.95, 1e-8, 256,
                               need, None) == B.GPT_ESHAPE


def test_status_strings():
    for s in (B.GPT_OK, B.GPT_EINVAL, B.GPT_ESHAPE, B.GPT_ERANGE, B.GPT_EWORKSPACE, B.GPT_EHIP):
        assert B.lib().gpt_status_string(s).decode() not in ("", "unknown status")


@pytest.mark.parametrize("M,N,K,splits", [
    # shapes of the shipped workloads: the measured per-shape plans
    (768, 768, 8192, 4), (2304, 768, 8192, 4), (3072, 768, 8192, 2), (768, 3072, 8192, 2),
    (2048, 2048, 16384, 4), (6144, 2048, 16384, 1),
    # other shapes: the general rule
    (640, 640, 8192, 16), (2560, 1536, 16384, 8), (6144, 2048, 65536, 4),
    (2048, 8192, 65536, 1), (50304, 768, 8192, 1), (256, 384, 128, 1), (768, 768, 1024, 2), (768, 768, 1016, 1)])
def test_wgrad_split_k_workspace(M, N, K, splits):
    """Split-K weight-gradient plan: one fp32 M x N partial per split, none when not split."""
    assert B.gptk_gemm_wgrad_ws_floats(M, N, K) == (splits * M * N if splits > 1 else 0)
    assert B.gptk_gemm_wgrad_ws_floats(0, N, K) == 0


def test_optimizer_schedules_match_hand_worked_values():
    """The library's host schedules against the same hand-worked values as the oracle's."""
    path = os.path.join(ROOT, "tests", "golden", "optim_schedules.txt")
    for line in open(path):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        if f[0] == "lr":
            got = B.gpt_lr_multiplier(int(f[1]), int(f[2]), float(f[3]), float(f[4]), float(f[5]))
        else:
            got = B.gpt_muon_momentum(int(f[1]))
        assert got == pytest.approx(float(f[-1]), abs=1e-12), line


@pytest.mark.parametrize("cfg", list(configs.PRESETS.values()), ids=list(configs.PRESETS))
def test_optimizer_state_and_workspace_sizes(cfg):
    total = configs.param_elems(cfg)
    vd = cfg.vocab * cfg.d_model
    assert B.gpt_opt_state_elems(cfg) == total + 2 * ((vd + 63) // 64 * 64)
    ws = B.gpt_opt_workspace_bytes(cfg)
    D, F, L = cfg.d_model, cfg.d_mlp, cfg.n_layer
    # the q/k/v/o group: X, X' (4L matrices of D x D) and A, B (D x D each) in bf16
    assert ws >= 4 * (4 * L * D * D * 2)
    assert ws >= 2 * (L * F * D * 2)


def test_optimizer_step_argument_checks_without_gpu():
    cfg = configs.TINY
    c = B.make_config(cfg)
    L = B.lib()
    hp = B.gpt_opt_hparams(0.02, 0.2, 0.004, 1.0, 0.95, 0.8, 0.95, 1e-10, 0.0, 1.0, 1, 5, 1)
    need = B.gpt_opt_workspace_bytes(cfg)
    args = lambda ws, n, h=hp: L.gpt_opt_step(C.byref(c), 256, None, 256, 256, C.byref(h), ws, n, None, None)
    assert args(None, need) == B.GPT_EINVAL                       # no workspace
    assert args(256, need - 1) == B.GPT_EWORKSPACE               # too small
    bad = B.gpt_opt_hparams(0.02, 0.2, 0.004, 1.0, 0.95, 0.8, 1.5, 1e-10, 0.0, 1.0, 1, 5, 1)
    assert args(256, need, bad) == B.GPT_ERANGE                   # beta2 >= 1
    zero_step = B.gpt_opt_hparams(0.02, 0.2, 0.004, 1.0, 0.95, 0.8, 0.95, 1e-10, 0.0, 1.0, 1, 5, 0)
    assert args(256, need, zero_step) == B.GPT_ERANGE             # Adam step count starts at 1
    assert L.gpt_opt_step(C.byref(c), None, None, 256, 256, C.byref(hp), 256, need, None, None) == B.GPT_EINVAL


@pytest.mark.parametrize("cfg", [configs.TINY, configs.D32], ids=["tiny", "d32"])
def test_inference_workspace_holds_the_cache(cfg):
    cfg = cfg.replace(has_x0_add=0, has_v_add=0, has_trigram=0)
    esz = 2 if cfg.dtype == B.BF16 else 4
    b1 = B.gpt_infer_workspace_bytes(cfg, 4, 256)
    b2 = B.gpt_infer_workspace_bytes(cfg, 4, 512)
    cache = 2 * cfg.n_layer * 4 * cfg.n_head * 256 * cfg.head_dim * esz
    assert b1 >= cache
    # every buffer but the last-position ones scales with max_seq: the cache, rotary tables and
    # per-token activations (fp32 residual, qkv, attention, MLP)
    per_tok = (2 * cfg.n_layer * cfg.n_head * cfg.head_dim + 3 * cfg.d_model + cfg.d_mlp) * esz * 4
    assert b2 - b1 >= 256 * per_tok


def test_inference_argument_checks_without_gpu():
    L = B.lib()
    cfg = configs.TINY.replace(has_x0_add=0, has_v_add=0, has_trigram=0)
    c = B.make_config(cfg)
    sz = C.c_size_t(0)
    assert L.gpt_infer_workspace_bytes(C.byref(c), 1, 8193, C.byref(sz)) == B.GPT_ESHAPE
    assert L.gpt_infer_workspace_bytes(C.byref(c), 0, 64, C.byref(sz)) == B.GPT_ESHAPE
    assert L.gpt_infer_workspace_bytes(C.byref(c), 1, 64, None) == B.GPT_EINVAL
    need = B.gpt_infer_workspace_bytes(cfg, 2, 64)
    h = C.c_void_p()
    assert L.gpt_infer_init(C.byref(c), 2, 64, None, need, None, C.byref(h)) == B.GPT_EWORKSPACE
    assert L.gpt_infer_init(C.byref(c), 2, 64, 256, need - 1, None, C.byref(h)) == B.GPT_EWORKSPACE
    assert L.gpt_infer_init(C.byref(c), 2, 64, 4100, need, None, C.byref(h)) == B.GPT_EWORKSPACE
    tables = B.make_config(configs.TINY.replace(has_x0_add=1))
    assert L.gpt_infer_init(C.byref(tables), 2, 64, 256, 1 << 40, None, C.byref(h)) == B.GPT_EINVAL
    assert L.gpt_infer_position(None) == -1
    assert L.gpt_infer_reset(None) == B.GPT_EINVAL
    assert L.gpt_infer_forward(None, 256, 256, 1, 1, 256, None) == B.GPT_EINVAL
    assert L.gpt_infer_profile(None, 1) == B.GPT_EINVAL
    assert L.gpt_infer_check_errors(None, None, C.byref(C.c_int32(0))) == B.GPT_EINVAL
    assert L.gpt_infer_profile_read(None, None, C.byref(C.c_int32(0))) == B.GPT_EINVAL
    assert L.gpt_sample(None, 0, 10, 1.0, 0, None, None, None) == B.GPT_OK          # empty batch
    assert L.gpt_sample(256, 1, 0, 1.0, 0, 256, 256, None) == B.GPT_ESHAPE
    assert L.gpt_sample(256, 1, 65537, 1.0, 0, 256, 256, None) == B.GPT_ESHAPE
    assert L.gpt_sample(256, 1, 10, -1.0, 0, 256, 256, None) == B.GPT_ERANGE
    assert L.gpt_sample(256, 1, 10, 1.0, -2, 256, 256, None) == B.GPT_ERANGE
    assert L.gpt_sample(256, 1, 10, 1.0, 0, None, 256, None) == B.GPT_EINVAL       # no uniforms
