"""ctypes binding of libgpt.so: the C ABI of include/gpt.h under the same names.

Argument marshalling only: torch tensors give device pointers and the current HIP stream;
every step of the computation runs in the library's kernels.  Loading fails loudly when the
library is missing (run gpt_lm_step_amd.build first); there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import List, Optional, Tuple

from .configs import GPTConfig

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgpt.so")
_lib = None

GPT_OK, GPT_EINVAL, GPT_ESHAPE, GPT_ERANGE, GPT_EWORKSPACE, GPT_EHIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1

# Every symbol include/gpt.h declares.
EXPORTS = [
    "gpt_param_layout", "gpt_workspace_bytes", "gpt_init", "gpt_fwd_bwd", "gpt_check_errors",
    "gpt_profile", "gpt_profile_read", "gpt_destroy", "bigram_fwd", "bigram_workspace_bytes", "bigram_bwd_update",
    "bigram_bwd_update_noalloc",
    "gpt_last_error", "gpt_status_string", "gpt_opt_state_elems", "gpt_opt_workspace_bytes",
    "gpt_opt_step", "gpt_lr_multiplier", "gpt_muon_momentum", "gpt_infer_workspace_bytes",
    "gpt_infer_init", "gpt_infer_reset", "gpt_infer_position", "gpt_infer_forward",
    "gpt_infer_profile", "gpt_infer_profile_read", "gpt_infer_check_errors", "gpt_infer_destroy",
    "gpt_sample",
]
# Every symbol include/gpt_kernels.h declares.
KERNEL_EXPORTS = [
    "gptk_gemm", "gptk_gemm_wgrad", "gptk_gemm_wgrad_ws_floats", "gptk_rmsnorm_fwd", "gptk_rmsnorm_bwd", "gptk_rope_table",
    "gptk_rope_qknorm_fwd", "gptk_rope_qknorm_bwd", "gptk_qkv_rope_fwd", "gptk_attention_fwd",
    "gptk_attention_bwd",
    "gptk_softcap_ce",
]


class GptError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class gpt_config(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("n_layer", "d_model", "n_head", "n_kv_head", "head_dim",
                                         "d_mlp", "vocab", "seq_len", "batch", "dtype")] + \
               [("rms_eps", C.c_float), ("rope_base", C.c_float), ("softcap", C.c_float)] + \
               [(n, C.c_int32) for n in ("qk_norm", "has_x0_add", "has_v_add", "has_trigram",
                                         "ce_chunk_tokens", "wgrad_stream")]


class gpt_profile_entry(C.Structure):
    _fields_ = [("name", C.c_char * 32), ("calls", C.c_int32), ("ms", C.c_float),
                ("flops", C.c_double), ("bytes", C.c_double)]


class gpt_tensor_desc(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("offset_elems", C.c_int64), ("ndim", C.c_int32),
                ("shape", C.c_int64 * 2)]


class gpt_opt_hparams(C.Structure):
    _fields_ = [("lr_matrix", C.c_float), ("lr_embedding", C.c_float),
                ("lr_unembedding", C.c_float), ("lr_mult", C.c_float), ("momentum", C.c_float),
                ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("grad_clip", C.c_float), ("nesterov", C.c_int32),
                ("ns_steps", C.c_int32), ("adam_step", C.c_int64)]


def lib() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m gpt_lm_step_amd.build` (no fallback exists)")
        L = C.CDLL(_LIB_PATH)
        vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
        cfgp = C.POINTER(gpt_config)
        sig = {
            "gpt_param_layout": (i32, [cfgp, vp, C.POINTER(i32), C.POINTER(i64)]),
            "gpt_workspace_bytes": (i32, [cfgp, C.POINTER(sz)]),
            "gpt_init": (i32, [cfgp, vp, sz, vp, C.POINTER(vp)]),
            "gpt_fwd_bwd": (i32, [vp, vp, vp, vp, vp, f32, i32, vp, vp, vp, vp, vp, vp, vp]),
            "gpt_check_errors": (i32, [vp, vp, C.POINTER(i32)]),
            "gpt_destroy": (i32, [vp]),
            "gpt_profile": (i32, [vp, i32]),
            "gpt_profile_read": (i32, [vp, vp, C.POINTER(i32)]),
            "bigram_fwd": (i32, [vp, i32, i32, i32, i32, vp, i64, i32, i32, vp, vp, vp]),
            "bigram_workspace_bytes": (sz, [i64, i32]),
            "bigram_bwd_update": (i32, [vp, vp, i64, i32, i32, vp, vp, i64, f32, f32, f32, vp,
                                        sz, vp]),
            "bigram_bwd_update_noalloc": (i32, [vp, vp, i64, i32, i32, vp, vp, i64, f32, f32,
                                                f32, vp]),
            "gpt_last_error": (C.c_char_p, []),
            "gpt_status_string": (C.c_char_p, [i32]),
            "gptk_gemm": (i32, [i32, i32, i32, i32, i32, i32, vp, i64, vp, i64, vp, i64, i32, vp]),
            "gptk_gemm_wgrad": (i32, [i32, i32, i32, i32, i32, i32, vp, i64, vp, i64, vp, i64, i32,
                                      vp, i64, vp]),
            "gptk_gemm_wgrad_ws_floats": (i64, [i32, i32, i32]),
            "gptk_rmsnorm_fwd": (i32, [i32, vp, vp, vp, i64, i32, f32, vp]),
            "gptk_rmsnorm_bwd": (i32, [i32, vp, vp, vp, vp, vp, vp, i64, i32, vp]),
            "gptk_rope_table": (i32, [i32, vp, vp, i32, i32, f32, vp]),
            "gptk_rope_qknorm_fwd": (i32, [i32, vp, vp, vp, vp, i64, i32, i32, i32, i32, f32, vp]),
            "gptk_rope_qknorm_bwd": (i32, [i32, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, vp]),
            "gptk_qkv_rope_fwd": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i32, i32, i32, i32, f32,
                                        vp]),
            "gptk_attention_fwd": (i32, [i32, vp, vp, vp, i32, i32, i32, i32, vp]),
            "gptk_attention_bwd": (i32, [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]),
            "gptk_softcap_ce": (i32, [i32, vp, i64, vp, i64, i32, f32, f32, vp, vp, vp]),
            "gpt_opt_state_elems": (i64, [cfgp]),
            "gpt_opt_workspace_bytes": (i32, [cfgp, C.POINTER(sz)]),
            "gpt_opt_step": (i32, [cfgp, vp, vp, vp, vp, C.POINTER(gpt_opt_hparams), vp, sz, vp,
                                   vp]),
            "gpt_lr_multiplier": (C.c_double, [i64, i64, C.c_double, C.c_double, C.c_double]),
            "gpt_muon_momentum": (C.c_double, [i64]),
            "gpt_infer_workspace_bytes": (i32, [cfgp, i32, i32, C.POINTER(sz)]),
            "gpt_infer_init": (i32, [cfgp, i32, i32, vp, sz, vp, C.POINTER(vp)]),
            "gpt_infer_reset": (i32, [vp]),
            "gpt_infer_position": (i32, [vp]),
            "gpt_infer_forward": (i32, [vp, vp, vp, i32, i32, vp, vp]),
            "gpt_infer_profile": (i32, [vp, i32]),
            "gpt_infer_profile_read": (i32, [vp, vp, C.POINTER(i32)]),
            "gpt_infer_check_errors": (i32, [vp, vp, C.POINTER(i32)]),
            "gpt_infer_destroy": (i32, [vp]),
            "gpt_sample": (i32, [vp, i32, i32, f32, i32, vp, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int):
    if status != GPT_OK:
        raise GptError(status, lib().gpt_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def make_config(cfg: GPTConfig) -> gpt_config:
    return gpt_config(cfg.n_layer, cfg.d_model, cfg.n_head, cfg.n_kv_head, cfg.head_dim,
                      cfg.d_mlp, cfg.vocab, cfg.seq_len, cfg.batch, cfg.dtype, cfg.rms_eps,
                      cfg.rope_base, cfg.softcap, cfg.qk_norm, cfg.has_x0_add, cfg.has_v_add,
                      cfg.has_trigram, cfg.ce_chunk_tokens, cfg.wgrad_stream)


def gpt_param_layout(cfg: GPTConfig) -> Tuple[List[Tuple[str, int, Tuple[int, int]]], int]:
    c = make_config(cfg)
    n = C.c_int32(0)
    total = C.c_int64(0)
    _check(lib().gpt_param_layout(C.byref(c), None, C.byref(n), C.byref(total)))
    arr = (gpt_tensor_desc * n.value)()
    _check(lib().gpt_param_layout(C.byref(c), arr, C.byref(n), C.byref(total)))
    out = [(d.name.decode(), d.offset_elems, (d.shape[0], d.shape[1])) for d in arr]
    return out, total.value


def gpt_workspace_bytes(cfg: GPTConfig) -> int:
    c = make_config(cfg)
    b = C.c_size_t(0)
    _check(lib().gpt_workspace_bytes(C.byref(c), C.byref(b)))
    return b.value


class Context:
    """A gpt_ctx plus the workspace tensor that backs it."""

    def __init__(self, cfg: GPTConfig, stream=None):
        import torch
        self.cfg = cfg
        self._c = make_config(cfg)
        nbytes = gpt_workspace_bytes(cfg)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        h = C.c_void_p()
        _check(lib().gpt_init(C.byref(self._c), self.workspace.data_ptr(), nbytes,
                              _stream(stream), C.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            _check(lib().gpt_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gpt_init(cfg: GPTConfig, stream=None) -> Context:
    return Context(cfg, stream)


def gpt_fwd_bwd(ctx: Context, tokens, targets, params, grads, loss, grad_scale: float = 1.0,
                accumulate: int = 0, x0_add=None, v_add=None, tri_rows=None, d_x0_add=None,
                d_v_add=None, stream=None):
    _check(lib().gpt_fwd_bwd(ctx.handle, _ptr(tokens), _ptr(targets), _ptr(params), _ptr(grads),
                             float(grad_scale), int(accumulate), _ptr(x0_add), _ptr(v_add),
                             _ptr(tri_rows), _ptr(d_x0_add), _ptr(d_v_add), _ptr(loss),
                             _stream(stream)))


def gpt_check_errors(ctx: Context, stream=None) -> int:
    f = C.c_int32(0)
    _check(lib().gpt_check_errors(ctx.handle, _stream(stream), C.byref(f)))
    return f.value


def gpt_profile(ctx: Context, enable: bool):
    _check(lib().gpt_profile(ctx.handle, int(bool(enable))))


def gpt_profile_read(ctx: Context):
    """[(name, calls, ms, flops, bytes)] aggregated per stage since profiling was enabled."""
    n = C.c_int32(0)
    arr = (gpt_profile_entry * 256)()
    n.value = 256
    _check(lib().gpt_profile_read(ctx.handle, arr, C.byref(n)))
    return [(arr[i].name.decode(), arr[i].calls, arr[i].ms, arr[i].flops, arr[i].bytes)
            for i in range(min(n.value, 256))]


def gpt_destroy(ctx: Context):
    ctx.close()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def bigram_fwd(tokens, order: int, vocab: int, table, y, h_out=None, stream=None):
    B, T = tokens.shape
    _check(lib().bigram_fwd(_ptr(tokens), B, T, order, vocab, _ptr(table), table.shape[0],
                            table.shape[1], _dtype_code(table), _ptr(y), _ptr(h_out),
                            _stream(stream)))


def bigram_workspace_bytes(n: int, dim: int) -> int:
    return int(lib().bigram_workspace_bytes(n, dim))


def bigram_bwd_update(h, dy, table, v, lr: float, beta2: float = 0.95, eps: float = 1e-8,
                      workspace=None, stream=None):
    import torch
    n, dim = dy.shape[0], dy.shape[1]
    need = bigram_workspace_bytes(n, dim)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dy.device)
    _check(lib().bigram_bwd_update(_ptr(h), _ptr(dy), n, dim, _dtype_code(table), _ptr(table),
                                   _ptr(v), table.shape[0], float(lr), float(beta2), float(eps),
                                   _ptr(workspace), workspace.numel(), _stream(stream)))


def bigram_bwd_update_noalloc(h, dy, table, v, lr: float, beta2: float = 0.95,
                              eps: float = 1e-8, stream=None):
    n, dim = dy.shape[0], dy.shape[1]
    _check(lib().bigram_bwd_update_noalloc(_ptr(h), _ptr(dy), n, dim, _dtype_code(table),
                                           _ptr(table), _ptr(v), table.shape[0], float(lr),
                                           float(beta2), float(eps), _stream(stream)))


# ---------------------------------------------------------------- per-kernel entry points

def gptk_gemm(a_kc: bool, b_kc: bool, M: int, N: int, K: int, A, lda: int, B, ldb: int, C,
              ldc: int, beta: int = 0, stream=None):
    _check(lib().gptk_gemm(_dtype_code(A), int(a_kc), int(b_kc), M, N, K, _ptr(A), lda, _ptr(B),
                           ldb, _ptr(C), ldc, int(beta), _stream(stream)))


def gptk_gemm_wgrad_ws_floats(M: int, N: int, K: int) -> int:
    return int(lib().gptk_gemm_wgrad_ws_floats(M, N, K))


def gptk_gemm_wgrad(a_kc: bool, b_kc: bool, M: int, N: int, K: int, A, lda: int, B, ldb: int, C,
                    ldc: int, beta: int = 0, ws=None, stream=None):
    _check(lib().gptk_gemm_wgrad(_dtype_code(A), int(a_kc), int(b_kc), M, N, K, _ptr(A), lda,
                                 _ptr(B), ldb, _ptr(C), ldc, int(beta), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(stream)))


def gptk_rmsnorm_fwd(x, y, rstd, eps: float = 1e-6, stream=None):
    N, D = x.shape
    _check(lib().gptk_rmsnorm_fwd(_dtype_code(y), _ptr(x), _ptr(y), _ptr(rstd), N, D, eps,
                                  _stream(stream)))


def gptk_rmsnorm_bwd(x, rstd, dy, dres, dx, dx_t=None, stream=None):
    N, D = x.shape
    code = _dtype_code(dx_t) if dx_t is not None else F32
    _check(lib().gptk_rmsnorm_bwd(code, _ptr(x), _ptr(rstd), _ptr(dy), _ptr(dres), _ptr(dx),
                                  _ptr(dx_t), N, D, _stream(stream)))


def gptk_rope_table(cos_t, sin_t, T: int, hd: int, base: float = 10000.0, stream=None):
    _check(lib().gptk_rope_table(_dtype_code(cos_t), _ptr(cos_t), _ptr(sin_t), T, hd, base,
                                 _stream(stream)))


def gptk_rope_qknorm_fwd(qkv, cos_t, sin_t, rstd_qk, T: int, H: int, hd: int, qk_norm: int = 1,
                         eps: float = 1e-6, stream=None):
    _check(lib().gptk_rope_qknorm_fwd(_dtype_code(qkv), _ptr(qkv), _ptr(cos_t), _ptr(sin_t),
                                      _ptr(rstd_qk), qkv.shape[0], T, H, hd, qk_norm, eps,
                                      _stream(stream)))


def gptk_rope_qknorm_bwd(dqkv, qkv, cos_t, sin_t, rstd_qk, T: int, H: int, hd: int,
                         qk_norm: int = 1, stream=None):
    _check(lib().gptk_rope_qknorm_bwd(_dtype_code(qkv), _ptr(dqkv), _ptr(qkv), _ptr(cos_t),
                                      _ptr(sin_t), _ptr(rstd_qk), qkv.shape[0], T, H, hd,
                                      qk_norm, _stream(stream)))


def gptk_qkv_rope_fwd(x, wqkv, qkv, cos_t, sin_t, rstd_qk, u, T: int, H: int, hd: int,
                      qk_norm: int = 1, eps: float = 1e-6, stream=None):
    _check(lib().gptk_qkv_rope_fwd(_ptr(x), _ptr(wqkv), _ptr(qkv), _ptr(cos_t), _ptr(sin_t),
                                   _ptr(rstd_qk), _ptr(u), x.shape[0], T, H, hd, int(qk_norm),
                                   float(eps), _stream(stream)))


def gptk_attention_fwd(qkv, out, lse2, B: int, T: int, H: int, hd: int, stream=None):
    _check(lib().gptk_attention_fwd(_dtype_code(qkv), _ptr(qkv), _ptr(out), _ptr(lse2), B, T, H,
                                    hd, _stream(stream)))


def gptk_attention_bwd(qkv, out, dout, lse2, scratch, dqkv, B: int, T: int, H: int, hd: int,
                       stream=None):
    _check(lib().gptk_attention_bwd(_dtype_code(qkv), _ptr(qkv), _ptr(out), _ptr(dout),
                                    _ptr(lse2), _ptr(scratch), _ptr(dqkv), B, T, H, hd,
                                    _stream(stream)))


def gptk_softcap_ce(z, targets, n_valid, loss_rows, cap: float = 15.0, grad_scale: float = 1.0,
                    stream=None):
    rows, V = z.shape
    _check(lib().gptk_softcap_ce(_dtype_code(z), _ptr(z), z.stride(0), _ptr(targets), rows, V,
                                 cap, grad_scale, _ptr(n_valid), _ptr(loss_rows),
                                 _stream(stream)))


# ---------------------------------------------------------------- dense optimizer step
def gpt_opt_state_elems(cfg: GPTConfig) -> int:
    c = make_config(cfg)
    n = int(lib().gpt_opt_state_elems(C.byref(c)))
    if n < 0:
        raise GptError(GPT_EINVAL, lib().gpt_last_error().decode())
    return n


def gpt_opt_workspace_bytes(cfg: GPTConfig) -> int:
    c = make_config(cfg)
    b = C.c_size_t(0)
    _check(lib().gpt_opt_workspace_bytes(C.byref(c), C.byref(b)))
    return b.value


def gpt_opt_step(cfg: GPTConfig, master, params, grads, state, hp: dict, workspace,
                 grad_norm=None, stream=None):
    """One dense optimizer step (see gpt.h).  hp: the gpt_opt_hparams fields by name."""
    c = make_config(cfg)
    h = gpt_opt_hparams(**hp)
    _check(lib().gpt_opt_step(C.byref(c), _ptr(master), _ptr(params), _ptr(grads), _ptr(state),
                              C.byref(h), _ptr(workspace), workspace.numel(), _ptr(grad_norm),
                              _stream(stream)))


def gpt_lr_multiplier(it: int, num_iterations: int, warmup_ratio: float, warmdown_ratio: float,
                      final_lr_frac: float) -> float:
    return float(lib().gpt_lr_multiplier(it, num_iterations, warmup_ratio, warmdown_ratio,
                                         final_lr_frac))


def gpt_muon_momentum(it: int) -> float:
    return float(lib().gpt_muon_momentum(it))


# ---------------------------------------------------------------- inference with a key/value cache
def gpt_infer_workspace_bytes(cfg: GPTConfig, max_batch: int, max_seq: int) -> int:
    c = make_config(cfg)
    b = C.c_size_t(0)
    _check(lib().gpt_infer_workspace_bytes(C.byref(c), int(max_batch), int(max_seq), C.byref(b)))
    return b.value


class InferContext:
    """A gpt_infer context (key/value cache, rotary tables, activations) plus its workspace."""

    def __init__(self, cfg: GPTConfig, max_batch: int, max_seq: int, stream=None):
        import torch
        self.cfg = cfg
        self._c = make_config(cfg)
        nbytes = gpt_infer_workspace_bytes(cfg, max_batch, max_seq)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        h = C.c_void_p()
        _check(lib().gpt_infer_init(C.byref(self._c), int(max_batch), int(max_seq),
                                    self.workspace.data_ptr(), nbytes, _stream(stream),
                                    C.byref(h)))
        self.handle = h

    def close(self):
        if self.handle:
            _check(lib().gpt_infer_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gpt_infer_init(cfg: GPTConfig, max_batch: int, max_seq: int, stream=None) -> InferContext:
    return InferContext(cfg, max_batch, max_seq, stream)


def gpt_infer_reset(ctx: InferContext):
    _check(lib().gpt_infer_reset(ctx.handle))


def gpt_infer_position(ctx: InferContext) -> int:
    return int(lib().gpt_infer_position(ctx.handle))


def gpt_infer_forward(ctx: InferContext, params, tokens, logits, stream=None):
    """tokens: int32 [B, T] on the device; logits: fp32 [B, V], written."""
    B, T = tokens.shape
    _check(lib().gpt_infer_forward(ctx.handle, _ptr(params), _ptr(tokens), B, T, _ptr(logits),
                                   _stream(stream)))


def gpt_infer_profile(ctx: InferContext, enable: bool):
    _check(lib().gpt_infer_profile(ctx.handle, int(bool(enable))))


def gpt_infer_profile_read(ctx: InferContext):
    """[(name, calls, ms, flops, bytes)] aggregated per stage since profiling was enabled."""
    n = C.c_int32(256)
    arr = (gpt_profile_entry * 256)()
    _check(lib().gpt_infer_profile_read(ctx.handle, arr, C.byref(n)))
    return [(arr[i].name.decode(), arr[i].calls, arr[i].ms, arr[i].flops, arr[i].bytes)
            for i in range(min(n.value, 256))]


def gpt_infer_check_errors(ctx: InferContext, stream=None) -> int:
    f = C.c_int32(0)
    _check(lib().gpt_infer_check_errors(ctx.handle, _stream(stream), C.byref(f)))
    return f.value


def gpt_infer_destroy(ctx: InferContext):
    ctx.close()


def gpt_sample(logits, temperature: float, top_k: int, uniforms, tokens, stream=None):
    """logits fp32 [B, V]; uniforms fp32 [B] in [0, 1) (unused at temperature 0); tokens int32 [B]."""
    B, V = logits.shape
    _check(lib().gpt_sample(_ptr(logits), B, V, float(temperature), int(top_k), _ptr(uniforms),
                            _ptr(tokens), _stream(stream)))
