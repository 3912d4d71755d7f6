"""Model configurations, the flat parameter layout and the FLOP/parameter formulas.

Host-side logic only (no GPU, no method arithmetic beyond counting).

Shapes follow the GPT definition on the nanochat discussion page ("$1000 tier nanochat run",
the GPT / Block / CausalSelfAttention / MLP classes): untied embedding and LM head, bias-free
linears stored [out, in], MLP width 4*d_model, n_kv_head == n_head.  The MFU convention is the
estimate_flops method on the same page: 6*(params - embedding params) + 12*L*H*Hd*T per token.
The table shapes (2M-row and 1M-row bigram tables, a frozen 2M-row trigram table) come from the
decoder-rtx posts (page "Chris McCormick", the baseline-4 thread).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Tuple

F32 = 0
BF16 = 1

# Alignment of every tensor offset in the flat parameter buffer, in elements.
PARAM_ALIGN = 64


@dataclasses.dataclass(frozen=True)
class GPTConfig:
    n_layer: int
    d_model: int
    n_head: int
    head_dim: int
    d_mlp: int
    vocab: int
    seq_len: int
    batch: int
    dtype: int = BF16
    rms_eps: float = 1e-6
    rope_base: float = 10000.0
    softcap: float = 15.0
    qk_norm: int = 1
    has_x0_add: int = 0
    has_v_add: int = 0
    has_trigram: int = 0
    ce_chunk_tokens: int = 0     # LM-head / cross-entropy chunk (0: library default)
    wgrad_stream: int = 0        # weight gradients on their own stream: 1 yes, -1 no, 0 library
    name: str = ""

    @property
    def n_kv_head(self) -> int:
        return self.n_head

    @property
    def tokens(self) -> int:
        return self.batch * self.seq_len

    def replace(self, **kw) -> "GPTConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class TableConfig:
    """Hashed n-gram tables (decoder-rtx posts; sizes as the tables workload states them)."""
    x0_rows: int = 1 << 21
    v_rows: int = 1 << 20
    tri_rows: int = 1 << 21
    dim: int = 768
    vocab: int = 50304
    n_tokens: int = 196_608
    seq_len: int = 1024
    beta2: float = 0.95
    eps: float = 1e-8
    lr: float = 1e-2


# Tiny fp32 decoder: 2 layers, d128, 4 heads x 32, seq 64, batch 4, vocab 512.
TINY = GPTConfig(n_layer=2, d_model=128, n_head=4, head_dim=32, d_mlp=512, vocab=512,
                 seq_len=64, batch=4, dtype=F32, name="tiny-fp32")
# GPT-2-small shape: 12 layers, d768, 12 heads x 64, MLP 3072, seq 1024, batch 8, vocab 50304.
GPT2_SMALL = GPTConfig(n_layer=12, d_model=768, n_head=12, head_dim=64, d_mlp=3072, vocab=50304,
                       seq_len=1024, batch=8, dtype=BF16, name="gpt2-small-bf16")
# nanochat d32 shape: 32 layers, d2048, 16 heads x 128, MLP 8192, vocab 65536, seq 2048, batch 8.
D32 = GPTConfig(n_layer=32, d_model=2048, n_head=16, head_dim=128, d_mlp=8192, vocab=65536,
                seq_len=2048, batch=8, dtype=BF16, name="nanochat-d32-bf16")
# Speedrun-record shape: GPT-2-small model + x0 bigram, value bigram and frozen trigram tables.
SPEEDRUN = GPT2_SMALL.replace(has_x0_add=1, has_v_add=1, has_trigram=1, name="speedrun-bf16")
SPEEDRUN_MICRO_BATCHES = 24
TABLES = TableConfig()

PRESETS = {c.name: c for c in (TINY, GPT2_SMALL, D32, SPEEDRUN)}


def _align(n: int, a: int = PARAM_ALIGN) -> int:
    return (n + a - 1) // a * a


def param_layout(cfg: GPTConfig) -> List[Tuple[str, int, Tuple[int, ...]]]:
    """(name, offset_elems, shape) of every tensor in the flat parameter/gradient buffer.

    Order: wte [V,D]; per layer l: h{l}.wqkv [3D,D] (q, k, v rows stacked), h{l}.wo [D,D],
    h{l}.wfc [F,D], h{l}.wpr [D,F]; lm_head [V,D]; wtri [D,D] when the trigram addend is on.
    Offsets are multiples of PARAM_ALIGN elements.
    """
    D, F, V = cfg.d_model, cfg.d_mlp, cfg.vocab
    out = []
    off = 0

    def add(name, shape):
        nonlocal off
        out.append((name, off, shape))
        off = _align(off + math.prod(shape))

    add("wte", (V, D))
    for l in range(cfg.n_layer):
        add(f"h{l}.wqkv", (3 * D, D))
        add(f"h{l}.wo", (D, D))
        add(f"h{l}.wfc", (F, D))
        add(f"h{l}.wpr", (D, F))
    add("lm_head", (V, D))
    if cfg.has_trigram:
        add("wtri", (D, D))
    return out


def param_elems(cfg: GPTConfig) -> int:
    """Total elements of the flat buffer (including alignment padding)."""
    name, off, shape = param_layout(cfg)[-1]
    return _align(off + math.prod(shape))


def n_params(cfg: GPTConfig) -> int:
    """Parameter count of the model (tables and their projection excluded unless trigram on)."""
    return sum(math.prod(s) for _, _, s in param_layout(cfg))


def flops_per_token(cfg: GPTConfig) -> int:
    """6*(N - N_wte) + 12*L*H*Hd*T: the estimate_flops convention of the nanochat GPT class."""
    n_wte = cfg.vocab * cfg.d_model
    return 6 * (n_params(cfg) - n_wte) + 12 * cfg.n_layer * cfg.n_head * cfg.head_dim * cfg.seq_len


def hardware_flops_per_step(cfg: GPTConfig) -> float:
    """FLOPs the kernels actually execute per step with causal attention (half of T^2 counted)
    and the attention backward recomputing S and P: GEMMs 6*N*(params-wte), attention forward
    2 GEMMs, backward 5 GEMMs (recompute S, dP, dV, dQ, dK), each causal."""
    n_tok = cfg.tokens
    n_wte = cfg.vocab * cfg.d_model
    dense = 6.0 * (n_params(cfg) - n_wte) * n_tok
    causal_pairs = cfg.batch * cfg.seq_len * (cfg.seq_len + 1) / 2
    att = 2.0 * causal_pairs * cfg.head_dim * cfg.n_head * cfg.n_layer * (2 + 5)
    return dense + att
