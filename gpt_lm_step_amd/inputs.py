"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module only draws random numbers and lays them out; it holds none of the method's
arithmetic.  Every generator is numpy PCG64 (``default_rng``) from an explicit seed, so the
same buffers feed both the HIP path and the CPU oracle.

* Tokens: uniform ints, or Zipf(s) over the vocabulary with P(k) proportional to (k+1)^-s,
  k in [0, V), drawn by inverse CDF.  These stand in for the FineWeb / nanochat token shards
  the pages train on (not available offline).
* Weights: N(0, std) in float32, rounded to bfloat16 (round-to-nearest-even) for bf16 configs.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np

from .configs import BF16, GPTConfig, param_layout, param_elems


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def uniform_tokens(seed: int, shape, vocab: int) -> np.ndarray:
    return rng(seed).integers(0, vocab, size=shape, dtype=np.int64).astype(np.int32)


def zipf_tokens(seed: int, shape, vocab: int, s: float = 1.1) -> np.ndarray:
    w = np.arange(1, vocab + 1, dtype=np.float64) ** (-s)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    u = rng(seed).random(size=int(np.prod(shape)))
    idx = np.searchsorted(cdf, u, side="right")
    return np.minimum(idx, vocab - 1).astype(np.int32).reshape(shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bfloat16."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def normal(seed: int, shape, std: float, bf16: bool) -> np.ndarray:
    x = rng(seed).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return round_bf16(x) if bf16 else x


def model_params(cfg: GPTConfig, seed: int, std: float = 0.02,
                 zero_head: bool = False) -> Dict[str, np.ndarray]:
    """Every weight N(0, std) (float32 storage; bf16-representable for bf16 configs)."""
    bf16 = cfg.dtype == BF16
    out = {}
    for i, (name, _, shape) in enumerate(param_layout(cfg)):
        if zero_head and name == "lm_head":
            out[name] = np.zeros(shape, np.float32)
        else:
            out[name] = normal(seed * 1000 + i, shape, std, bf16)
    return out


def flatten_params(cfg: GPTConfig, params: Dict[str, np.ndarray]) -> np.ndarray:
    """Pack named tensors into the flat float32 buffer of the parameter layout."""
    flat = np.zeros(param_elems(cfg), np.float32)
    for name, off, shape in param_layout(cfg):
        flat[off:off + int(np.prod(shape))] = params[name].reshape(-1)
    return flat


def unflatten(cfg: GPTConfig, flat: np.ndarray) -> Dict[str, np.ndarray]:
    return {name: flat[off:off + int(np.prod(shape))].reshape(shape)
            for name, off, shape in param_layout(cfg)}


def step_tokens(cfg: GPTConfig, seed: int, zipf: bool = True) -> np.ndarray:
    """[B, T+1] token ids; inputs are [:, :T], next-token targets are [:, 1:]."""
    shape = (cfg.batch, cfg.seq_len + 1)
    if zipf:
        return zipf_tokens(seed, shape, cfg.vocab)
    return uniform_tokens(seed, shape, cfg.vocab)


def addend(seed: int, n: int, dim: int, std: float, bf16: bool) -> np.ndarray:
    return normal(seed, (n, dim), std, bf16)


def seeds_for(name: str) -> Dict[str, int]:
    """Seeds per workload (tokens, weights, tables, upstream grads)."""
    table = {
        "tiny-fp32": dict(tokens=1, weights=101),
        "gpt2-small-bf16": dict(tokens=2, weights=102),
        "nanochat-d32-bf16": dict(tokens=3, weights=103),
        "tables": dict(tokens=4, weights=104, dy=204),
        "speedrun-bf16": dict(tokens=5, weights=102, tables=104, trigram=105),
    }
    return table[name]


def device_params(cfg: GPTConfig, seed: int, std: float = 0.02, zero_head: bool = False):
    """Flat parameter buffer drawn on the GPU (torch Philox, seeded): every weight N(0, std),
    stored in the config's dtype.  Used where host generation of ~2e9 values would dominate."""
    import torch
    dt = torch.bfloat16 if cfg.dtype == BF16 else torch.float32
    flat = torch.zeros(param_elems(cfg), dtype=dt, device="cuda")
    g = torch.Generator(device="cuda")
    for i, (name, off, shape) in enumerate(param_layout(cfg)):
        n = int(np.prod(shape))
        if zero_head and name == "lm_head":
            continue
        g.manual_seed(seed * 1000 + i)
        flat[off:off + n] = (torch.randn(n, device="cuda", generator=g) * std).to(dt)
    return flat
