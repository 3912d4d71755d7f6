"""Helpers shared by the GPU parity tests: device transfer and error measures."""
import numpy as np
import torch

from gpt_lm_step_amd import inputs

DEV = "cuda"


def dev(a: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    """float32/int numpy -> device tensor (bf16 values are exact: inputs are bf16-rounded)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(DEV).to(dtype) if t.is_floating_point() else t.to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy() if t.is_floating_point() else t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return inputs.bf16_bits_to_f32(bits).astype(np.float64)


def rel_l2(got, want) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    den = np.linalg.norm(want)
    return float(np.linalg.norm(got - want) / (den if den > 0 else 1.0))


def cosine(got, want) -> float:
    got = np.asarray(got, np.float64).ravel()
    want = np.asarray(want, np.float64).ravel()
    d = np.linalg.norm(got) * np.linalg.norm(want)
    return float(got @ want / d) if d > 0 else 1.0


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance in bf16 ulps between two arrays of bf16 bit patterns (monotone integer map)."""
    def key(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + (x & 0x7FFF))
    return np.abs(key(a_bits) - key(b_bits))


def oracle_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """Round oracle fp64 values to bf16 (via fp32) bit patterns."""
    return inputs.f32_to_bf16_bits(np.asarray(x64, np.float64).astype(np.float32))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (normal range)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def table_update_bound(w0, want, dy, h_local, step):
    """Largest |gpu - oracle| a correct fp32 implementation of the per-row update can show.

    The kernel sums n_r bf16 gradient rows in fp32, forms step = lr / (sqrt(v) + eps) and
    w - step * g in fp32, then rounds once to bf16; the oracle does the same in fp64.  Bound:
    one bf16 ulp of the result (rounding on either side of a tie), fp32 error on |w| and
    |step * g|, and the fp32 summation error of g, n_r * 2^-24 * sum_t |dy_t| per element.
    """
    rows = want.shape[0]
    s_abs = np.zeros_like(want)
    np.add.at(s_abs, h_local, np.abs(dy))
    n_r = np.bincount(h_local, minlength=rows).astype(np.float64)[:, None]
    delta = np.abs(np.asarray(w0, np.float64) - want)
    return (bf16_ulp(want) + 2.0 ** -21 * (np.abs(w0) + delta)
            + np.asarray(step)[:, None] * n_r * 2.0 ** -23 * s_abs)
