"""Pins of the inference oracle (oracle/infer.py): causality against the pinned model forward and
closed-form cases of the sampling rule."""
import numpy as np
import pytest

from gpt_lm_step_amd import configs, inputs
from oracle import infer as oi
from oracle import model as om


def test_next_logits_equal_the_full_forward_at_every_prefix():
    """The logits after a prefix of length t are the full sequence's logits at position t - 1
    (causal attention: later ids never reach earlier positions)."""
    cfg = configs.TINY
    params = inputs.model_params(cfg, 101)
    tok = inputs.uniform_tokens(1, (2, 17), cfg.vocab)
    full = om.forward_backward(cfg.replace(batch=2, seq_len=16), params, tok, want_grads=False,
                               want_logits=True).logits
    for t in (1, 5, 16):
        np.testing.assert_allclose(oi.next_logits(cfg, params, tok[:, :t]), full[:, t - 1],
                                   rtol=1e-12, atol=1e-12)


def test_sampling_special_cases():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((4, 50))
    am = np.argmax(z, axis=1)
    for u in (0.0, 0.3, 0.999):
        np.testing.assert_array_equal(oi.sample(z, 0.0, 0, np.full(4, u)), am)   # temperature 0
        np.testing.assert_array_equal(oi.sample(z, 1.0, 1, np.full(4, u)), am)   # top_k 1
    # equal logits: the uniform distribution, so the id is floor(u V)
    flat = np.zeros((1, 40))
    for u in (0.0, 0.26, 0.51, 0.99):   # away from the cell edges k/40
        assert oi.sample(flat, 0.7, 0, np.array([u]))[0] == int(u * 40)
    # two ids with probabilities 3/4 and 1/4
    two = np.array([[np.log(3.0), 0.0]])
    assert oi.sample(two, 1.0, 0, np.array([0.74]))[0] == 0
    assert oi.sample(two, 1.0, 0, np.array([0.76]))[0] == 1
    # temperature 2 flattens them to sqrt(3) : 1, i.e. p0 = 0.634
    assert oi.sample(two, 2.0, 0, np.array([0.62]))[0] == 0
    assert oi.sample(two, 2.0, 0, np.array([0.65]))[0] == 1
    # top_k keeps ties: [1, 1, 1, 0] with k = 2 keeps the three ones, each 1/3
    ties = np.array([[1.0, 1.0, 1.0, 0.0]])
    assert [oi.sample(ties, 1.0, 2, np.array([u]))[0] for u in (0.1, 0.4, 0.9)] == [0, 1, 2]
    assert oi.sample(np.array([[0.0, 5.0, 5.0]]), 0.0, 0, np.zeros(1))[0] == 1  # first max


def test_sampling_frequencies_match_the_tempered_top_k_softmax():
    """Over an even grid of uniforms the share of each id is its probability: exp(z/T) over the
    top_k largest logits, normalised, zero elsewhere."""
    rng = np.random.default_rng(9)
    z = rng.standard_normal(12)
    T, k = 0.8, 5
    keep = np.argsort(-z)[:k]
    p = np.zeros(12)
    p[keep] = np.exp(z[keep] / T)
    p /= p.sum()
    n = 200000
    u = (np.arange(n) + 0.5) / n
    ids = oi.sample(np.broadcast_to(z, (n, 12)), T, k, u)
    share = np.bincount(ids, minlength=12) / n
    np.testing.assert_allclose(share, p, atol=2.0 / n)
