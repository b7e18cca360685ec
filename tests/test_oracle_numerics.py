"""Pins of the oracle's numerics against library routines, closed forms and exhaustion."""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

from oracle.numerics import (draft_logprobs_f32, int_weights, logsumexp_f64, probs_f32, round_bf16,
                             round_f32, sample_inverse_cdf, topk_desc)


def test_round_bf16_matches_torch_conversion():
    """Round-to-nearest-even to bfloat16 == torch's float32 -> bfloat16 conversion."""
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 1, 20000), rng.normal(0, 1e-3, 2000), rng.normal(0, 300, 2000),
                        1 + np.arange(-64, 64) * 2.0 ** -9])        # includes exact ties
    x32 = x.astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_bf16(x32.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    assert round_bf16(1 + 2.0 ** -8) == 1.0                         # tie -> even mantissa 0
    assert round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6            # tie -> even mantissa 2
    assert round_bf16(-(1 + 3 * 2.0 ** -8)) == -(1 + 2.0 ** -6)


def test_round_f32_matches_numpy_cast():
    x = np.random.default_rng(1).normal(0, 1, 1000)
    assert np.array_equal(round_f32(x), x.astype(np.float32).astype(np.float64))


def test_logsumexp_matches_scipy():
    z = np.random.default_rng(2).normal(0, 5, (7, 333))
    np.testing.assert_allclose(logsumexp_f64(z), logsumexp(z, axis=-1), rtol=1e-14)


def test_draft_logprobs_nonpositive_and_normalised():
    z = (np.random.default_rng(3).normal(0, 3, (5, 1000))).astype(np.float32)
    for row in z:
        lp = draft_logprobs_f32(row)
        assert lp.dtype == np.float32 and np.all(lp <= 0)
        assert abs(np.sum(np.exp(lp.astype(np.float64))) - 1) < 1e-4
    # uniform row: every log-prob is -log(V) rounded
    lp = draft_logprobs_f32(np.zeros(64, np.float32))
    np.testing.assert_allclose(lp, -np.log(64), rtol=1e-6)


def test_probs_temperature():
    z = np.random.default_rng(4).normal(0, 2, 100).astype(np.float32)
    p1 = probs_f32(z, 1.0)
    assert abs(p1.astype(np.float64).sum() - 1) < 1e-5
    p2 = probs_f32(z, 2.0)
    np.testing.assert_allclose(p2, torch.softmax(torch.from_numpy(z).double() / 2, 0).numpy(), rtol=1e-6)


def test_topk_order_and_ties():
    x = np.array([1.0, 3.0, 3.0, -1.0, 2.0], np.float32)
    assert list(topk_desc(x, 4)) == [1, 2, 4, 0]


def test_int_weights_exact():
    w = np.array([0.5, 0.25, 2.0 ** -48, 2.0 ** -49, 0.0], np.float32)
    assert list(int_weights(w)) == [2 ** 47, 2 ** 46, 1, 0, 0]


@pytest.mark.parametrize("weights", [[3, 0, 5, 1], [1, 1, 1, 1, 1, 1, 1], [7], [0, 0, 2, 0, 9, 4]])
def test_inverse_cdf_exhaustive_over_u_grid(weights):
    """Over all 2**24 uniforms the pick count of index v is 2**24 * W_v / S within 1."""
    w = np.array(weights, dtype=np.float64) * 2.0 ** -48           # integer weights exactly
    W = np.array(weights, dtype=np.int64)
    S = int(W.sum())
    u_int = np.arange(1 << 24, dtype=np.int64)
    r = (u_int * S) >> 24                                          # S small: no overflow
    pick = np.searchsorted(np.cumsum(W), r, side="right")
    counts = np.bincount(pick, minlength=len(W))
    np.testing.assert_allclose(counts, (1 << 24) * W / S, atol=1.0)
    # the oracle routine agrees on a sample of the grid
    idx = np.random.default_rng(5).integers(0, 1 << 24, 300)
    for ui in idx:
        assert sample_inverse_cdf(w.astype(np.float32), np.float32(ui * 2.0 ** -24)) == pick[ui]


def test_inverse_cdf_edges():
    w = np.array([0, 0, 0.5, 0, 0.5], np.float32)
    assert sample_inverse_cdf(w, np.float32(0.0)) == 2
    assert sample_inverse_cdf(w, np.float32(1 - 2.0 ** -24)) == 4
    assert sample_inverse_cdf(np.zeros(4, np.float32), np.float32(0.3)) == -1
