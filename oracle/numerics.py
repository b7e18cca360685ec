"""Numerics of the oracle: storage rounding, softmax, and the fp32 decision rules.

Arithmetic runs in float64.  Values are rounded to the model's storage dtype
(bf16 or fp32) exactly where the GPU path stores them in that dtype: weights,
GEMM-input activations (norm outputs, the draft's [e ; x] input, the attention
output, SiLU(g)*u), K/V cache entries, q, and the captured auxiliary features.

Where a float decides an integer (argmax, top-k, tree ranking, sampling), the
decision is taken on float32 values with the rules below so that a GPU kernel
can reproduce it bit for bit from equal float32 logits.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns float64.

    bfloat16 keeps 8 significant bits and float32's exponent range; the
    quantum of a value in [2**(e-1), 2**e) is 2**(e-8), and 2**-133 below
    the normal range.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    quantum_exp = np.maximum(e - 8, -133)
    q = np.ldexp(np.rint(np.ldexp(x, -quantum_exp)), quantum_exp)
    return np.where(np.isfinite(x), q, x)


def round_f32(x) -> np.ndarray:
    """Round float64 values to the nearest float32 (ties to even); returns float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rounder(dtype: str):
    if dtype == "bf16":
        return round_bf16
    if dtype == "f32":
        return round_f32
    raise ValueError(dtype)


def logsumexp_f64(z: np.ndarray) -> np.ndarray:
    """log(sum(exp(z))) over the last axis, float64, by its definition (max-shifted)."""
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=-1, keepdims=True)))[..., 0]


def softmax_f64(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ------------------------------------------------------------------ decisions

def argmax_first(x: np.ndarray) -> int:
    """Index of the largest value; the lowest index wins a tie (torch/numpy argmax)."""
    return int(np.argmax(np.asarray(x)))


def topk_desc(x32: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest float32 values, larger value first, lower index on ties."""
    x = np.asarray(x32, dtype=np.float32)
    order = np.lexsort((np.arange(x.size), -x.astype(np.float64)))
    return order[:k]


def draft_logprobs_f32(logits32: np.ndarray) -> np.ndarray:
    """Draft log-probabilities used to rank tree candidates.

    log_softmax of float32 logits at temperature 1: the log-sum-exp is taken
    in float64 and rounded to float32, then logp = fl32(logit - lse).  Every
    logp is <= 0 because lse >= max(logit) and rounding is monotone.
    """
    l32 = np.asarray(logits32, dtype=np.float32)
    lse = np.float32(logsumexp_f64(l32.astype(np.float64)))
    return (l32 - lse).astype(np.float32)


def probs_f32(logits32: np.ndarray, temperature: float) -> np.ndarray:
    """softmax(logits / T) in float64, rounded to float32 (the sampler's p and q)."""
    z = np.asarray(logits32, dtype=np.float32).astype(np.float64) / np.float64(np.float32(temperature))
    return softmax_f64(z).astype(np.float32)


W_SHIFT = 48  # integer sampling weights are floor(w * 2**48)


def int_weights(w32: np.ndarray) -> np.ndarray:
    """Non-negative float32 weights -> exact integer weights floor(w * 2**48)."""
    w = np.asarray(w32, dtype=np.float32).astype(np.float64)
    assert np.all(w >= 0)
    return np.floor(np.ldexp(w, W_SHIFT)).astype(np.uint64)


def sample_inverse_cdf(w32: np.ndarray, u32: float) -> int:
    """Draw one index from the distribution proportional to non-negative float32 weights.

    Inverse CDF on exact integers: W_v = floor(w_v * 2**48), S = sum W,
    r = floor(u * S) with u a multiple of 2**-24 in [0, 1), and the pick is the
    first v whose inclusive prefix sum exceeds r.  P(v) = W_v / S up to the
    2**-24 grid of u.  Returns -1 when every weight is zero.
    """
    W = int_weights(w32)
    prefix = np.cumsum(W, dtype=np.uint64)          # exact: S < 2**64
    S = int(prefix[-1])
    if S == 0:
        return -1
    u_int = int(np.float64(np.float32(u32)) * (1 << 24))
    assert 0 <= u_int < (1 << 24)
    r = (u_int * S) >> 24                           # floor(u * S), exact
    v = int(np.searchsorted(prefix, np.uint64(r), side="right"))
    assert W[v] > 0 and int(prefix[v]) > r
    return v
