"""Acceptance: greedy longest path over a tree, and chain rejection sampling.

Sources (page title, section):
  * "Advanced speculative decoding: tree drafts and EAGLE", Implementation
    (from the root, follow the child whose token equals the argmax of the
    node's logits; the next root is the argmax at the end of the path).
  * "EAGLE-3: Engineering Implementation of LLM Inference Acceleration",
    III.5 and X.3-X.6 (accept d_i with probability min(1, p_i(d_i)/q_i(d_i))
    front to back; the first rejection resamples from norm(max(0, p_i - q_i))
    and discards the rest; if every draft is accepted a bonus token is drawn
    from p at the last position), and "EAGLE-3: Training-Time Test for
    Speculative Decoding", Lossless Verification Makes Prefix Survival the
    Contract (the same rule, printed intact).
  * "Speculative Decoding (EAGLE3) in the vLLM Neuron Framework", Rejection
    Sampling (greedy drafts: draft probability 1, recovered token from
    max(p - q, 0) with the draft token zeroed; output [B, K+1] padded with -1).
"""
from __future__ import annotations

import numpy as np

from .numerics import argmax_first, sample_inverse_cdf


def greedy_walk(tokens, parents, argmax_rows):
    """Longest accepted path.  Returns (path node indices, next root token).

    argmax_rows[i] is the target's argmax at tree row i.  Among the children of
    the current node the lowest-index one whose token equals that argmax is
    followed (siblings are distinct tokens, so at most one matches).
    """
    path, node = [0], 0
    n = len(tokens)
    while True:
        pred = int(argmax_rows[node])
        child = next((c for c in range(n) if parents[c] == node and tokens[c] == pred), None)
        if child is None:
            break
        path.append(child)
        node = child
    return path, int(argmax_rows[node])


def argmax_rows_f32(logits) -> list:
    """Per-row argmax of float32-rounded logits (the decision precision)."""
    l32 = np.asarray(logits, dtype=np.float64).astype(np.float32)
    return [argmax_first(r) for r in l32]


def chain_rejection(draft_tokens, q32, p32, u32):
    """Sequential rejection sampling over a chain of K drafts.

    draft_tokens [K]; q32 [K, V] the draft distributions d_i was drawn from;
    p32 [K+1, V] the target distributions at the same rows plus one;
    u32 [K+1]: u[i] decides draft i, u[K] drives the single final draw.
    Accept d_i iff u[i] < fl32(p_i(d_i) / q_i(d_i)) (u < 1, so this is
    u < min(1, ratio)).  On the first rejection draw from max(0, p_i - q_i)
    (float32, exact); if that residual is all zero (impossible in exact
    arithmetic) draw from p_i.  If all K are accepted draw the bonus from p_K.
    Returns (n_accepted, next_token).
    """
    K = len(draft_tokens)
    p32 = np.asarray(p32, dtype=np.float32)
    q32 = np.asarray(q32, dtype=np.float32)
    for i in range(K):
        t = int(draft_tokens[i])
        ratio = np.float32(p32[i, t] / q32[i, t])
        if np.float32(u32[i]) < ratio:
            continue
        resid = np.maximum(p32[i] - q32[i], np.float32(0)).astype(np.float32)
        tok = sample_inverse_cdf(resid, u32[K])
        if tok < 0:
            tok = sample_inverse_cdf(p32[i], u32[K])
        return i, tok
    return K, sample_inverse_cdf(p32[K], u32[K])


def emitted_row(path_tokens, width):
    """[width] row: the committed tokens of one step, -1 padded (the [B, K+1] format)."""
    row = [-1] * width
    for i, t in enumerate(path_tokens[:width]):
        row[i] = int(t)
    return row
