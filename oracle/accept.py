"""Acceptance: greedy longest path over a tree, chain rejection sampling, and
level-by-level rejection sampling over a tree.

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
  * "Advanced speculative decoding: tree drafts and EAGLE", Exercises (trees
    under sampling: a node's candidates are tested in turn, each rejection
    turns p into norm(max(0, p - q)), all rejected draws from the final
    residual).
"""
from __future__ import annotations

import numpy as np

from .numerics import argmax_first, int_weights, sample_inverse_cdf


def greedy_walk(tokens, parents, argmax_rows):
    """Longest accepted path.  Returns (path node indices, next root token).

    argmax_rows[i] is the target's argmax at tree row i.  A tree edge is named
    by (parent row, token); from the root the walk keeps taking the edge whose
    token is the current row's argmax, and stops at the first row where no such
    edge exists.  Siblings carry distinct tokens, so an edge names at most one
    row (the lowest one is kept if a malformed tree repeats a token).  The next
    root is the argmax of the last row reached.
    """
    edge = {}
    for row in range(len(tokens) - 1, 0, -1):          # descending: the lowest row wins
        edge[(int(parents[row]), int(tokens[row]))] = row
    path = [0]
    while (path[-1], int(argmax_rows[path[-1]])) in edge:
        path.append(edge[(path[-1], int(argmax_rows[path[-1]]))])
    return path, int(argmax_rows[path[-1]])


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


def tree_rejection(tokens, parents, p32, u32, topk, max_depth):
    """Level-by-level rejection sampling over a draft tree ("Advanced speculative
    decoding: tree drafts and EAGLE", Exercises, trees under sampling).

    tokens, parents [n] (root row 0, parents[i] < i); p32 [n, V] the target
    distribution at every tree row (float32); u32 [max_depth * topk + 1].
    At the current node (depth d) its children are considered in row order:
    child i (token x) is accepted with probability min(1, p'(x) / q(x)), where
    p' is the node's residual target distribution.  The tree's children are
    chosen deterministically (draft top-k), so each candidate's q is the point
    mass at its token, the test is u < p'(x), and a rejection updates
    p' <- norm(max(0, p' - q)), i.e. removes x's mass.  An accepted child
    becomes the current node; when every child is rejected (or the node has
    none) one token is drawn from the final residual and the walk stops.

    Fixed point, as in the draws: W_v = floor(p(v) * 2**48); the residual mass
    before child i is S_i = sum of W over the tokens not yet removed, and child i
    is accepted iff floor(u * S_i) < W_x with u = u32[d * topk + i].  The final
    draw uses u32[max_depth * topk].  Returns (path row indices, next token).
    """
    n = len(tokens)
    path, node = [0], 0
    while True:
        d = len(path) - 1
        W = int_weights(p32[node])
        kids = [c for c in range(n) if parents[c] == node] if d < max_depth else []
        removed = set()
        S = int(sum(int(w) for w in W))
        accepted = None
        for i, c in enumerate(kids[:topk]):
            x = int(tokens[c])
            w_x = 0 if x in removed else int(W[x])
            s_i = S - sum(int(W[t]) for t in removed)
            u_int = int(np.float64(np.float32(u32[d * topk + i])) * (1 << 24))
            if (u_int * s_i) >> 24 < w_x:
                accepted = c
                break
            removed.add(x)
        if accepted is None:
            resid = np.asarray(p32[node], dtype=np.float32).copy()
            for t in removed:
                resid[t] = 0
            return path, sample_inverse_cdf(resid, u32[max_depth * topk])
        path.append(accepted)
        node = accepted


def emitted_row(path_tokens, width):
    """[width] row: the committed tokens of one step, -1 padded (the [B, K+1] format)."""
    row = [-1] * width
    for i, t in enumerate(path_tokens[:width]):
        row[i] = int(t)
    return row
