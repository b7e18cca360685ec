"""Training-time-test attention forward.  TEST INFRASTRUCTURE ONLY (see oracle/__init__).

Source: "EAGLE-3: Engineering Implementation of LLM Inference Acceleration",
VII.5 (attention mask during training-time test) and VIII (the draft layer's
forward_ttt): the native step's keys are attended causally; each simulated
step s >= 1 adds one key per position that only the query at the same
position sees (the diagonal), and all scores of a query share one softmax.
"""
from __future__ import annotations

import numpy as np


def ttt_attention(q, k0, v0, ks, vs, positions=None):
    """q [T, Hq, hd]; k0, v0 [Hkv, T, hd] (native step); ks, vs [S, Hkv, T, hd]
    (simulated steps; S may be 0).  Query head h reads KV head h // (Hq / Hkv).

    Scores of query i: scale * q_i . k0_j for j <= i (causal), then one
    diagonal score scale * q_i . ks[s]_i per simulated step; softmax over the
    i + 1 + S scores; output = the weighted sum of the matching values.
    float64 throughout.  Returns [T, Hq, hd] (only the rows in `positions`
    filled when it is given; the others are zero).
    """
    q = np.asarray(q, dtype=np.float64)
    k0 = np.asarray(k0, dtype=np.float64)
    v0 = np.asarray(v0, dtype=np.float64)
    ks = np.asarray(ks, dtype=np.float64)
    vs = np.asarray(vs, dtype=np.float64)
    T, Hq, hd = q.shape
    Hkv = k0.shape[0]
    S = ks.shape[0]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(hd)
    out = np.zeros((T, Hq, hd))
    rows = range(T) if positions is None else positions
    for h in range(Hq):
        g = h // G
        for i in rows:
            native = scale * (k0[g, :i + 1] @ q[i, h])                            # [i + 1]
            diag = np.array([scale * (ks[s, g, i] @ q[i, h]) for s in range(S)])  # [S]
            sc = np.concatenate([native, diag])
            w = np.exp(sc - sc.max())
            w /= w.sum()
            out[i, h] = w[:i + 1] @ v0[g, :i + 1]
            for s in range(S):
                out[i, h] += w[i + 1 + s] * vs[s, g, i]
    return out


def ttt_visible(T: int, S: int, i: int, step: int):
    """Keys a query at position i of step `step` (0 = native) sees, as (step, position)
    pairs: the native prefix 0..i and its own position's keys of steps 1..step."""
    return [(0, j) for j in range(i + 1)] + [(s, i) for s in range(1, step + 1)]
