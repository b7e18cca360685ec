"""Pins of the training-time-test attention oracle ("EAGLE-3: Engineering
Implementation of LLM Inference Acceleration", VII.5 and VIII forward_ttt)."""
import json
import os

import numpy as np

from oracle.ttt import ttt_attention, ttt_visible

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_visibility_matches_figure6():
    """The page's worked example: which tokens each simulated token attends to."""
    g = json.load(open(os.path.join(GOLDEN, "ttt_mask_figure6.json")))
    steps = g["steps"]
    T = len(steps[0])
    for s in range(1, len(steps)):
        for i in range(T):
            seen = [steps[st][j] for st, j in ttt_visible(T, len(steps) - 1, i, s)]
            assert seen == g["attends"][steps[s][i]]


def _dense_masked(q, k0, v0, ks, vs):
    """All steps' keys concatenated with the explicit mask (a plain masked softmax):
    key (s, j) is visible to query i iff s == 0 and j <= i, or s >= 1 and j == i."""
    T, Hq, hd = q.shape
    Hkv, S = k0.shape[0], ks.shape[0]
    G = Hq // Hkv
    K = np.concatenate([k0[None], ks], 0)  # [S+1, Hkv, T, hd]
    Vv = np.concatenate([v0[None], vs], 0)
    mask = np.zeros((T, (S + 1) * T), dtype=bool)
    for i in range(T):
        mask[i, :i + 1] = True
        for s in range(1, S + 1):
            mask[i, s * T + i] = True
    out = np.zeros((T, Hq, hd))
    for h in range(Hq):
        g = h // G
        keys = K[:, g].reshape((S + 1) * T, hd)
        vals = Vv[:, g].reshape((S + 1) * T, hd)
        sc = (q[:, h] @ keys.T) / np.sqrt(hd)
        sc = np.where(mask, sc, -np.inf)
        w = np.exp(sc - sc.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        out[:, h] = w @ vals
    return out


def test_ttt_equals_dense_masked_attention():
    """The diagonal form equals attention over every step's keys under the explicit
    mask (the page's own check reports float32 rounding; here float64)."""
    rng = np.random.default_rng(3)
    for T, S, Hq, Hkv, hd in [(1, 0, 2, 1, 8), (7, 3, 4, 2, 16), (19, 1, 6, 3, 8), (12, 0, 2, 2, 4)]:
        q = rng.normal(size=(T, Hq, hd))
        k0, v0 = rng.normal(size=(Hkv, T, hd)), rng.normal(size=(Hkv, T, hd))
        ks, vs = rng.normal(size=(S, Hkv, T, hd)), rng.normal(size=(S, Hkv, T, hd))
        np.testing.assert_allclose(ttt_attention(q, k0, v0, ks, vs), _dense_masked(q, k0, v0, ks, vs), atol=1e-12)


def test_ttt_special_cases():
    rng = np.random.default_rng(4)
    T, S, Hq, Hkv, hd = 5, 2, 2, 1, 8
    q = rng.normal(size=(T, Hq, hd))
    k0, v0 = rng.normal(size=(Hkv, T, hd)), rng.normal(size=(Hkv, T, hd))
    ks, vs = rng.normal(size=(S, Hkv, T, hd)), rng.normal(size=(S, Hkv, T, hd))
    out = ttt_attention(q, k0, v0, ks, vs)
    # position 0 sees k0_0 and its own diagonal keys only: a softmax over 1 + S scores
    for h in range(Hq):
        sc = np.array([k0[0, 0] @ q[0, h]] + [ks[s, 0, 0] @ q[0, h] for s in range(S)]) / np.sqrt(hd)
        w = np.exp(sc - sc.max())
        w /= w.sum()
        ref = w[0] * v0[0, 0] + sum(w[1 + s] * vs[s, 0, 0] for s in range(S))
        np.testing.assert_allclose(out[0, h], ref, atol=1e-12)
    # a zero query weighs every visible key equally
    qz = np.zeros_like(q)
    oz = ttt_attention(qz, k0, v0, ks, vs)
    for i in range(T):
        ref = (v0[0, :i + 1].sum(0) + vs[:, 0, i].sum(0)) / (i + 1 + S)
        np.testing.assert_allclose(oz[i, 0], ref, atol=1e-12)
    # a diagonal key far above every other score takes all the weight
    kb = ks.copy()
    kb[1, 0, 3] = 1e3 * q[3, 0] / np.linalg.norm(q[3, 0])
    ob = ttt_attention(q, k0, v0, kb, vs)
    np.testing.assert_allclose(ob[3, 0], vs[1, 0, 3], atol=1e-9)
