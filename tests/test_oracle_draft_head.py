"""Pins of the oracle's EAGLE-3 draft head against the structure the pages fix.

"EAGLE-3: Engineering Implementation of LLM Inference Acceleration":
  * VIII.1 / VIII.3 - the draft decoder layer normalises the token embedding e
    (input_norm) and the feature x (hidden_norm) separately, concatenates them
    embedding first into one 2d-wide attention input, and carries only x as
    its residual stream; post_norm + SwiGLU MLP follow.
  * VIII.5 - the draft has its own final norm in front of the LM head.
  * IX.5 - the fused feature is a bias-free FC over [l ; m ; h], the three taps
    in ascending layer order.
"EAGLE-3: Engineering Implementation ...", XI.6 and X.2: drafts are drawn from
q = softmax(draft logits / T).

Each pin is chosen so that a plausible slip in the oracle fails it; the tests
named *_catches_* plant that slip (on the CPU, in the oracle) and check that
the pin rejects it.
"""
import numpy as np
import pytest
from scipy.special import expit, softmax
from scipy.stats import chi2

import oracle.llama as llama
from oracle.llama import Shape, draft_fuse, draft_layer, draft_logits, target_forward, causal_visible, KVCache
from oracle.step import build_sampled_chain

D, HQ, HKV, HD, F, V = 16, 2, 1, 8, 24, 12


def _shape(eps=0.0, dtype="f32", layers=1, taps=(0, 0, 0)):
    return Shape(layers, D, HQ, HKV, HD, F, V, 1e4, eps, dtype, taps)


def _head(seed=0, sigma=0.3):
    rng = np.random.default_rng(seed)
    g = lambda *s: rng.normal(0, sigma, s)
    H = {"fc": g(D, 3 * D), "input_norm": np.ones(D), "hidden_norm": np.ones(D),
         "wq": g(HQ * HD, 2 * D), "wk": g(HKV * HD, 2 * D), "wv": g(HKV * HD, 2 * D), "wo": g(D, HQ * HD),
         "post_norm": np.ones(D), "w_gate": g(F, D), "w_up": g(F, D), "w_down": g(D, F), "final_norm": np.ones(D)}
    W = {"embed": g(V, D), "lm_head": g(V, D), "final_norm": np.ones(D)}
    return H, W


def _causal(i, k, v):
    return k[:i + 1], v[:i + 1]


def _run(H, W, shp, toks, x, fn=None):
    fn = fn or draft_layer
    a, _, _ = fn(H, W, shp, toks, x, np.arange(len(toks)), _causal)
    return a


TOKS = [3, 7, 1]
TOKS2 = [5, 0, 9]


def _x(seed=1, scale=1.0):
    return np.random.default_rng(seed).normal(0, scale, (len(TOKS), D))


# --------------------------------------------------------------- residual stream

def test_residual_stream_is_x_only():
    """With wo = w_down = 0 the layer adds nothing: a == x bit for bit (the
    embedding never joins the residual sum)."""
    H, W = _head()
    H["wo"][:] = 0
    H["w_down"][:] = 0
    x = _x()
    assert np.array_equal(_run(H, W, _shape(), TOKS, x), x)


def test_residual_pin_catches_embedding_in_the_residual():
    H, W = _head()
    H["wo"][:] = 0
    H["w_down"][:] = 0
    x = _x()

    def planted(H, W, shp, toks, x, pos, ctx):          # residual stream e + x
        a, k, v = draft_layer(H, W, shp, toks, x, pos, ctx)
        return a + W["embed"][np.asarray(toks)], k, v

    assert np.abs(_run(H, W, _shape(), TOKS, x, planted) - x).max() > 1e-3


# ------------------------------------------------------------------ concat order

def _no_mlp(H):
    H["w_gate"][:] = 0        # silu(0) * u = 0: a - x is the attention term alone
    return H


def test_concat_order_embedding_first():
    """Zeroing the first d input columns of q/k/v removes every trace of the tokens;
    zeroing the last d removes every trace of x from the attention term."""
    H, W = _head()
    _no_mlp(H)
    x = _x()
    He = {**H, **{w: H[w].copy() for w in ("wq", "wk", "wv")}}
    for w in ("wq", "wk", "wv"):
        He[w][:, :D] = 0
    assert np.array_equal(_run(He, W, _shape(), TOKS, x), _run(He, W, _shape(), TOKS2, x))
    Hx = {**H, **{w: H[w].copy() for w in ("wq", "wk", "wv")}}
    for w in ("wq", "wk", "wv"):
        Hx[w][:, D:] = 0
    x2 = _x(seed=5, scale=3.0)
    np.testing.assert_allclose(_run(Hx, W, _shape(), TOKS, x) - x, _run(Hx, W, _shape(), TOKS, x2) - x2, rtol=0,
                               atol=1e-12)
    # and each half really is read: the unzeroed version depends on both
    assert not np.array_equal(_run(H, W, _shape(), TOKS, x), _run(H, W, _shape(), TOKS2, x))


def test_concat_pin_catches_swapped_halves():
    H, W = _head()
    _no_mlp(H)
    x = _x()
    He = {**H, **{w: H[w].copy() for w in ("wq", "wk", "wv")}}
    for w in ("wq", "wk", "wv"):
        He[w][:, :D] = 0

    def planted(H, W, shp, toks, x, pos, ctx):          # [x ; e] instead of [e ; x]
        Hs = {**H, **{w: np.hstack((H[w][:, D:], H[w][:, :D])) for w in ("wq", "wk", "wv")}}
        return draft_layer(Hs, W, shp, toks, x, pos, ctx)

    diff = _run(He, W, _shape(), TOKS, x, planted) - _run(He, W, _shape(), TOKS2, x, planted)
    assert np.abs(diff).max() > 1e-3


# ------------------------------------------------------------------- the two norms

def test_hidden_norm_makes_attention_input_scale_free():
    """eps = 0: scaling x by 2 (exact in binary) leaves the attention input, hence
    the attention term a - x, bit-identical; scaling the embedding table by 2 leaves
    the whole output bit-identical."""
    H, W = _head()
    _no_mlp(H)
    x = _x()
    a1 = _run(H, W, _shape(), TOKS, x)
    a2 = _run(H, W, _shape(), TOKS, 2 * x)
    np.testing.assert_allclose(a1 - x, a2 - 2 * x, rtol=0, atol=1e-12)
    W2 = {**W, "embed": 2 * W["embed"]}
    H_full, _ = _head()
    np.testing.assert_array_equal(_run(H_full, W, _shape(), TOKS, x), _run(H_full, W2, _shape(), TOKS, x))


def test_hidden_norm_pin_catches_missing_norm(monkeypatch):
    H, W = _head()
    _no_mlp(H)
    x = _x()
    real = llama.rms_norm
    hidden = H["hidden_norm"]
    monkeypatch.setattr(llama, "rms_norm", lambda v, w, eps: v * w if w is hidden else real(v, w, eps))
    a1 = _run(H, W, _shape(), TOKS, x)
    a2 = _run(H, W, _shape(), TOKS, 2 * x)
    assert np.abs((a1 - x) - (a2 - 2 * x)).max() > 1e-3


def test_norm_weights_scale_their_own_half():
    """input_norm's weight multiplies the embedding half of the input and hidden_norm's
    the feature half: a weight of 2 equals doubling that half's q/k/v columns."""
    H, W = _head()
    x = _x()
    for norm, cols in (("input_norm", slice(0, D)), ("hidden_norm", slice(D, 2 * D))):
        Hn = {**H, norm: np.full(D, 2.0)}
        Hc = {**H, **{w: H[w].copy() for w in ("wq", "wk", "wv")}}
        for w in ("wq", "wk", "wv"):
            Hc[w][:, cols] *= 2
        np.testing.assert_allclose(_run(Hn, W, _shape(), TOKS, x), _run(Hc, W, _shape(), TOKS, x), rtol=1e-12,
                                   atol=1e-12)


# ------------------------------------------------------------- post_norm + SwiGLU

def test_post_norm_and_swiglu_closed_form():
    """wo = 0 (no attention term), eps = 0, x a constant row c * 1: post_norm(x) is
    the all-ones vector, so a = x + w_down (silu(rowsum w_gate) * rowsum w_up)
    (silu from scipy's expit; the product is stored in the model's dtype, fp32
    here).  Gate and up are not interchangeable."""
    H, W = _head()
    H["wo"][:] = 0
    x = np.full((1, D), 3.5)
    a = _run(H, W, _shape(), TOKS[:1], x)
    g, u = H["w_gate"].sum(1), H["w_up"].sum(1)
    ref = x[0] + H["w_down"] @ (g * expit(g) * u).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(a[0], ref, rtol=1e-6, atol=1e-9)
    swapped = x[0] + H["w_down"] @ (u * expit(u) * g)
    assert np.abs(a[0] - swapped).max() > 1e-3


# ------------------------------------------------------------------------ fusion FC

def test_fuse_bias_free_and_linear():
    H, _ = _head()
    rng = np.random.default_rng(4)
    a, b = rng.normal(0, 1, (2, 3 * D)), rng.normal(0, 1, (2, 3 * D))
    assert np.array_equal(draft_fuse(H, np.zeros((2, 3 * D))), np.zeros((2, D)))
    np.testing.assert_allclose(draft_fuse(H, 2 * a - 3 * b), 2 * draft_fuse(H, a) - 3 * draft_fuse(H, b),
                               rtol=1e-12, atol=1e-12)


def test_taps_feed_the_fusion_in_ascending_layer_order():
    """A 3-layer target with taps (0, 1, 2) whose layer 0 is the identity (wo =
    w_down = 0): the state entering layers 0 and 1 is the embedding, the state
    entering layer 2 is not.  So the first two d-blocks of the captured row are the
    (rounded) embedding and the third differs; an FC that selects block 0 then
    returns the lowest tap exactly."""
    shp = _shape(dtype="f32", layers=3, taps=(0, 1, 2))
    rng = np.random.default_rng(6)
    g = lambda *s: rng.normal(0, 0.3, s)
    layers = []
    for l in range(3):
        L = {"attn_norm": np.ones(D), "ffn_norm": np.ones(D), "wq": g(HQ * HD, D), "wk": g(HKV * HD, D),
             "wv": g(HKV * HD, D), "wo": g(D, HQ * HD), "w_gate": g(F, D), "w_up": g(F, D), "w_down": g(D, F)}
        if l == 0:
            L["wo"][:] = 0
            L["w_down"][:] = 0
        layers.append(L)
    W = {"embed": g(V, D), "lm_head": g(V, D), "final_norm": np.ones(D), "layers": layers}
    toks = [2, 8, 4]
    cache = KVCache(3, 8, HKV, HD)
    _, _, _, aux = target_forward(W, shp, cache, toks, np.arange(3), causal_visible(3))
    emb = W["embed"][toks].astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(aux[:, :D], emb)
    np.testing.assert_array_equal(aux[:, D:2 * D], emb)
    assert np.abs(aux[:, 2 * D:] - emb).max() > 1e-3
    H = {"fc": np.hstack((np.eye(D), np.zeros((D, 2 * D))))}
    np.testing.assert_array_equal(draft_fuse(H, aux), aux[:, :D])


# ------------------------------------------------------------------ draft logits

def test_draft_logits_use_the_drafts_own_final_norm():
    """Scale-free in a (eps = 0, factor 2: bit-identical); the target's final norm
    weight has no effect, the draft's scales the logits."""
    H, W = _head()
    rng = np.random.default_rng(7)
    a = rng.normal(0, 1, (2, D))
    shp = _shape()
    l1 = draft_logits(H, W, shp, a)
    np.testing.assert_array_equal(l1, draft_logits(H, W, shp, 2 * a))
    np.testing.assert_array_equal(l1, draft_logits(H, {**W, "final_norm": np.full(D, 3.0)}, shp, a))
    np.testing.assert_allclose(draft_logits({**H, "final_norm": np.full(D, 2.0)}, W, shp, a), 2 * l1, rtol=1e-6)
    # the closed form: unit-RMS rows times the head
    r = a / np.sqrt(np.mean(a * a, axis=1, keepdims=True))
    np.testing.assert_allclose(l1, r.astype(np.float32).astype(np.float64) @ W["lm_head"].T, rtol=1e-12)


def test_draft_logits_pin_catches_the_targets_norm(monkeypatch):
    H, W = _head()
    a = np.random.default_rng(7).normal(0, 1, (2, D))
    W3 = {**W, "final_norm": np.full(D, 3.0)}

    def planted(H, W, shp, a):                          # the target's final norm instead of the draft's
        return llama.rounder(shp.dtype)(llama.rms_norm(a, W["final_norm"], shp.eps)) @ W["lm_head"].T

    assert not np.array_equal(planted(H, W, _shape(), a), planted(H, W3, _shape(), a))


# ------------------------------------------------------------ sampled chain draws

def _grid_uniforms(seed, n):
    return np.random.default_rng(seed).integers(0, 1 << 24, n) / float(1 << 24)


def _chi2_p(counts, p):
    exp = p * counts.sum()
    keep = exp >= 5
    obs = np.append(counts[keep], counts[~keep].sum())
    ex = np.append(exp[keep], exp[~keep].sum())
    if ex[-1] < 5:
        obs, ex = obs[:-1], ex[:-1]
    stat = ((obs - ex) ** 2 / ex).sum()
    return chi2.sf(stat, len(obs) - 1)


def _draw_counts(logits, T, n, seed):
    u = _grid_uniforms(seed, n)
    counts = np.zeros(len(logits))
    for i in range(n):
        toks, _ = build_sampled_chain(0, logits, None, 1, T, [u[i]], False)
        counts[toks[1]] += 1
    return counts


def test_sampled_chain_draw_follows_tempered_softmax():
    """1e5 seeded draws of the first draft at T = 0.7 on a 64-id vocabulary match
    softmax(logits / T) (scipy) by chi-square; q returned is that distribution."""
    logits = np.random.default_rng(8).normal(0, 1.5, 64).astype(np.float32)
    T = 0.7
    p = softmax(logits.astype(np.float64) / np.float64(np.float32(T)))
    counts = _draw_counts(logits, T, 100000, 9)
    assert _chi2_p(counts, p) > 1e-3
    _, q = build_sampled_chain(0, logits, None, 1, T, [0.5], False)
    np.testing.assert_allclose(q[0], p, rtol=1e-6)


def test_sampled_chain_pin_catches_untempered_draw():
    """Drawing at T = 1 instead of 0.7 fails the same chi-square (planted by
    calling the draw with the wrong temperature)."""
    logits = np.random.default_rng(8).normal(0, 1.5, 64).astype(np.float32)
    p = softmax(logits.astype(np.float64) / np.float64(np.float32(0.7)))
    counts = _draw_counts(logits, 1.0, 20000, 10)
    assert _chi2_p(counts, p) < 1e-6


def test_sampled_chain_second_draft_is_conditional():
    """K = 2 on an 8-id vocabulary: expand() is called with the first draft and its
    row gives q_2; the pair (d1, d2) is distributed as q_1(d1) q_2(d2 | d1) (64-cell
    chi-square over 4e4 draws)."""
    Vs, T = 8, 1.0
    rng = np.random.default_rng(11)
    root_logits = rng.normal(0, 1, Vs).astype(np.float32)
    table = rng.normal(0, 1.2, (Vs, Vs)).astype(np.float32)   # row = first draft token

    def expand(d, info):
        assert d == 1 and len(info) == 1
        return [table[info[0][0]]]

    n = 40000
    u = _grid_uniforms(12, 2 * n).reshape(n, 2)
    counts = np.zeros((Vs, Vs))
    for i in range(n):
        toks, q = build_sampled_chain(0, root_logits, expand, 2, T, list(u[i]), False)
        counts[toks[1], toks[2]] += 1
    p1 = softmax(root_logits.astype(np.float64))
    joint = p1[:, None] * softmax(table.astype(np.float64), axis=1)
    assert _chi2_p(counts.ravel(), joint.ravel()) > 1e-3


def test_greedy_draft_chain_is_argmax_with_point_mass_q():
    logits = np.array([0.1, 2.0, 2.0, -1.0], dtype=np.float32)
    toks, q = build_sampled_chain(5, logits, None, 1, 1.0, [0.99], True)
    assert toks == [5, 1]                              # first of the tied maxima
    np.testing.assert_array_equal(q[0], [0, 1, 0, 0])
