"""Pins of the oracle's model code: closed forms, invariants and the pages' tree check."""
import numpy as np
from scipy.special import expit

from oracle.llama import KVCache, attend, causal_visible, rms_norm, rope, silu, target_forward
from oracle.tree import tree_mask


def test_rms_norm_unit_rms():
    x = np.random.default_rng(0).normal(0, 3, (4, 96))
    y = rms_norm(x, np.ones(96), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, -1)), 1.0, rtol=1e-12)
    y2 = rms_norm(x, np.full(96, 2.0), 0.0)
    np.testing.assert_allclose(y2, 2 * y, rtol=1e-12)


def test_rope_is_complex_rotation():
    """Rotate-half RoPE == multiplying (x_i + j x_{i+hd/2}) by exp(j pos theta^(-2i/hd))."""
    rng = np.random.default_rng(1)
    hd, theta = 16, 1e4
    x = rng.normal(0, 1, (3, 2, hd))
    pos = np.array([0, 5, 1234])
    y = rope(x, pos, theta)
    half = hd // 2
    z = x[..., :half] + 1j * x[..., half:]
    ang = pos[:, None, None] * theta ** (-2.0 * np.arange(half) / hd)
    w = z * np.exp(1j * ang)
    np.testing.assert_allclose(y[..., :half], w.real, atol=1e-12)
    np.testing.assert_allclose(y[..., half:], w.imag, atol=1e-12)
    np.testing.assert_allclose(y[0], x[0], atol=0)                 # position 0 is the identity


def test_rope_relative_position():
    rng = np.random.default_rng(2)
    q, k = rng.normal(0, 1, (1, 1, 32)), rng.normal(0, 1, (1, 1, 32))
    a = np.sum(rope(q, np.array([17]), 5e5) * rope(k, np.array([9]), 5e5))
    b = np.sum(rope(q, np.array([1017]), 5e5) * rope(k, np.array([1009]), 5e5))
    assert abs(a - b) < 1e-9


def test_silu_closed_form():
    x = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(silu(x), x * expit(x), rtol=1e-12, atol=1e-300)


def test_attend_special_cases():
    rng = np.random.default_rng(3)
    hq, hkv, hd = 4, 2, 8
    q = rng.normal(0, 1, (hq, hd))
    keys = rng.normal(0, 1, (1, hkv, hd))
    vals = rng.normal(0, 1, (1, hkv, hd))
    out = attend(q, keys, vals, hkv)                        # one key: output is that value
    for h in range(hq):
        np.testing.assert_allclose(out[h], vals[0, h // 2], atol=1e-14)
    keys = rng.normal(0, 1, (5, hkv, hd))
    vals = rng.normal(0, 1, (5, hkv, hd))
    out = attend(np.zeros((hq, hd)), keys, vals, hkv)        # q = 0: the mean of the values
    for h in range(hq):
        np.testing.assert_allclose(out[h], vals[:, h // 2].mean(0), atol=1e-14)
    # explicit softmax for one head
    h = 3
    s = keys[:, 1] @ q[h] / np.sqrt(hd)
    p = np.exp(s) / np.exp(s).sum()
    np.testing.assert_allclose(attend(q, keys, vals, hkv)[h], p @ vals[:, 1], atol=1e-13)


def test_tap_zero_is_the_embedding(toy_model):
    ms, shp, W, H = toy_model(taps=(0, 1, 1))
    cache = KVCache(shp.n_layers, 32, shp.n_kv_heads, shp.head_dim)
    toks = [1, 4, 2]
    _, _, _, aux = target_forward(W, shp, cache, toks, np.arange(3), causal_visible(3))
    np.testing.assert_array_equal(aux[:, :shp.d], W["embed"][toks])


def test_tree_rows_equal_per_path_recompute(toy_model):
    """The pages' tree-attention check: each tree node's logits equal those of its path
    computed as an ordinary causal sequence after the same prefix (pages: < 1e-3)."""
    ms, shp, W, H = toy_model(dtype="f32", vocab=32)
    cache = KVCache(shp.n_layers, 64, shp.n_kv_heads, shp.head_dim)
    prefix = [3, 9, 1, 30, 7]
    n = len(prefix)
    _, k, v, _ = target_forward(W, shp, cache, prefix, np.arange(n), causal_visible(n))
    for l in range(shp.n_layers):
        cache.k[l][:n], cache.v[l][:n] = k[l], v[l]
    cache.length = n
    tokens, parents = [10, 20, 31, 4, 5, 6], [-1, 0, 0, 1, 1, 2]
    m = tree_mask(parents)
    dep = [0, 1, 1, 2, 2, 2]
    logits, _, _, _ = target_forward(W, shp, cache, tokens, n + np.array(dep),
                                     [list(np.nonzero(m[i])[0]) for i in range(6)])
    worst = 0.0
    for node in range(6):
        chain = [tokens[j] for j in np.nonzero(m[node])[0]]
        c2 = KVCache(shp.n_layers, 64, shp.n_kv_heads, shp.head_dim)
        full = prefix + chain
        ref, _, _, _ = target_forward(W, shp, c2, full, np.arange(len(full)), causal_visible(len(full)))
        worst = max(worst, np.abs(logits[node] - ref[-1]).max())
    assert worst < 1e-9


def test_tap_at_layer_count_is_the_last_output(toy_model):
    """hidden_states[L] (a tap index equal to the layer count) is the output of
    the last layer: the residual entering layer L of a deeper model."""
    ms, shp, W, H = toy_model(taps=(0, 1, 2), layers=2)
    deeper = dict(W)
    deeper["layers"] = W["layers"] + [W["layers"][0]]
    from dataclasses import replace
    shp3 = replace(shp, n_layers=3)
    toks = [3, 1, 4, 1]
    c2 = KVCache(2, 8, shp.n_kv_heads, shp.head_dim)
    c3 = KVCache(3, 8, shp.n_kv_heads, shp.head_dim)
    _, _, _, a2 = target_forward(W, shp, c2, toks, np.arange(4), causal_visible(4))
    _, _, _, a3 = target_forward(deeper, shp3, c3, toks, np.arange(4), causal_visible(4))
    np.testing.assert_array_equal(a2, a3)
