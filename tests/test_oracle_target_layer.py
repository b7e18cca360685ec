"""Pins of the oracle's target decoder layer, final norm + LM head and decision helpers.

"EAGLE-3: Engineering Implementation of LLM Inference Acceleration", Appendix C
(the LLaMA block the target runs): pre-norm residual blocks, x + o(attention(
RMSNorm(x))) then x + down(SiLU(gate(h)) * up(h)) with h = RMSNorm(x),
grouped-query attention (query head h reads KV head h / (Hq / Hkv)), scores
q . k / sqrt(hd) after rotate-half RoPE, and a final RMSNorm in front of the LM
head.  "Advanced speculative decoding: tree drafts and EAGLE", Implementation:
the verify's decision is the argmax of each row (the first maximal index).

The expected values are computed by other routes than the oracle's own code:
RoPE as a complex rotation (only the position difference enters a score), the
single-key softmax as the identity on the value, SiLU through scipy's expit.
The tests named *_catches_* plant a slip in the oracle (on the CPU) and check
that the pin rejects it.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle.llama as llama
from oracle.accept import argmax_rows_f32
from oracle.llama import Shape, target_layer, target_logits
from oracle.numerics import argmax_first, softmax_f64

HQ, HKV, HD = 4, 2, 8
D = HQ * HD          # the output projection can be the identity
F = D
TOL = 2e-6           # the oracle rounds its f32-stored intermediates; the expected values do not


def _shape(eps=1e-6, theta=1e4):
    return Shape(1, D, HQ, HKV, HD, F, 11, theta, eps, "f32", (0, 0, 0))


def _layer(seed=0, sigma=0.3):
    rng = np.random.default_rng(seed)
    g = lambda *s: rng.normal(0, sigma, s)
    return {"attn_norm": 1.0 + 0.1 * g(D), "wq": g(HQ * HD, D), "wk": g(HKV * HD, D), "wv": g(HKV * HD, D),
            "wo": np.eye(D), "ffn_norm": 1.0 + 0.1 * g(D), "w_gate": g(F, D), "w_up": g(F, D),
            "w_down": np.zeros((D, F))}


def _norm(x, w, eps):
    """RMSNorm written out per row."""
    return np.stack([r * w / np.sqrt(np.sum(r * r) / r.size + eps) for r in np.asarray(x, dtype=np.float64)])


def _run(L, x, positions, visible, shp=None):
    shp = shp or _shape()
    P = 0
    out, k, v = target_layer(L, shp, x, np.zeros((P, HKV, HD)), np.zeros((P, HKV, HD)), positions, visible)
    return out, k, v


# ----------------------------------------------------------------- residuals

def test_zero_branches_leave_the_residual():
    """With the output and down projections zero, both blocks add nothing: the
    layer returns its input exactly (a block that replaced x would not)."""
    L = _layer()
    L["wo"] = np.zeros((D, HQ * HD))
    x = np.random.default_rng(1).normal(0, 1, (3, D))
    out, _, _ = _run(L, x, np.arange(3), [[0], [0, 1], [0, 1, 2]])
    assert np.array_equal(out, x)


# --------------------------------------------------------- attention: value path

def _value_path_expected(L, x, shp):
    h = _norm(x, L["attn_norm"], shp.eps)
    v = (h @ L["wv"].T).reshape(len(x), HKV, HD)
    G = HQ // HKV
    return x + np.concatenate([v[:, qh // G, :] for qh in range(HQ)], axis=1)


def test_single_key_attention_is_the_value_of_its_kv_head():
    """A row that sees one key attends with weight 1: with the identity output
    projection and no MLP, query head h's slice of the output delta is the
    value of KV head h / (Hq / Hkv) of the row's own (normed) input."""
    shp = _shape()
    L = _layer(2)
    x = np.random.default_rng(3).normal(0, 1, (2, D))
    out, _, _ = _run(L, x, np.array([5, 9]), [[0], [1]], shp)   # each row sees only itself
    np.testing.assert_allclose(out, _value_path_expected(L, x, shp), rtol=TOL, atol=TOL)


def test_gqa_pin_catches_interleaved_head_map(monkeypatch):
    """Planted slip: query head h reads KV head h mod Hkv."""
    def bad_attend(q, keys, vals, n_kv_heads):
        hq, hd = q.shape
        out = np.empty((hq, hd))
        for h in range(hq):
            kv = h % n_kv_heads
            s = keys[:, kv, :] @ q[h] / np.sqrt(hd)
            p = np.exp(s - s.max())
            out[h] = (p / p.sum()) @ vals[:, kv, :]
        return out
    monkeypatch.setattr(llama, "attend", bad_attend)
    shp = _shape()
    L = _layer(2)
    x = np.random.default_rng(3).normal(0, 1, (2, D))
    out, _, _ = _run(L, x, np.array([5, 9]), [[0], [1]], shp)
    assert not np.allclose(out, _value_path_expected(L, x, shp), atol=1e-6)


# ------------------------------------------------------ attention: two keys, RoPE

def _complex(v):
    """Rotate-half layout as complex pairs: dims i and i + hd/2 are re, im."""
    h = v.shape[-1] // 2
    return v[..., :h] + 1j * v[..., h:]


def _two_key_expected(L, x, pos, shp):
    """Row 1 sees rows 0 and 1.  The score of query head h against key j is
    Re(sum_i q_i conj(k_i) e^{i (p_1 - p_j) w_i}) / sqrt(hd) with w_i =
    theta^(-2i/hd): RoPE as a complex rotation, where only the position
    difference enters."""
    h = _norm(x, L["attn_norm"], shp.eps)
    q = (h @ L["wq"].T).reshape(2, HQ, HD)
    k = (h @ L["wk"].T).reshape(2, HKV, HD)
    v = (h @ L["wv"].T).reshape(2, HKV, HD)
    w = shp.rope_theta ** (-np.arange(0, HD, 2) / HD)
    G = HQ // HKV
    o = []
    for qh in range(HQ):
        kv = qh // G
        qc = _complex(q[1, qh])
        s = np.array([np.real(np.sum(qc * np.conj(_complex(k[j, kv])) * np.exp(1j * (pos[1] - pos[j]) * w)))
                      for j in range(2)]) / np.sqrt(HD)
        a = expit(s[1] - s[0])          # two-way softmax: weight of key 1
        o.append((1 - a) * v[0, kv] + a * v[1, kv])
    return x[1] + np.concatenate(o)


@pytest.mark.parametrize("pos", [(0, 1), (7, 19), (100, 96)])
def test_two_key_attention_matches_complex_rope_form(pos):
    shp = _shape()
    L = _layer(4, sigma=0.5)
    x = np.random.default_rng(5).normal(0, 1, (2, D))
    out, _, _ = _run(L, x, np.array(pos), [[0], [0, 1]], shp)
    np.testing.assert_allclose(out[1], _two_key_expected(L, x, pos, shp), rtol=TOL, atol=TOL)


def test_rope_pin_catches_swapped_query_and_key():
    """Planted slip: the query is built from wk and the key from wq (equal
    scores at equal positions, not across a position gap)."""
    shp = _shape()
    L = _layer(4, sigma=0.5)
    x = np.random.default_rng(5).normal(0, 1, (2, D))
    pos = (7, 19)
    want = _two_key_expected(L, x, pos, shp)
    Lbad = dict(L)
    Lbad["wq"] = np.concatenate([L["wk"]] * (HQ // HKV), axis=0)[:HQ * HD]
    Lbad["wk"] = L["wq"][:HKV * HD]
    out, _, _ = _run(Lbad, x, np.array(pos), [[0], [0, 1]], shp)
    assert not np.allclose(out[1], want, atol=1e-6)


def test_rope_pin_catches_a_reversed_rotation(monkeypatch):
    """Planted slip: the rotation runs the other way (sin with the wrong sign)."""
    good = llama.rope
    monkeypatch.setattr(llama, "rope", lambda x, pos, theta: good(x, -np.asarray(pos, dtype=np.float64), theta))
    shp = _shape()
    L = _layer(4, sigma=0.5)
    x = np.random.default_rng(5).normal(0, 1, (2, D))
    pos = (7, 19)
    out, _, _ = _run(L, x, np.array(pos), [[0], [0, 1]], shp)
    assert not np.allclose(out[1], _two_key_expected(L, x, pos, shp), atol=1e-5)


# ----------------------------------------------------------------------- MLP

def _mlp_expected(L, x, shp):
    h = _norm(x, L["ffn_norm"], shp.eps)
    g, u = h @ L["w_gate"].T, h @ L["w_up"].T
    return x + (g * expit(g) * u) @ L["w_down"].T


def test_mlp_block_is_silu_gate_times_up():
    """With the attention's output projection zero, the layer adds
    down(SiLU(gate(h)) * up(h)), h = RMSNorm(x) with the MLP's own norm weight."""
    shp = _shape()
    L = _layer(6, sigma=0.4)
    L["wo"] = np.zeros((D, HQ * HD))
    L["w_down"] = np.random.default_rng(7).normal(0, 0.3, (D, F))
    x = np.random.default_rng(8).normal(0, 1, (3, D))
    out, _, _ = _run(L, x, np.arange(3), [[0], [0, 1], [0, 1, 2]], shp)
    np.testing.assert_allclose(out, _mlp_expected(L, x, shp), rtol=TOL, atol=TOL)


def test_mlp_pin_catches_swapped_gate_and_up():
    shp = _shape()
    L = _layer(6, sigma=0.4)
    L["wo"] = np.zeros((D, HQ * HD))
    L["w_down"] = np.random.default_rng(7).normal(0, 0.3, (D, F))
    x = np.random.default_rng(8).normal(0, 1, (3, D))
    want = _mlp_expected(L, x, shp)
    Lbad = dict(L)
    Lbad["w_gate"], Lbad["w_up"] = L["w_up"], L["w_gate"]
    out, _, _ = _run(Lbad, x, np.arange(3), [[0], [0, 1], [0, 1, 2]], shp)
    assert not np.allclose(out, want, atol=1e-6)


# -------------------------------------------------------- final norm + LM head

def test_logits_are_the_final_norm_through_the_head():
    """Identity LM head: the logits are RMSNorm(x) with the final norm weight,
    so they do not change when x is scaled."""
    shp = Shape(1, D, HQ, HKV, HD, F, D, 1e4, 0.0, "f32", (0, 0, 0))
    w = 1.0 + 0.2 * np.random.default_rng(9).normal(0, 1, D)
    W = {"final_norm": w, "lm_head": np.eye(D)}
    x = np.random.default_rng(10).normal(0, 1, (3, D))
    lg = target_logits(W, shp, x)
    np.testing.assert_allclose(lg, _norm(x, w, 0.0), rtol=TOL, atol=TOL)
    np.testing.assert_allclose(target_logits(W, shp, 4.0 * x), lg, rtol=2e-7)


def test_logits_pin_catches_a_missing_final_norm(monkeypatch):
    monkeypatch.setattr(llama, "rms_norm", lambda x, w, eps: np.asarray(x, dtype=np.float64) * w)
    shp = Shape(1, D, HQ, HKV, HD, F, D, 1e4, 0.0, "f32", (0, 0, 0))
    W = {"final_norm": np.ones(D), "lm_head": np.eye(D)}
    x = np.random.default_rng(10).normal(0, 1, (3, D))
    assert not np.allclose(target_logits(W, shp, 4.0 * x), target_logits(W, shp, x), rtol=1e-3)


# ------------------------------------------------------------ decision helpers

def test_argmax_first_takes_the_lowest_index_of_a_tie():
    rng = np.random.default_rng(11)
    for _ in range(50):
        r = rng.integers(0, 5, 17).astype(np.float64)
        top = np.flatnonzero(r == r.max())
        assert argmax_first(r) == top[0]


def test_row_argmax_decides_in_float32():
    """Two values that differ only below float32 precision are a tie at the
    decision precision: the lower index wins."""
    a = np.float64(np.float32(1.25))
    rows = np.array([[0.0, a, a + 1e-12, -1.0],
                     [3.0, 2.0, 3.0 + 1e-13, 3.0],
                     [-2.0, -1.0, -3.0, -1.5]])
    assert argmax_rows_f32(rows) == [1, 0, 1]


def test_softmax_two_way_is_the_logistic_and_shift_free():
    rng = np.random.default_rng(12)
    for _ in range(20):
        a, b = rng.normal(0, 20, 2)
        p = softmax_f64(np.array([a, b]))
        np.testing.assert_allclose(p, [expit(a - b), expit(b - a)], rtol=1e-13, atol=1e-300)
    z = rng.normal(0, 5, (4, 9))
    np.testing.assert_allclose(softmax_f64(z + 1234.5), softmax_f64(z), rtol=1e-12)
    np.testing.assert_allclose(softmax_f64(z).sum(axis=-1), 1.0, rtol=1e-14)
