"""LLaMA-shaped target forward and the EAGLE-3 draft head, float64 with storage rounding.

Sources (page title, section):
  * "EAGLE-3: Engineering Implementation of LLM Inference Acceleration",
    VIII.1 (draft decoder layer: two RMSNorms, [e ; x] into attention, the
    residual stream is x only, SwiGLU MLP), VIII.2 (Q/K/V read the 2k input,
    grouped-query attention), VIII.4-VIII.5 (frozen shared embedding, final
    norm + LM head), IX.1-IX.6 (taps: hidden state entering decoder layer i,
    concatenated low/mid/high and fused by a bias-free 3k->k FC), Appendix C
    (RMSNorm, rotate-half RoPE with inverse frequencies theta^(-2i/d)).
  * "Advanced speculative decoding: tree drafts and EAGLE", Implementation
    (forward_with_mask: new rows see the whole cached prefix plus the rows the
    mask allows; positions are prefix length + depth; the cache is untouched).
  * "Speculative Decoding (EAGLE3) in the vLLM Neuron Framework", Eagle3 Draft
    Model Architecture (input_layernorm(embeds), hidden_norm(hidden), concat,
    attention, residual, post-attention norm + MLP; the pre-norm output is the
    recurrent state).

Weights are float64 arrays whose values are exact in the storage dtype; a
linear layer's weight is [out, in] and is applied as x @ W.T.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import rounder


@dataclass
class Shape:
    n_layers: int
    d: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float
    eps: float
    dtype: str           # storage dtype: "bf16" or "f32"
    taps: tuple          # hidden_states indices (residual entering 0-indexed layer t)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis (Appendix C, RMSNorm)."""
    x = np.asarray(x, dtype=np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * w


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding (Appendix C, rope).  x: [T, H, hd], pos: [T]."""
    hd = x.shape[-1]
    half = hd // 2
    inv = 1.0 / (float(theta) ** (np.arange(0, hd, 2, dtype=np.float64) / hd))   # [half]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]             # [T, half]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def attend(q: np.ndarray, keys: np.ndarray, vals: np.ndarray, n_kv_heads: int) -> np.ndarray:
    """One query row over an explicit key list, grouped-query.

    q: [Hq, hd]; keys, vals: [n, Hkv, hd] in ascending position order.
    Query head h reads KV head h // (Hq / Hkv) (repeat_interleave of the KV
    heads).  Scores are scaled by 1/sqrt(hd) and softmaxed in float64.
    """
    hq, hd = q.shape
    group = hq // n_kv_heads
    out = np.empty((hq, hd), dtype=np.float64)
    for h in range(hq):
        kv = h // group
        s = keys[:, kv, :] @ q[h] / np.sqrt(hd)
        s = s - np.max(s)
        p = np.exp(s)
        p /= np.sum(p)
        out[h] = p @ vals[:, kv, :]
    return out


class KVCache:
    """Per-layer K and V, [capacity, Hkv, hd] each; positions [0, length) are committed."""

    def __init__(self, n_layers: int, capacity: int, n_kv_heads: int, head_dim: int):
        self.k = [np.zeros((capacity, n_kv_heads, head_dim)) for _ in range(n_layers)]
        self.v = [np.zeros((capacity, n_kv_heads, head_dim)) for _ in range(n_layers)]
        self.length = 0


def causal_visible(t: int):
    return [list(range(i + 1)) for i in range(t)]


def target_layer(L: dict, shp: Shape, x: np.ndarray, past_k: np.ndarray, past_v: np.ndarray, positions, visible):
    """One target decoder layer over T new rows (Appendix C's LLaMA block; the
    new rows attend as in the pages' forward_with_mask).

    x: [T, d] residual stream entering the layer.  past_k / past_v: [P, Hkv, hd]
    the layer's committed keys and values.  Row i sees all P committed keys and
    the new rows listed in visible[i].  Returns (x leaving the layer, the new
    rows' rotated, rounded K and V [T, Hkv, hd]).
    """
    rnd = rounder(shp.dtype)
    T = x.shape[0]
    hq, hkv, hd = shp.n_heads, shp.n_kv_heads, shp.head_dim
    h = rnd(rms_norm(x, L["attn_norm"], shp.eps))
    q = rnd(rope((h @ L["wq"].T).reshape(T, hq, hd), positions, shp.rope_theta))
    k = rnd(rope((h @ L["wk"].T).reshape(T, hkv, hd), positions, shp.rope_theta))
    v = rnd((h @ L["wv"].T).reshape(T, hkv, hd))
    o = np.empty((T, hq, hd))
    for i in range(T):
        sel = list(visible[i])
        o[i] = attend(q[i], np.concatenate([past_k, k[sel]], axis=0), np.concatenate([past_v, v[sel]], axis=0), hkv)
    x = x + rnd(o).reshape(T, hq * hd) @ L["wo"].T
    h2 = rnd(rms_norm(x, L["ffn_norm"], shp.eps))
    act = rnd(silu(h2 @ L["w_gate"].T) * (h2 @ L["w_up"].T))
    return x + act @ L["w_down"].T, k, v


def target_logits(W: dict, shp: Shape, x: np.ndarray) -> np.ndarray:
    """Final RMSNorm, storage rounding, LM head: logits [T, V] of the residual x [T, d]."""
    return rounder(shp.dtype)(rms_norm(x, W["final_norm"], shp.eps)) @ W["lm_head"].T


def target_forward(W: dict, shp: Shape, cache: KVCache, tokens, positions, visible):
    """One target pass over T new rows (the pages' forward_with_mask).

    Every new row sees the cache's committed prefix [0, cache.length) and the
    new rows listed in ``visible[i]`` (ascending, including i itself).
    Returns (logits [T, V] float64, new K and V per layer [T, Hkv, hd],
    aux [T, 3d] = the storage-rounded residual entering each tap layer).
    The cache is not modified.
    """
    rnd = rounder(shp.dtype)
    tokens = np.asarray(tokens, dtype=np.int64)
    T, d = len(tokens), shp.d
    P = cache.length
    x = W["embed"][tokens].astype(np.float64)
    aux = np.zeros((T, len(shp.taps) * d))
    new_k, new_v = [], []
    for l in range(shp.n_layers):
        for ti, t in enumerate(shp.taps):
            if t == l:
                aux[:, ti * d:(ti + 1) * d] = rnd(x)
        x, k, v = target_layer(W["layers"][l], shp, x, cache.k[l][:P], cache.v[l][:P], positions, visible)
        new_k.append(k)
        new_v.append(v)
    for ti, t in enumerate(shp.taps):       # hidden_states[L]: the last layer's output
        if t == shp.n_layers:
            aux[:, ti * d:(ti + 1) * d] = rnd(x)
    return target_logits(W, shp, x), new_k, new_v, aux


# ----------------------------------------------------------------- EAGLE-3 head

def draft_fuse(H: dict, aux_rows: np.ndarray) -> np.ndarray:
    """g = W_fc [l; m; h], bias-free 3d -> d (IX.5 FC Projection).  Kept unrounded."""
    return np.asarray(aux_rows, dtype=np.float64) @ H["fc"].T


def draft_layer(H: dict, W: dict, shp: Shape, e_tokens, x: np.ndarray, positions, context):
    """The EAGLE-3 draft decoder layer over T rows (VIII.1, VIII.2).

    e_tokens: [T] token ids whose (shared, frozen) embeddings form the e stream.
    x:        [T, d] the feature stream (g at real positions, a at drafted ones).
    context(i, k_new, v_new) -> (keys, vals) the ascending key list row i
              attends to, given this call's rotated, rounded K and V [T, Hkv, hd].
    Returns (a [T, d] float64, the layer output before the final norm;
             k_new, v_new [T, Hkv, hd]).

    Two separate RMSNorms (input_norm on e, hidden_norm on x) feed one 2d-wide
    input to q/k/v, embedding half first.  Only x is carried forward: the
    attention and MLP outputs are added to x, and the embedding never enters
    the sum.  The MLP is SwiGLU on post_norm of that sum.
    """
    rnd = rounder(shp.dtype)
    T = len(e_tokens)
    hq, hkv, hd = shp.n_heads, shp.n_kv_heads, shp.head_dim
    e = W["embed"][np.asarray(e_tokens, dtype=np.int64)].astype(np.float64)
    feat = np.asarray(x, dtype=np.float64)
    joint = np.hstack((rnd(rms_norm(e, H["input_norm"], shp.eps)),
                       rnd(rms_norm(feat, H["hidden_norm"], shp.eps))))       # [T, 2d]

    def heads(w, n):
        return (joint @ w.T).reshape(T, n, hd)

    q = rnd(rope(heads(H["wq"], hq), positions, shp.rope_theta))
    k = rnd(rope(heads(H["wk"], hkv), positions, shp.rope_theta))
    v = rnd(heads(H["wv"], hkv))
    att = np.stack([attend(q[i], *context(i, k, v), hkv) for i in range(T)])
    mid = feat + rnd(att).reshape(T, hq * hd) @ H["wo"].T
    z = rnd(rms_norm(mid, H["post_norm"], shp.eps))
    gated = rnd(silu(z @ H["w_gate"].T) * (z @ H["w_up"].T))
    return mid + gated @ H["w_down"].T, k, v


def draft_logits(H: dict, W: dict, shp: Shape, a: np.ndarray) -> np.ndarray:
    """logits = lm_head(norm(a)) with the draft's own final norm.  The head is the
    target's (shared, full vocabulary), or the draft's own head over a reduced draft
    vocabulary when H holds "lm_head" ("EAGLE-3: Engineering Implementation of LLM
    Inference Acceleration", VIII.5-VIII.6: logits over V_d, d2t back to target ids)."""
    rnd = rounder(shp.dtype)
    head = H["lm_head"] if "lm_head" in H else W["lm_head"]
    return rnd(rms_norm(a, H["final_norm"], shp.eps)) @ head.T
