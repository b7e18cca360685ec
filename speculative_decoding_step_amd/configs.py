"""The five workloads and their seeded synthetic weights.

Shapes follow the pages' LLaMA-style target (RMSNorm eps 1e-5, rotate-half
RoPE, SwiGLU) and the EAGLE-3 head of "EAGLE-3: Engineering Implementation of
LLM Inference Acceleration" (VIII, IX).  Taps are hidden_states indices: the
residual stream entering 0-indexed decoder layer t.

Every matrix is drawn from N(0, 0.02) through :mod:`synth`; norm weights are 1.
Seeds: target 1000 + id, head 2000 + id, prompts 3000 + id, ragged lengths
4000, sampler uniforms 5000.
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from . import synth


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float
    taps: tuple
    dtype: str = "bf16"
    eps: float = 1e-5
    draft_vocab: int = 0    # 0: the draft shares the target's full-vocabulary head; else its own head over V_d ids


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    shape: ModelShape
    mode: str               # "greedy_tree" | "sample_chain" | "sample_tree"
    depth: int
    topk: int
    n_nodes: int
    batch: int
    prompt_len: int         # fixed length, or the upper bound when ragged
    max_new: int
    temperature: float = 0.0
    draft_greedy: bool = False
    ragged_min: int = 0     # > 0: prompt lengths uniform in [ragged_min, prompt_len]
    max_len: int = 0        # > 0: sequences stop at this total length
    block_size: int = 0     # > 0: paged KV caches of blocks of this many positions (shuffled over the pool)

    @property
    def rows(self):
        return self.n_nodes + 1

    @property
    def target_seed(self):
        return 1000 + self.cid

    @property
    def head_seed(self):
        return 2000 + self.cid

    @property
    def prompt_seed(self):
        return 3000 + self.cid


TINY = ModelShape(4, 256, 4, 4, 64, 688, 1024, 1e4, (1, 2, 3), dtype="f32")
SMALL = ModelShape(8, 1024, 16, 16, 64, 2816, 32000, 1e4, (1, 4, 7))
L8B = ModelShape(32, 4096, 32, 8, 128, 14336, 128256, 5e5, (2, 16, 29))
L8B_DV32K = replace(L8B, draft_vocab=32000)  # the official recipe's reduced draft vocabulary

WORKLOADS = {
    "tiny_f32_chain": Workload(1, "tiny_f32_chain", TINY, "greedy_tree", 4, 1, 4, 1, 32, 64),
    "small_bf16_tree": Workload(2, "small_bf16_tree", SMALL, "greedy_tree", 6, 4, 32, 1, 512, 256),
    "llama8b_tree_b1": Workload(3, "llama8b_tree_b1", L8B, "greedy_tree", 6, 10, 60, 1, 2048, 128),
    "llama8b_sample_chain_b4": Workload(4, "llama8b_sample_chain_b4", L8B, "sample_chain", 5, 1, 5,
                                        4, 64, 192, temperature=1.0, max_len=256),
    "llama8b_tree_b64": Workload(5, "llama8b_tree_b64", L8B, "greedy_tree", 4, 4, 16, 64, 4096, 32,
                                 ragged_min=128),
    # the batch-1 tree under sampling: the same draft tree, accepted by level-by-level rejection sampling at T = 1
    "llama8b_sample_tree_b1": Workload(6, "llama8b_sample_tree_b1", L8B, "sample_tree", 6, 10, 60, 1, 2048, 128,
                                       temperature=1.0),
    # the batch-1 tree with a 32,000-id draft vocabulary (draft-owned head, d2t)
    "llama8b_tree_b1_dv32k": Workload(7, "llama8b_tree_b1_dv32k", L8B_DV32K, "greedy_tree", 6, 10, 60, 1, 2048, 128),
}
# the batch-1 and batch-64 trees on paged KV caches of 64-position blocks (same seeds and prompts as the
# contiguous workloads, so the lines compare directly)
WORKLOADS["llama8b_tree_b1_paged"] = replace(WORKLOADS["llama8b_tree_b1"], name="llama8b_tree_b1_paged",
                                             block_size=64)
WORKLOADS["llama8b_tree_b64_paged"] = replace(WORKLOADS["llama8b_tree_b64"], name="llama8b_tree_b64_paged",
                                              block_size=64)


def scaled(w: Workload, **kw) -> Workload:
    return replace(w, **kw)


def prompt_lengths(w: Workload) -> np.ndarray:
    if w.ragged_min > 0:
        return synth.randint_np(4000, "ragged_len", w.batch, w.ragged_min, w.prompt_len)
    return np.full(w.batch, w.prompt_len, dtype=np.int64)


def prompts_np(w: Workload):
    lens = prompt_lengths(w)
    return [synth.tokens_np(w.prompt_seed, f"prompt{b}", int(lens[b]), w.shape.vocab)
            for b in range(w.batch)]


def target_tensor_specs(s: ModelShape):
    """(name, shape, kind) of every target tensor; kind 'mat' ~ N(0, 0.02), 'norm' = 1."""
    d, hd = s.d, s.head_dim
    out = [("embed", (s.vocab, d), "mat")]
    for l in range(s.n_layers):
        out += [
            (f"l{l}.attn_norm", (d,), "norm"),
            (f"l{l}.wq", (s.n_heads * hd, d), "mat"),
            (f"l{l}.wk", (s.n_kv_heads * hd, d), "mat"),
            (f"l{l}.wv", (s.n_kv_heads * hd, d), "mat"),
            (f"l{l}.wo", (d, s.n_heads * hd), "mat"),
            (f"l{l}.ffn_norm", (d,), "norm"),
            (f"l{l}.w_gate", (s.ffn, d), "mat"),
            (f"l{l}.w_up", (s.ffn, d), "mat"),
            (f"l{l}.w_down", (d, s.ffn), "mat"),
        ]
    out += [("final_norm", (d,), "norm"), ("lm_head", (s.vocab, d), "mat")]
    return out


def head_tensor_specs(s: ModelShape):
    d, hd = s.d, s.head_dim
    return [
        ("h.fc", (d, 3 * d), "mat"),
        ("h.input_norm", (d,), "norm"),
        ("h.hidden_norm", (d,), "norm"),
        ("h.wq", (s.n_heads * hd, 2 * d), "mat"),
        ("h.wk", (s.n_kv_heads * hd, 2 * d), "mat"),
        ("h.wv", (s.n_kv_heads * hd, 2 * d), "mat"),
        ("h.wo", (d, s.n_heads * hd), "mat"),
        ("h.post_norm", (d,), "norm"),
        ("h.w_gate", (s.ffn, d), "mat"),
        ("h.w_up", (s.ffn, d), "mat"),
        ("h.w_down", (d, s.ffn), "mat"),
        ("h.final_norm", (d,), "norm"),
    ] + ([("h.lm_head", (s.draft_vocab, d), "mat")] if s.draft_vocab > 0 else [])


def d2t_np(s: ModelShape, head_seed: int) -> np.ndarray:
    """The reduced draft vocabulary's map to target ids (ascending): a seeded subset of
    V_d ids.  The pages pick the most frequent tokens of the training responses; with
    synthetic weights any fixed subset has the same shapes."""
    return synth.subset_np(head_seed, "h.d2t", s.draft_vocab, s.vocab)


def tensor_np(seed: int, name: str, shape, kind: str, dtype: str, sigma: float = 0.02) -> np.ndarray:
    if kind == "norm":
        return np.ones(shape, dtype=np.float32)
    return synth.normal_np(seed, name, shape, sigma, dtype)


def weights_np(s: ModelShape, target_seed: int, head_seed: int, layers=None, sigma: float = 0.02):
    """float64 weight dicts (W target, H head) in the oracle's layout.

    ``layers`` restricts which target layers are materialised (others are None),
    so the 8B shape can be sampled layer by layer on a host.  ``sigma`` other
    than the configs' 0.02 is for small test models only.
    """
    W = {"layers": [None] * s.n_layers}
    for name, shp, kind in target_tensor_specs(s):
        if name[0] == "l" and name[1].isdigit():
            l, key = name[1:].split(".", 1)
            l = int(l)
            if layers is not None and l not in layers:
                continue
            if W["layers"][l] is None:
                W["layers"][l] = {}
            W["layers"][l][key] = tensor_np(target_seed, name, shp, kind, s.dtype, sigma).astype(np.float64)
        else:
            W[name] = tensor_np(target_seed, name, shp, kind, s.dtype, sigma).astype(np.float64)
    H = {}
    for name, shp, kind in head_tensor_specs(s):
        H[name[2:]] = tensor_np(head_seed, name, shp, kind, s.dtype, sigma).astype(np.float64)
    if s.draft_vocab > 0:
        H["d2t"] = d2t_np(s, head_seed)
    return W, H
