"""Shared helpers of the GPU parity tests (engine factories, oracle twins)."""
import numpy as np
import torch

from conftest import oracle_shape
from speculative_decoding_step_amd import configs
from speculative_decoding_step_amd.engine import Engine, Spec


def toy_shape(dtype="bf16", vocab=512, layers=2, d=256, heads=4, kv=2, hd=64, ffn=512, taps=(0, 1, 1)):
    return configs.ModelShape(layers, d, heads, kv, hd, ffn, vocab, 1e4, taps, dtype=dtype)


def make_engine(ms, spec: Spec, batch=1, max_seq=256, seed=11, sigma=0.02, **kw):
    return Engine(ms, spec, batch, max_seq, seed, seed + 1, sigma=sigma, **kw)


def oracle_weights(ms, seed=11, sigma=0.02):
    W, H = configs.weights_np(ms, seed, seed + 1, sigma=sigma)
    return oracle_shape(ms), W, H


def kv_view(eng: Engine):
    """Target KV cache as [L, 2, B, Hkv, S, hd] in position order (device tensor; a
    gathered copy when the cache is paged)."""
    return eng.kv_logical("target")


def logits_close(gpu, ref, dtype):
    """The logits parity bar: 2e-2 absolute for bf16 models, 1e-4 relative (to the
    row's largest magnitude) for fp32 models."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(gpu - ref)
    if dtype == "bf16":
        return float(err.max()), bool(err.max() <= 2e-2)
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    rel = (err / scale).max()
    return float(rel), bool(rel <= 1e-4)


def margin_tol(dtype, row):
    return 2e-2 if dtype == "bf16" else 1e-4 * float(np.abs(row).max())


def top2_margin(row):
    s = np.sort(np.asarray(row, dtype=np.float64))
    return s[-1] - s[-2]


def random_tree(rng, n_rows, vocab):
    """Random valid tree: parents[i] < i, sibling tokens distinct."""
    parents = [-1] + [int(rng.integers(0, i)) for i in range(1, n_rows)]
    tokens = [int(rng.integers(vocab))]
    for i in range(1, n_rows):
        taken = {tokens[c] for c in range(i) if parents[c] == parents[i]}
        t = int(rng.integers(vocab))
        while t in taken:
            t = int(rng.integers(vocab))
        tokens.append(t)
    return tokens, parents


def to_dev(a, dtype=torch.int32):
    return torch.as_tensor(np.asarray(a), device="cuda").to(dtype)


def dev_weight_np(seed, name, shape, dtype="bf16", sigma=0.02, rows=None):
    """A seeded weight generated on the device exactly as the engine generates it,
    returned as float64 numpy (optionally only the given rows)."""
    from speculative_decoding_step_amd import synth
    t = synth.normal_t(seed, name, shape, "cuda", sigma, dtype)
    if rows is not None:
        t = t[torch.as_tensor(np.asarray(rows, dtype=np.int64), device="cuda")]
    out = t.to(torch.float64).cpu().numpy()
    del t
    return out


class LazyLayers:
    """W["layers"] for the oracle at the 8B shape: layer l's float64 weights are made
    on first access (seeded on the device, as the engine makes them) and the previous
    layer's are dropped, so a full-depth oracle pass holds one layer at a time."""

    def __init__(self, ms, seed, log=None):
        self.ms, self.seed, self.log = ms, seed, log
        self.cur, self.layer = -1, None

    def __len__(self):
        return self.ms.n_layers

    def __getitem__(self, l):
        if l != self.cur:
            ms = self.ms
            d, qd, kvd = ms.d, ms.n_heads * ms.head_dim, ms.n_kv_heads * ms.head_dim
            self.layer = None
            L = {"attn_norm": np.ones(d), "ffn_norm": np.ones(d)}
            for key, shape in [("wq", (qd, d)), ("wk", (kvd, d)), ("wv", (kvd, d)), ("wo", (d, qd)),
                               ("w_gate", (ms.ffn, d)), ("w_up", (ms.ffn, d)), ("w_down", (d, ms.ffn))]:
                L[key] = dev_weight_np(self.seed, f"l{l}.{key}", shape, ms.dtype)
            self.layer, self.cur = L, l
            if self.log:
                self.log(l)
        return self.layer
