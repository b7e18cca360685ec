"""Full-depth verify parity at the 8B shape: every layer and the LM head.

"Advanced speculative decoding: tree drafts and EAGLE", Implementation: one
target pass over the tree rows, each seeing the committed prefix, its
ancestors and itself at position prefix + depth, gives every node the logits
of the path that leads to it.  The GPU's verify call records the fp32
residual stream entering each of the 32 layers and leaving the last
(eagle3_set_hidden_out); the oracle then recomputes every layer from the
GPU's stream entering it (float64, the same bf16 rounding points, the GPU's
committed prefix K/V) and the 128,256-id LM head from the GPU's final stream.
Bars: each layer's output within 1e-2 of its largest magnitude, the tree
rows' K/V likewise, and the logits within 2e-2 absolute with the argmax
wherever the oracle's top-2 margin exceeds twice that.

The same loop also runs the oracle free from the GPU's stream (its own
32-layer pass over the tree rows) and reports how far its logits drift from
the GPU's: bf16 rounding points turn fp32-vs-float64 summation differences
into one-ulp flips of single activations, and 32 layers compound them, so the
free-running distance is a measurement, bounded here only loosely.
"""
import numpy as np
import pytest
import torch

from gpu_util import LazyLayers, dev_weight_np, kv_view
from oracle.llama import Shape, target_layer, target_logits
from oracle.tree import tree_mask
from speculative_decoding_step_amd import binding as B
from speculative_decoding_step_amd import configs
from speculative_decoding_step_amd.engine import Engine, Spec

pytestmark = pytest.mark.gpu

TOL = 2e-2          # bf16 logits bar
HID_REL = 1e-2      # per-layer hidden-state / K/V bar, relative to the largest magnitude
FREE_BOUND = 0.5    # loose sanity bound on the free-running 32-layer drift


def check_logits(g, ref, what, tol=TOL):
    """The bf16 logits bar; returns (max error, rows whose argmax was checked)."""
    err = float(np.abs(np.asarray(g, dtype=np.float64) - ref).max())
    assert err <= tol, (what, err)
    checked = 0
    for i in range(ref.shape[0]):
        s = np.sort(ref[i])
        if s[-1] - s[-2] > 2 * tol:
            assert int(np.argmax(g[i])) == int(np.argmax(ref[i])), (what, i)
            checked += 1
    return err, checked


def per_layer_parity(ms, seed, kv_prefix, hid, tree_kv, tokens, parents, P, g_logits, what):
    """Teacher-forced per-layer parity of one sequence's tree rows (see the module doc).

    kv_prefix: float64 [L, 2, Hkv, P, hd]; hid: float32 [L + 1, n, d] (GPU);
    tree_kv: float32 [L, 2, Hkv, n, hd] (the GPU's K/V of the tree rows);
    g_logits [n, V] (GPU).  Returns a dict of the measured errors."""
    d, n, L = ms.d, len(tokens), ms.n_layers
    shp = Shape(L, d, ms.n_heads, ms.n_kv_heads, ms.head_dim, ms.ffn, ms.vocab, ms.rope_theta, ms.eps, "bf16",
                ms.taps)
    emb = dev_weight_np(seed, "embed", (ms.vocab, d), rows=[int(t) for t in tokens])
    assert np.array_equal(hid[0].astype(np.float64), emb), (what, "embedding rows")
    dep = [0] * n
    for i in range(1, n):
        dep[i] = dep[parents[i]] + 1
    pos = P + np.array(dep)
    m = tree_mask(parents)
    vis = [list(np.nonzero(m[i])[0]) for i in range(n)]
    layers = LazyLayers(ms, seed)
    x_free = emb.copy()
    worst_h, worst_kv = 0.0, 0.0
    for l in range(L):
        Lw = layers[l]
        pk, pv = kv_prefix[l, 0].transpose(1, 0, 2), kv_prefix[l, 1].transpose(1, 0, 2)
        ref, k, v = target_layer(Lw, shp, hid[l].astype(np.float64), pk, pv, pos, vis)
        err = float(np.abs(hid[l + 1] - ref).max())
        scale = float(np.abs(ref).max())
        assert err <= HID_REL * scale, (what, "layer", l, err, scale)
        worst_h = max(worst_h, err / scale)
        for which, r in ((0, k), (1, v)):
            gk = tree_kv[l, which].transpose(1, 0, 2)                   # [n, Hkv, hd]
            e = float(np.abs(gk - r).max())
            assert e <= HID_REL * float(np.abs(r).max()), (what, "tree K/V", l, which, e)
            worst_kv = max(worst_kv, e / float(np.abs(r).max()))
        x_free, _, _ = target_layer(Lw, shp, x_free, pk, pv, pos, vis)
        if l % 8 == 7:
            print(f"    layer {l}: hidden err {err:.3g} (scale {scale:.3g})", flush=True)
    W = {"final_norm": np.ones(d), "lm_head": dev_weight_np(seed, "lm_head", (ms.vocab, d))}
    ref_logits = target_logits(W, shp, hid[L].astype(np.float64))
    err, checked = check_logits(g_logits, ref_logits, (what, "LM head"))
    free = target_logits(W, shp, x_free)
    free_err = float(np.abs(g_logits - free).max())
    free_rms = float(np.sqrt(np.mean((g_logits - free) ** 2)))
    agree = float(np.mean(np.argmax(g_logits, 1) == np.argmax(free, 1)))
    print(f"  {what}: per-layer hidden err <= {worst_h:.3g} x scale, tree K/V <= {worst_kv:.3g} x scale; "
          f"logits err {err:.4g} (argmax checked on {checked}/{n} rows); free-running 32-layer drift: max "
          f"{free_err:.4g}, rms {free_rms:.3g}, argmax agreement {agree:.3f}", flush=True)
    assert free_err <= FREE_BOUND, (what, "free-running drift", free_err)
    return dict(hidden=worst_h, kv=worst_kv, logits=err, checked=checked, free_max=free_err, free_rms=free_rms)


def test_8b_tree_verify_every_layer_and_logits():
    """Config 3 (batch 1, prompt 2048): the drafted 61-row tree through all 32 layers
    and the LM head (the 64-row weight-streaming GEMMs, 128,256 rows)."""
    w = configs.WORKLOADS["llama8b_tree_b1"]
    ms, P, n = w.shape, w.prompt_len, w.rows
    prompt = configs.prompts_np(w)[0]
    print(f"\n[8B verify, every layer] P={P} rows={n}", flush=True)
    eng = Engine(ms, Spec.of(w), 1, P + 256, w.target_seed, w.head_seed, prefill_chunk=512)
    eng.prefill([prompt])
    eng.draft()
    logits = torch.zeros(n, ms.vocab, dtype=torch.float32, device="cuda")
    hid = torch.zeros(ms.n_layers + 1, n, ms.d, dtype=torch.float32, device="cuda")
    B.eagle3_set_hidden_out(eng.ctx, hid.data_ptr())
    B.eagle3_verify_tree(eng.ctx, 0, 1, eng.seq_lens.data_ptr(), n, eng.tokens.data_ptr(), eng.pos.data_ptr(),
                         eng.mask.data_ptr(), B.LM_ALL, logits.data_ptr(), None, None, None)
    B.eagle3_set_hidden_out(eng.ctx, None)
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    g = logits.cpu().numpy()
    h = hid.cpu().numpy()
    tokens, parents = eng.tokens[0].cpu().numpy(), [int(x) for x in eng.parents[0].cpu().numpy()]
    kv = kv_view(eng)
    kvp = kv[:, :, 0, :, :P].to(torch.float64).cpu().numpy()          # [L, 2, Hkv, P, hd]
    tkv = kv[:, :, 0, :, P:P + n].float().cpu().numpy()               # [L, 2, Hkv, n, hd]
    eng.close()
    del eng, logits, hid, kv
    torch.cuda.empty_cache()
    per_layer_parity(ms, w.target_seed, kvp, h, tkv, tokens, parents, P, g, "batch-1 tree")
