"""The bf16 draft stage against the oracle, element by element.

The draft head ("EAGLE-3: Engineering Implementation of LLM Inference
Acceleration", IX.5 fusion FC, VIII.1 decoder layer, VIII.5-VIII.6 LM head)
runs on the bf16 MFMA kernels: the FC GEMM over [l ; m ; h], the 2d-input
QKV GEMM, the draft-mode tree-masked attention (speculative draft K/V seen
by descendants only), the o / gate-up / down GEMMs and the full-vocabulary
LM-head GEMM.  Its logits table (root row + every expansion row) is compared
with the oracle's at the bf16 bar, 2e-2 absolute, over the same frontiers;
the tree must be exactly the one the oracle's builder makes from the GPU's
own logits (integer parity given equal logits), and, where the seed's
decisions clear the measured logits error (asserted for the toy seed), the
one the oracle makes from its own logits.
"""
import dataclasses

import numpy as np
import pytest
import torch

from gpu_util import LazyLayers, dev_weight_np, make_engine, oracle_weights, toy_shape
from oracle.llama import Shape, draft_fuse, draft_layer, draft_logits
from oracle.numerics import topk_desc
from oracle.step import OracleSequence, SpecConfig, f32
from oracle.tree import build_dynamic_tree, tree_from_table
from speculative_decoding_step_amd import configs, synth
from speculative_decoding_step_amd.engine import Engine, Spec

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _clearance(tree, rows, k, D, eps):
    """True when every decision the tree takes clears an error of eps per logit:
    adjacent gaps among each row's top k+1 logits exceed 2 eps, and adjacent gaps
    among the kept nodes' cumulative scores exceed 4 D eps (a score at depth d
    moves by at most 2 d eps: the logit and the log-sum-exp each by eps)."""
    lg = min(float(np.min(-np.diff(np.sort(r)[::-1][:k + 1]))) for r in rows)
    sc = np.sort(np.array(tree.score[1:], dtype=np.float64))
    sg = float(np.min(np.diff(sc))) if len(sc) > 1 else np.inf
    return lg > 2 * eps and sg > 4 * D * eps, lg, sg


def _check_ranked(picks, ref, k, tol):
    """The GPU's ranked top-k picks against the oracle's row: rank i must be the
    oracle's rank-i token wherever that token's value is more than 2 tol from its
    neighbours in the oracle's order; elsewhere (a tie within the tolerance) the
    pick's oracle value must be within 2 tol of the oracle's rank-i value, and
    picks are distinct.  Returns the number of ranks checked exactly."""
    order = [int(t) for t in topk_desc(ref, k + 1)]
    vals = ref[order]
    assert len(set(picks)) == len(picks)
    strict = 0
    for i, t in enumerate(picks):
        lo = vals[i] - vals[i + 1]
        hi = vals[i - 1] - vals[i] if i > 0 else np.inf
        if min(lo, hi) > 2 * tol:
            assert t == order[i], (i, t, order[i])
            strict += 1
        else:
            assert abs(ref[t] - vals[i]) <= 2 * tol, (i, t, ref[t], vals[i])
    return strict


@pytest.mark.parametrize("dv,seed", [(0, 39), (3000, 41)])
def test_draft_stage_bf16_mfma_matches_oracle(dv, seed):
    """Toy bf16 model on the MFMA kernels (d 256, 4x64 heads over 2 KV heads, FFN
    512, vocabulary 10,240 so the draft LM head takes the wide 16-row GEMM): the
    whole draft stage after a 40-token prefill, depth 4, top-3, 10 nodes.  The
    oracle starts from the GPU prefill's outputs (tap row, root, committed draft
    K/V), so the comparison covers exactly the draft stage: catch-up (fusion FC,
    decoder layer), every expansion (speculative draft K/V seen by descendants
    only) and the LM head.  dv > 0: the draft's own head over a reduced vocabulary
    of dv ids (a partial last 128-id slice), its rows over draft ids and the tree's
    tokens mapped through d2t ("EAGLE-3: Engineering Implementation of LLM
    Inference Acceleration", VIII.5-VIII.6)."""
    ms = toy_shape(dtype="bf16", vocab=10240, layers=2)
    if dv:
        ms = dataclasses.replace(ms, draft_vocab=dv)
    D, k, N, P = 4, 3, 10, 40
    spec = Spec("greedy_tree", D, k, N)
    shp, W, H = oracle_weights(ms, seed=seed, sigma=0.07)
    prompt = synth.tokens_np(42, "p", P, ms.vocab)
    eng = make_engine(ms, spec, max_seq=128, seed=seed, sigma=0.07)
    eng.prefill([prompt])
    # the draft stage's inputs as the GPU's prefill left them: the tap row of position P - 1, the root and
    # the committed draft K/V of positions [0, P - 1)
    aux_row = eng.aux_new[0, :1].to(torch.float64).cpu().numpy()
    root = int(eng.next_tok[0, 0])
    dkv = eng.kv_logical("draft")[0, :, 0, :, :P - 1].to(torch.float64).cpu().numpy()
    eng.record_draft_logits()
    eng.draft()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    table = eng.draft_table[0].cpu().numpy()
    g_tok, g_par = list(eng.tokens[0].cpu().numpy()), list(eng.parents[0].cpu().numpy())
    g_score = eng.score[0].cpu().numpy()
    eng.close()

    seq = OracleSequence(W, H, shp, SpecConfig("greedy_tree", D, k, N), 128)
    seq.cache.length = P
    seq.root, seq.aux_new, seq.next_tok = root, aux_row, [root]
    seq.dcache.k[0][:P - 1] = dkv[0].transpose(1, 0, 2)
    seq.dcache.v[0][:P - 1] = dkv[1].transpose(1, 0, 2)
    seq.dcache.length = P - 1

    # (1) integer parity given equal logits: the tree the GPU's own logits table implies (the oracle's builder
    #     over the table) is the GPU's tree; it also names the frontier of every expansion
    frontiers = []
    nxt = [1]

    def from_table(d, info):
        frontiers.append(info)
        out = [table[nxt[0] + i] for i in range(len(info))]
        nxt[0] += len(info)
        return out

    d2t = H.get("d2t")
    implied = build_dynamic_tree(root, table[0], from_table, D, k, N, d2t)
    assert g_tok == implied.tokens and g_par == implied.parents
    assert np.array_equal(g_score, np.array(implied.score, dtype=np.float32))

    # (2) logits parity: the oracle's draft stage over the same frontiers (catch-up, then each expansion with the
    #     ancestors' speculative K/V it computed itself), row by row against the GPU's table
    a_last = seq.draft_catchup()
    rows = [f32(draft_logits(H, W, shp, a_last))]
    expand = seq._expander(a_last)
    for d, info in enumerate(frontiers):
        rows.extend(expand(d + 1, info))
    assert len(rows) == 1 + (D - 1) * k == table.shape[0]
    errs = [float(np.abs(table[r].astype(np.float64) - rows[r]).max()) for r in range(len(rows))]
    eps = max(errs)

    # (3) the oracle's own tree from its own logits: equal to the GPU's when the seed's decisions clear the
    #     measured error (asserted, so the seed is not near a tie)
    own = tree_from_table(root, np.stack(rows), D, k, N, d2t)
    ok, lg, sg = _clearance(own, rows, k, D, eps)
    print(f"\n  draft logits max err per row {np.round(errs, 5).tolist()}; decision gaps: logits {lg:.4f}, "
          f"scores {sg:.4f}", flush=True)
    assert eps <= BF16_TOL
    assert ok, "seed too close to a tie for the measured error"
    assert own.tokens == g_tok and own.parents == g_par


def test_8b_draft_catchup_and_first_expansion_vs_oracle():
    """8B shape (config 3): after the 2048-token prefill, the draft's catch-up row
    (FC 12288 -> 4096 over the GPU's tap row, the decoder layer over the GPU's
    committed draft K/V) and its first expansion (10 rows at draft position P) are
    recomputed by the oracle from the GPU's inputs; the root row and the ten
    expansion rows of draft logits over all 128,256 ids agree within 2e-2, the
    depth-1 tokens are the oracle's top-10 and the depth-2 children of each
    expanded node its row's top-ranked tokens (exactly where the oracle's
    neighbouring logits are more than twice the tolerance apart, within the
    tolerance of the oracle's value where they are not: random weights give
    nearly flat draft distributions with many near-ties)."""
    w = configs.WORKLOADS["llama8b_tree_b1"]
    ms, D, k = w.shape, w.depth, w.topk
    d, P = ms.d, w.prompt_len
    prompt = configs.prompts_np(w)[0]
    print(f"\n[8B draft parity] P={P}", flush=True)
    eng = Engine(ms, Spec.of(w), 1, P + 256, w.target_seed, w.head_seed, prefill_chunk=512)
    eng.prefill([prompt])
    torch.cuda.synchronize()
    aux_row = eng.aux_new[0, 0].to(torch.float64).cpu().numpy()
    root = int(eng.next_tok[0, 0])
    dkv = eng.kv_logical("draft")[0, :, 0, :, :P - 1].to(torch.float64).cpu().numpy()   # [2, Hkv, P-1, hd]
    eng.record_draft_logits()
    eng.draft()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    table = eng.draft_table[0, :1 + k].cpu().numpy()
    g_tok, g_par = eng.tokens[0].cpu().numpy(), eng.parents[0].cpu().numpy()
    g_dep = eng.depth[0].cpu().numpy()
    eng.close()
    del eng
    torch.cuda.empty_cache()
    print("  GPU draft done; building the oracle's head weights", flush=True)

    hs = w.head_seed
    qd, kvd = ms.n_heads * ms.head_dim, ms.n_kv_heads * ms.head_dim
    H = {"input_norm": np.ones(d), "hidden_norm": np.ones(d), "post_norm": np.ones(d), "final_norm": np.ones(d)}
    for key, shape in [("fc", (d, 3 * d)), ("wq", (qd, 2 * d)), ("wk", (kvd, 2 * d)), ("wv", (kvd, 2 * d)),
                       ("wo", (d, qd)), ("w_gate", (ms.ffn, d)), ("w_up", (ms.ffn, d)), ("w_down", (d, ms.ffn))]:
        H[key] = dev_weight_np(hs, "h." + key, shape)
    # depth-1 tokens come from the root row; embedding rows are remapped to the ones used
    d1 = [int(t) for t in g_tok[1:][g_dep[1:] == 1]]
    used = sorted(set([root] + d1))
    remap = {t: i for i, t in enumerate(used)}
    W = {"embed": dev_weight_np(w.target_seed, "embed", (ms.vocab, d), rows=used),
         "lm_head": dev_weight_np(w.target_seed, "lm_head", (ms.vocab, d))}
    shp = Shape(1, d, ms.n_heads, ms.n_kv_heads, ms.head_dim, ms.ffn, ms.vocab, ms.rope_theta, ms.eps, "bf16",
                ms.taps)
    ck, cv = dkv[0].transpose(1, 0, 2), dkv[1].transpose(1, 0, 2)             # [P-1, Hkv, hd]

    # catch-up row at position P - 1: g from the GPU's tap row, paired with the root's embedding
    g = draft_fuse(H, aux_row[None])
    a_last, k_new, v_new = draft_layer(H, W, shp, [remap[root]], g, np.array([P - 1]),
                                       lambda i, kk, vv: (np.concatenate([ck, kk[:1]]), np.concatenate([cv, vv[:1]])))
    root_logits = f32(draft_logits(H, W, shp, a_last))[0]
    err0 = float(np.abs(table[0].astype(np.float64) - root_logits).max())
    print(f"  root row: max err {err0:.4g}", flush=True)
    assert err0 <= BF16_TOL
    strict0 = _check_ranked(d1, root_logits, k, BF16_TOL)

    # first expansion: the k depth-1 nodes (score order = top-k order) at draft position P, each
    # over the committed draft K/V [0, P) and its own entry
    ck2, cv2 = np.concatenate([ck, k_new]), np.concatenate([cv, v_new])
    xs = np.repeat(a_last, k, axis=0)
    a_rows, _, _ = draft_layer(H, W, shp, [remap[t] for t in d1], xs, np.full(k, P),
                               lambda i, kk, vv: (np.concatenate([ck2, kk[i:i + 1]]),
                                                  np.concatenate([cv2, vv[i:i + 1]])))
    errs, strict = [], strict0
    for i in range(k):
        ref = f32(draft_logits(H, W, shp, a_rows[i:i + 1]))[0]
        errs.append(float(np.abs(table[1 + i].astype(np.float64) - ref).max()))
        # the children of depth-1 node i that survived the final top-N are a prefix of its row's top-k
        kids = [int(g_tok[c]) for c in range(len(g_tok)) if g_par[c] == 1 + i]
        strict += _check_ranked(kids, ref, len(kids), BF16_TOL)
    print(f"  expansion rows: max err {np.round(errs, 4).tolist()}; {strict} ranked picks matched exactly "
          f"(the rest are within the tolerance of a tie)", flush=True)
    assert max(errs) <= BF16_TOL
    assert strict >= k
