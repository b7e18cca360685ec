"""GPU parity of each C-ABI call against the oracle on the same seeded inputs.

Integer and index work (trees, masks, paths, samples, compaction) must match
bit for bit given equal float inputs; logits within 2e-2 absolute (bf16) or
1e-4 relative (fp32); argmax wherever the oracle's top-2 margin exceeds that.
"""
import dataclasses
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import (kv_view, logits_close, make_engine, margin_tol, oracle_weights, random_tree, to_dev,
                      toy_shape, top2_margin)
from oracle.accept import chain_rejection, greedy_walk, tree_rejection
from oracle.step import compaction_moves
from oracle.llama import KVCache, causal_visible, target_forward
from oracle.numerics import probs_f32, sample_inverse_cdf
from oracle.step import build_sampled_chain
from oracle.tree import mask_words, tree_from_table, tree_mask
from speculative_decoding_step_amd import binding as B
from speculative_decoding_step_amd import configs
from speculative_decoding_step_amd import synth
from speculative_decoding_step_amd.engine import Spec

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _p(t):
    return None if t is None else t.data_ptr()


def _status_clear(eng):
    assert eng.device_status() == 0


# ------------------------------------------------------------------ verify_tree
@pytest.mark.parametrize("dtype,chunk", [("f32", 24), ("bf16", 24), ("bf16", 96)])
def test_verify_prefill_and_tree_vs_oracle(dtype, chunk):
    """Prefill in chunks (a 96-row chunk takes the large-M GEMM), then a tree verify."""
    print(f"\n[verify parity {dtype} chunk {chunk}]", flush=True)
    ms = toy_shape(dtype=dtype, vocab=1000)
    spec = Spec("greedy_tree", 4, 3, 12)
    eng = make_engine(ms, spec, max_seq=160, sigma=0.05, prefill_chunk=chunk)
    shp, W, H = oracle_weights(ms, sigma=0.05)
    P = 50 if chunk < 64 else 110
    prompt = synth.tokens_np(31, "p", P, ms.vocab)
    eng.prefill([prompt])
    torch.cuda.synchronize()
    _status_clear(eng)
    # oracle prefill
    cache = KVCache(shp.n_layers, 160, shp.n_kv_heads, shp.head_dim)
    lg, k, v, aux = target_forward(W, shp, cache, prompt, np.arange(P), causal_visible(P))
    for l in range(shp.n_layers):
        cache.k[l][:P], cache.v[l][:P] = k[l], v[l]
    cache.length = P
    kvg = kv_view(eng)[:, :, 0, :, :P].float().cpu().numpy()      # [L, 2, Hkv, P, hd]
    for l in range(shp.n_layers):
        err_k = np.abs(kvg[l, 0].transpose(1, 0, 2) - k[l]).max()
        err_v = np.abs(kvg[l, 1].transpose(1, 0, 2) - v[l]).max()
        assert err_k < (2e-2 if dtype == "bf16" else 1e-4) and err_v < (2e-2 if dtype == "bf16" else 1e-4)
    # the prefill's last-position aux (what the catch-up consumes)
    aux_g = eng.aux_new[0, 0].float().cpu().numpy()
    assert np.abs(aux_g - aux[-1]).max() < (2e-2 if dtype == "bf16" else 1e-4)
    # tree verify at P
    rng = np.random.default_rng(5)
    n = 13
    tokens, parents = random_tree(rng, n, ms.vocab)
    dep = [0] * n
    for i in range(1, n):
        dep[i] = dep[parents[i]] + 1
    m = tree_mask(parents)
    ref, rk, rv, raux = target_forward(W, shp, cache, tokens, P + np.array(dep),
                                       [list(np.nonzero(m[i])[0]) for i in range(n)])
    seq_lens = to_dev([P])
    logits = torch.zeros(n, ms.vocab, dtype=torch.float32, device="cuda")
    am = torch.zeros(n, dtype=torch.int32, device="cuda")
    mg = torch.zeros(n, dtype=torch.float32, device="cuda")
    auxo = torch.zeros(n, 3 * ms.d, dtype=eng.tdt, device="cuda")
    mw = torch.as_tensor(mask_words(parents).view(np.int64), device="cuda")
    tok_d, pos_d = to_dev(tokens), to_dev(P + np.array(dep))
    B.eagle3_verify_tree(eng.ctx, 0, 1, _p(seq_lens), n, _p(tok_d), _p(pos_d), _p(mw),
                         B.LM_ALL, _p(logits), _p(am), _p(mg), _p(auxo))
    torch.cuda.synchronize()
    _status_clear(eng)
    g = logits.cpu().numpy()
    err, ok = logits_close(g, ref, dtype)
    print(f"  tree logits err {err:.3g}", flush=True)
    assert ok
    amg = am.cpu().numpy()
    for i in range(n):
        if top2_margin(ref[i]) > 2 * margin_tol(dtype, ref[i]):
            assert amg[i] == int(np.argmax(ref[i]))
    assert np.abs(auxo.float().cpu().numpy() - raux).max() < (2e-2 if dtype == "bf16" else 1e-4)
    kvt = kv_view(eng)[:, :, 0, :, P:P + n].float().cpu().numpy()
    for l in range(shp.n_layers):
        assert np.abs(kvt[l, 0].transpose(1, 0, 2) - rk[l]).max() < (2e-2 if dtype == "bf16" else 1e-4)
    eng.close()


def test_batched_ragged_tree_verify_vs_oracle():
    """40 ragged prompts (60..1000 tokens) at head size 128: the verify attention launch has
    40 sequences x 4 KV heads x 4 key chunks = 640 work items, the size that takes the
    two-stage ring with two workgroups per CU.  Every sequence gets its own random tree;
    the shortest, a middle and the longest sequence are checked against the oracle.
    Weights at sigma 0.02 keep the logits near 2 in magnitude, as in the other cases: at
    d 512 and sigma 0.05 they reach 5.6, where the bf16 rounding of the final hidden state
    alone is about 0.02 (2^-8 relative)."""
    ms = toy_shape(dtype="bf16", vocab=1000, layers=2, d=512, heads=4, kv=4, hd=128, ffn=512)
    spec = Spec("greedy_tree", 4, 3, 12)
    Bn, n = 40, 13
    lens = np.linspace(60, 1000, Bn).astype(int)
    assert Bn * ms.n_kv_heads * -(-(int(lens.max()) + n) // 256) >= 512
    print(f"\n[batched ragged verify, {Bn} sequences, {lens.min()}..{lens.max()} tokens]", flush=True)
    eng = make_engine(ms, spec, batch=Bn, max_seq=1100, sigma=0.02)
    shp, W, H = oracle_weights(ms, sigma=0.02)
    prompts = [synth.tokens_np(41, f"r{b}", int(lens[b]), ms.vocab) for b in range(Bn)]
    eng.prefill(prompts)
    torch.cuda.synchronize()
    _status_clear(eng)
    rng = np.random.default_rng(9)
    trees = [random_tree(rng, n, ms.vocab) for _ in range(Bn)]
    deps = []
    for tokens, parents in trees:
        dep = [0] * n
        for i in range(1, n):
            dep[i] = dep[parents[i]] + 1
        deps.append(np.array(dep))
    tok_d = to_dev(np.concatenate([t for t, _ in trees]))
    pos_d = to_dev(np.concatenate([lens[b] + deps[b] for b in range(Bn)]))
    mw = torch.as_tensor(np.concatenate([mask_words(p) for _, p in trees]).view(np.int64), device="cuda")
    seq_lens = to_dev(lens)
    logits = torch.zeros(Bn * n, ms.vocab, dtype=torch.float32, device="cuda")
    am = torch.zeros(Bn * n, dtype=torch.int32, device="cuda")
    mg = torch.zeros(Bn * n, dtype=torch.float32, device="cuda")
    auxo = torch.zeros(Bn * n, 3 * ms.d, dtype=eng.tdt, device="cuda")
    B.eagle3_verify_tree(eng.ctx, 0, Bn, _p(seq_lens), n, _p(tok_d), _p(pos_d), _p(mw),
                         B.LM_ALL, _p(logits), _p(am), _p(mg), _p(auxo))
    torch.cuda.synchronize()
    _status_clear(eng)
    g_all, am_all = logits.cpu().numpy().reshape(Bn, n, -1), am.cpu().numpy().reshape(Bn, n)
    eng.close()
    for b in (0, Bn // 2, Bn - 1):
        P = int(lens[b])
        cache = KVCache(shp.n_layers, 1100, shp.n_kv_heads, shp.head_dim)
        _, k, v, _ = target_forward(W, shp, cache, prompts[b], np.arange(P), causal_visible(P))
        for l in range(shp.n_layers):
            cache.k[l][:P], cache.v[l][:P] = k[l], v[l]
        cache.length = P
        tokens, parents = trees[b]
        m = tree_mask(parents)
        ref, _, _, _ = target_forward(W, shp, cache, tokens, P + deps[b],
                                      [list(np.nonzero(m[i])[0]) for i in range(n)])
        err, ok = logits_close(g_all[b], ref, "bf16")
        print(f"  seq {b} (P={P}): tree logits err {err:.3g}", flush=True)
        assert ok
        for i in range(n):
            if top2_margin(ref[i]) > 2 * margin_tol("bf16", ref[i]):
                assert am_all[b, i] == int(np.argmax(ref[i]))


# ------------------------------------------------------------- tree from logits
def _tree_engine(D, k, N, V, mode="greedy_tree", T=0.0, batch=1, draft_greedy=False, dv=0):
    ms = toy_shape(dtype="bf16", vocab=V, layers=1, d=256, heads=4, kv=4, hd=64, ffn=256, taps=(0, 0, 0))
    if dv:
        ms = dataclasses.replace(ms, draft_vocab=dv)
    return make_engine(ms, Spec(mode, D, k, N, T, draft_greedy), batch=batch, max_seq=128)


def _run_tree_from_logits(eng, roots, table, uniforms=None):
    Bn = len(roots)
    R = eng.rows
    outs = dict(tokens=torch.zeros(Bn, R, dtype=torch.int32, device="cuda"),
                parents=torch.zeros(Bn, R, dtype=torch.int32, device="cuda"),
                depth=torch.zeros(Bn, R, dtype=torch.int32, device="cuda"),
                pos=torch.zeros(Bn, R, dtype=torch.int32, device="cuda"),
                mask=torch.zeros(Bn, R, dtype=torch.int64, device="cuda"),
                score=torch.zeros(Bn, R, dtype=torch.float32, device="cuda"))
    q = torch.zeros(Bn, eng.spec.depth, eng.ms.vocab, dtype=torch.float32, device="cuda") if eng.sampling else None
    seq_lens = to_dev([40 + b for b in range(Bn)])
    tab = torch.as_tensor(np.ascontiguousarray(table, dtype=np.float32), device="cuda")
    u = None if uniforms is None else torch.as_tensor(uniforms, device="cuda")
    roots_d = to_dev(roots)
    B.eagle3_tree_from_logits(eng.ctx, Bn, _p(roots_d), _p(seq_lens), _p(tab), _p(u), _p(outs["tokens"]),
                              _p(outs["parents"]), _p(outs["depth"]), _p(outs["pos"]), _p(outs["mask"]),
                              _p(outs["score"]), _p(q))
    torch.cuda.synchronize()
    _status_clear(eng)
    res = {k: v.cpu().numpy() for k, v in outs.items()}
    if q is not None:
        res["q"] = q.cpu().numpy()
    return res


def test_tree_from_logits_hand_worked_golden():
    g = json.load(open(os.path.join(GOLDEN, "dynamic_tree_hand.json")))
    table = np.log(np.array(g["probs"], dtype=np.float64)).astype(np.float32)
    for n, exp in g["expect"].items():
        eng = _tree_engine(g["depth"], g["topk"], int(n), table.shape[1])
        r = _run_tree_from_logits(eng, [g["root"]], table[None])
        assert list(r["tokens"][0]) == exp["tokens"]
        assert list(r["parents"][0]) == exp["parents"]
        assert list(r["depth"][0]) == exp["depth"]
        assert list(r["pos"][0]) == [40 + x for x in exp["depth"]]
        assert [int(x) for x in r["mask"][0].view(np.uint64)] == [int(x) for x in mask_words(exp["parents"])]
        eng.close()


@pytest.mark.parametrize("D,k,N,V,Bn", [(6, 4, 32, 32000, 2), (6, 10, 60, 128256, 1), (4, 4, 16, 5000, 3),
                                        (4, 1, 4, 1024, 2), (3, 2, 5, 7, 4),
                                        # degenerate shapes: one level, a single node, one node per level
                                        (1, 5, 5, 300, 2), (2, 3, 1, 50, 1), (1, 1, 1, 16, 3), (6, 1, 6, 90, 2),
                                        # the largest vocabulary and top-k the library takes (64 slices of 4096)
                                        (3, 16, 40, 262144, 1)])
def test_tree_from_logits_matches_oracle(D, k, N, V, Bn):
    print(f"\n[tree D{D} k{k} N{N} V{V} B{Bn}]", flush=True)
    rng = np.random.default_rng(D * 1000 + k * 100 + N)
    E = (D - 1) * k
    table = rng.normal(0, 3, size=(Bn, 1 + E, V)).astype(np.float32)
    if V > 64:  # plant exact ties in logits to exercise the tie rules
        table[:, :, 7] = table[:, :, 3]
    roots = list(rng.integers(0, V, Bn))
    eng = _tree_engine(D, k, N, V, batch=Bn)
    r = _run_tree_from_logits(eng, roots, table)
    for b in range(Bn):
        t = tree_from_table(int(roots[b]), table[b], D, k, N)
        assert list(r["tokens"][b]) == t.tokens
        assert list(r["parents"][b]) == t.parents
        assert list(r["depth"][b]) == t.depth
        assert list(r["pos"][b]) == [40 + b + x for x in t.depth]
        assert np.array_equal(r["score"][b], np.array(t.score, dtype=np.float32))
        assert [int(x) for x in r["mask"][b].view(np.uint64)] == [int(x) for x in mask_words(t.parents)]
    eng.close()


@pytest.mark.parametrize("greedy,V", [(False, 3000), (True, 3000), (False, 262144)])
def test_sampled_chain_from_logits_matches_oracle(greedy, V):
    K, Bn, T = 5, 4, 1.0
    rng = np.random.default_rng(17)
    table = rng.normal(0, 2, size=(Bn, K, V)).astype(np.float32)
    u = synth.uniform24_np(5, "ud", Bn * K).reshape(Bn, K)
    roots = list(rng.integers(0, V, Bn))
    eng = _tree_engine(K, 1, K, V, mode="sample_chain", T=T, batch=Bn, draft_greedy=greedy)
    r = _run_tree_from_logits(eng, roots, table, None if greedy else u)
    for b in range(Bn):
        cnt = [0]

        def expand(d, info):
            cnt[0] += 1
            return [table[b, cnt[0]]]

        toks, q = build_sampled_chain(int(roots[b]), table[b, 0], expand, K, T, u[b], greedy)
        assert list(r["tokens"][b]) == toks
        assert list(r["parents"][b]) == [-1, 0, 1, 2, 3, 4]
        np.testing.assert_allclose(r["q"][b], q, rtol=2e-7, atol=0)
    eng.close()


@pytest.mark.parametrize("D,k,N,V,Vd,Bn", [(6, 10, 60, 128256, 32000, 1), (4, 4, 16, 5000, 1234, 3)])
def test_tree_from_logits_reduced_vocab_matches_oracle(D, k, N, V, Vd, Bn):
    """Draft rows over a reduced draft vocabulary: top-k and scores in draft space,
    tokens mapped through d2t, bit-exact against the oracle."""
    print(f"\n[tree D{D} k{k} N{N} V{V} Vd{Vd} B{Bn}]", flush=True)
    rng = np.random.default_rng(Vd)
    E = (D - 1) * k
    table = rng.normal(0, 3, size=(Bn, 1 + E, Vd)).astype(np.float32)
    table[:, :, 9] = table[:, :, 4]  # exact ties
    roots = list(rng.integers(0, V, Bn))
    eng = _tree_engine(D, k, N, V, batch=Bn, dv=Vd)
    d2t = configs.d2t_np(eng.ms, 12)
    r = _run_tree_from_logits(eng, roots, table)
    assert eng.device_status() == 0
    for b in range(Bn):
        t = tree_from_table(int(roots[b]), table[b], D, k, N, d2t)
        assert list(r["tokens"][b]) == t.tokens
        assert list(r["parents"][b]) == t.parents
        assert np.array_equal(r["score"][b], np.array(t.score, dtype=np.float32))
    eng.close()


@pytest.mark.parametrize("greedy", [False, True])
def test_sampled_chain_reduced_vocab_matches_oracle(greedy):
    """Chains drawn over a reduced draft vocabulary: tokens are d2t of the draft-space
    draw and q is scattered into the target vocabulary, exactly as in the oracle."""
    K, V, Vd, Bn, T = 5, 3000, 701, 4, 1.0
    rng = np.random.default_rng(19)
    table = rng.normal(0, 2, size=(Bn, K, Vd)).astype(np.float32)
    u = synth.uniform24_np(6, "ud", Bn * K).reshape(Bn, K)
    roots = list(rng.integers(0, V, Bn))
    eng = _tree_engine(K, 1, K, V, mode="sample_chain", T=T, batch=Bn, draft_greedy=greedy, dv=Vd)
    d2t = configs.d2t_np(eng.ms, 12)
    r = _run_tree_from_logits(eng, roots, table, None if greedy else u)
    for b in range(Bn):
        cnt = [0]

        def expand(d, info):
            cnt[0] += 1
            return [table[b, cnt[0]]]

        toks, q = build_sampled_chain(int(roots[b]), table[b, 0], expand, K, T, u[b], greedy, d2t, V)
        assert list(r["tokens"][b]) == toks
        np.testing.assert_allclose(r["q"][b], q, rtol=2e-7, atol=0)
    eng.close()


# ------------------------------------------------------------------ accept
def test_accept_greedy_matches_walk():
    rng = np.random.default_rng(3)
    D, k, N, V, Bn = 6, 4, 32, 50, 8
    eng = _tree_engine(D, k, N, V, batch=Bn)
    n = N + 1
    toks, pars, am = [], [], []
    for b in range(Bn):
        # a planted branch: argmax follows it for a random length
        t, p = random_tree(rng, n, V)
        a = [int(x) for x in rng.integers(0, V, n)]
        node = 0
        for _ in range(int(rng.integers(0, D + 1))):
            kids = [c for c in range(n) if p[c] == node]
            if not kids:
                break
            c = kids[int(rng.integers(len(kids)))]
            a[node] = t[c]
            node = c
        toks.append(t)
        pars.append(p)
        am.append(a)
    maxp = D + 1
    path = torch.zeros(Bn, maxp, dtype=torch.int32, device="cuda")
    plen = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    em = torch.zeros(Bn, maxp, dtype=torch.int32, device="cuda")
    keep = [to_dev(toks), to_dev(pars), to_dev(am)]
    B.eagle3_accept(eng.ctx, Bn, n, _p(keep[0]), _p(keep[1]), _p(keep[2]), None, None, None, _p(path),
                    _p(plen), _p(nxt), _p(em))
    torch.cuda.synchronize()
    for b in range(Bn):
        ref_path, ref_next = greedy_walk(toks[b], pars[b], am[b])
        assert plen[b].item() == len(ref_path)
        assert list(path[b].cpu().numpy()) == ref_path + [-1] * (maxp - len(ref_path))
        assert nxt[b].item() == ref_next
        assert list(em[b].cpu().numpy()[:len(ref_path)]) == [toks[b][i] for i in ref_path]
    _status_clear(eng)
    eng.close()


def _chain_inputs(rng, Bn, K, V, T):
    logits = rng.normal(0, 1.5, size=(Bn, K + 1, V)).astype(np.float32)
    qlog = (logits[:, :K] + rng.normal(0, 1.0, size=(Bn, K, V))).astype(np.float32)
    q = np.stack([[probs_f32(qlog[b, i], T) for i in range(K)] for b in range(Bn)])
    u_d = rng.integers(0, 1 << 24, size=(Bn, K)) * 2.0 ** -24
    drafts = np.array([[sample_inverse_cdf(q[b, i], np.float32(u_d[b, i])) for i in range(K)] for b in range(Bn)])
    return logits, q, drafts


@pytest.mark.parametrize("V,Bn", [(4000, 16), (262144, 6)])
def test_accept_chain_matches_oracle(V, Bn):
    rng = np.random.default_rng(4)
    K, T = 5, 1.0
    eng = _tree_engine(K, 1, K, V, mode="sample_chain", T=T, batch=Bn)
    logits, q, drafts = _chain_inputs(rng, Bn, K, V, T)
    u = (rng.integers(0, 1 << 24, size=(Bn, K + 1)) * 2.0 ** -24).astype(np.float32)
    u[:, :K] *= 0.3  # bias toward accepting so several drafts pass
    toks = np.concatenate([rng.integers(0, V, (Bn, 1)), drafts], axis=1)
    path = torch.zeros(Bn, K + 1, dtype=torch.int32, device="cuda")
    plen = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    em = torch.zeros(Bn, K + 1, dtype=torch.int32, device="cuda")
    keep = [to_dev(toks), to_dev(logits, torch.float32), to_dev(q, torch.float32), to_dev(u, torch.float32)]
    B.eagle3_accept(eng.ctx, Bn, K + 1, _p(keep[0]), None, None, _p(keep[1]), _p(keep[2]), _p(keep[3]), _p(path),
                    _p(plen), _p(nxt), _p(em))
    torch.cuda.synchronize()
    seen = set()
    for b in range(Bn):
        p = np.stack([probs_f32(logits[b, i], T) for i in range(K + 1)])
        n_acc, tok = chain_rejection(toks[b, 1:], q[b], p, u[b])
        seen.add(n_acc)
        assert plen[b].item() == n_acc + 1
        assert nxt[b].item() == tok
        assert list(em[b].cpu().numpy()) == [int(x) for x in toks[b, :n_acc + 1]] + [-1] * (K - n_acc)
    assert len(seen) >= 2
    eng.close()


def _random_tree(rng, D, k, N, V):
    """Rows in (depth, creation) order: each level's nodes pick a parent on the previous
    level with fewer than k children; siblings hold distinct tokens."""
    tokens, parents, depth, kids = [int(rng.integers(0, V))], [-1], [0], [set()]
    level = [0]
    while len(tokens) < N + 1:
        d = depth[level[0]] + 1
        if d > D:
            break
        nxt = []
        slots = [(p, j) for p in level for j in range(k)]
        rng.shuffle(slots)
        for p, _ in slots[:min(len(slots), N + 1 - len(tokens))]:
            t = int(rng.integers(0, V))
            while t in kids[p]:
                t = int(rng.integers(0, V))
            kids[p].add(t)
            tokens.append(t)
            parents.append(p)
            depth.append(d)
            kids.append(set())
            nxt.append(len(tokens) - 1)
        level = nxt
    # renumber so that each level's rows follow their parents' order (children of one node stay in creation order)
    order = sorted(range(len(tokens)), key=lambda i: (depth[i], i))
    new = {o: i for i, o in enumerate(order)}
    return ([tokens[o] for o in order], [-1 if parents[o] < 0 else new[parents[o]] for o in order],
            [depth[o] for o in order])


@pytest.mark.parametrize("T,V,Bn,bump", [(1.0, 3000, 24, (2.0, 7.0)), (0.7, 3000, 24, (2.0, 7.0)),
                                         (1.0, 262144, 16, (10.0, 15.0))])
def test_accept_tree_matches_oracle(T, V, Bn, bump):
    """Level-by-level rejection sampling over trees: path, path length, next token and the
    emitted row equal the oracle's bit for bit on random trees, target rows that favour
    each node's candidates (so long paths occur) and seeded uniforms; also at the largest
    vocabulary (262,144 ids)."""
    rng = np.random.default_rng(11)
    D, k, N = 4, 3, 14
    eng = _tree_engine(D, k, N, V, mode="sample_tree", T=T, batch=Bn)
    R = N + 1
    toks = np.zeros((Bn, R), np.int32)
    pars = np.zeros((Bn, R), np.int32)
    trees = []
    for b in range(Bn):
        t, pa, _ = _random_tree(rng, D, k, N, V)
        assert len(t) == R
        toks[b], pars[b] = t, pa
        trees.append((t, pa))
    logits = rng.normal(0, 1.0, size=(Bn, R, V)).astype(np.float32)
    for b in range(Bn):
        for i in range(1, R):
            logits[b, pars[b, i], toks[b, i]] += rng.uniform(*bump)
    nu = D * k + 1
    u = (rng.integers(0, 1 << 24, size=(Bn, nu)) * 2.0 ** -24).astype(np.float32)
    maxp = D + 1
    path = torch.zeros(Bn, maxp, dtype=torch.int32, device="cuda")
    plen = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    nxt = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    em = torch.zeros(Bn, maxp, dtype=torch.int32, device="cuda")
    keep = [to_dev(toks), to_dev(pars), to_dev(logits, torch.float32), to_dev(u, torch.float32)]
    B.eagle3_accept(eng.ctx, Bn, R, _p(keep[0]), _p(keep[1]), None, _p(keep[2]), None, _p(keep[3]), _p(path),
                    _p(plen), _p(nxt), _p(em))
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    lens = set()
    for b in range(Bn):
        p = np.stack([probs_f32(logits[b, i], T) for i in range(R)])
        ref_path, ref_next = tree_rejection(trees[b][0], trees[b][1], p, u[b], k, D)
        lens.add(len(ref_path))
        assert plen[b].item() == len(ref_path)
        assert list(path[b].cpu().numpy()) == ref_path + [-1] * (maxp - len(ref_path))
        assert nxt[b].item() == ref_next
        assert list(em[b].cpu().numpy()) == [trees[b][0][i] for i in ref_path] + [-1] * (maxp - len(ref_path))
    assert len(lens) >= 3  # short and long walks both covered
    eng.close()


def test_accept_tree_flags_malformed_input():
    """A parent index not below its row, or a token outside the vocabulary, raises the
    context's status bits (the walk still ends and every lookup stays in range)."""
    D, k, N, V = 3, 2, 4, 500
    eng = _tree_engine(D, k, N, V, mode="sample_tree", T=1.0, batch=2)
    R = N + 1
    toks = np.array([[1, 2, 3, 4, 5], [1, 2, 3, V + 7, 5]], np.int32)
    pars = np.array([[-1, 0, 3, 0, 1], [-1, 0, 0, 1, 1]], np.int32)
    logits = np.zeros((2, R, V), np.float32)
    u = np.full((2, D * k + 1), 0.5, np.float32)
    maxp = D + 1
    outs = [torch.zeros(2, maxp, dtype=torch.int32, device="cuda"), torch.zeros(2, dtype=torch.int32, device="cuda"),
            torch.zeros(2, dtype=torch.int32, device="cuda"), torch.zeros(2, maxp, dtype=torch.int32, device="cuda")]
    keep = [to_dev(toks), to_dev(pars), to_dev(logits, torch.float32), to_dev(u, torch.float32)]
    B.eagle3_accept(eng.ctx, 2, R, _p(keep[0]), _p(keep[1]), None, _p(keep[2]), None, _p(keep[3]),
                    *[_p(t) for t in outs])
    torch.cuda.synchronize()
    flags = eng.device_status()
    assert flags & B.DEV_BAD_TREE and flags & B.DEV_BAD_TOKEN
    for b in range(2):
        n = outs[1][b].item()
        assert 1 <= n <= maxp and 0 <= outs[2][b].item() < V
    eng.close()


@pytest.mark.parametrize("dtype,T,S,Hq,Hkv,hd", [("bf16", 300, 3, 8, 2, 128), ("bf16", 1, 2, 4, 4, 64),
                                                ("bf16", 777, 7, 4, 1, 64), ("bf16", 513, 0, 8, 4, 128),
                                                ("f32", 129, 2, 4, 2, 96), ("f32", 40, 0, 2, 1, 32),
                                                ("bf16", 200, 20, 8, 2, 128), ("bf16", 2048, 7, 32, 8, 128)])
def test_ttt_attention_matches_oracle(dtype, T, S, Hq, Hkv, hd):
    """Training-time-test attention (causal native keys + diagonal simulated keys)
    against the oracle: every position for the small cases, sampled positions (first,
    last, chunk boundaries, random) at the 8B head layout with T = 2048, S = 7."""
    from oracle.ttt import ttt_attention
    print(f"\n[ttt {dtype} T{T} S{S} Hq{Hq} Hkv{Hkv} hd{hd}]", flush=True)
    rng = np.random.default_rng(T + 31 * S)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def dev(a):
        t = torch.as_tensor(a, dtype=torch.float32).to(tdt)
        return t.cuda(), t.float().numpy().astype(np.float64)  # device copy, and the stored values

    q, qn = dev(rng.normal(size=(T, Hq, hd)))
    k0, k0n = dev(rng.normal(size=(Hkv, T, hd)))
    v0, v0n = dev(rng.normal(size=(Hkv, T, hd)))
    ks, ksn = dev(rng.normal(size=(S, Hkv, T, hd)))
    vs, vsn = dev(rng.normal(size=(S, Hkv, T, hd)))
    out = torch.zeros(T, Hq, hd, dtype=tdt, device="cuda")
    wsb = B.eagle3_ttt_workspace_bytes(T, Hq, hd)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    B.eagle3_ttt_attention(B.BF16 if dtype == "bf16" else B.F32, T, S, Hq, Hkv, hd, _p(q), _p(k0), _p(v0),
                           _p(ks) if S else None, _p(vs) if S else None, _p(out), _p(ws), wsb, None)
    torch.cuda.synchronize()
    pos = list(range(T)) if T * Hq <= 8192 else sorted(set([0, 1, 255, 256, 767, 768, T - 1] +
                                                            [int(x) for x in rng.integers(0, T, 17)]))
    ref = ttt_attention(qn, k0n, v0n, ksn, vsn, positions=pos)[pos]
    got = out.float().cpu().numpy()[pos]
    err = np.abs(got - ref).max()
    print(f"  max |diff| {err:.3g} over {len(pos)} positions", flush=True)
    assert err <= (2e-2 if dtype == "bf16" else 1e-4 * np.abs(ref).max())


def test_sample_rows_match_oracle():
    rng = np.random.default_rng(6)
    V, n = 32000, 24
    eng = _tree_engine(2, 2, 3, V, batch=1)
    logits = rng.normal(0, 2, size=(n, V)).astype(np.float32)
    u = (rng.integers(0, 1 << 24, size=n) * 2.0 ** -24).astype(np.float32)
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    lg_d, u_d = to_dev(logits, torch.float32), to_dev(u, torch.float32)
    for T in (1.0, 0.7, 0.0):
        B.eagle3_sample(eng.ctx, n, _p(lg_d), T, _p(u_d), _p(out))
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for i in range(n):
            ref = int(np.argmax(logits[i])) if T == 0 else sample_inverse_cdf(probs_f32(logits[i], T), u[i])
            assert got[i] == ref
    eng.close()


# ------------------------------------------------------------------ compaction
def test_compact_kv_moves_path_rows():
    rng = np.random.default_rng(8)
    D, k, N, V, Bn = 6, 4, 32, 300, 3
    eng = _tree_engine(D, k, N, V, batch=Bn)
    kv = kv_view(eng)
    kv.copy_(torch.randn(kv.shape, device="cuda").to(eng.tdt))
    before = kv.clone()
    n = N + 1
    P = [17, 40, 3]
    maxp = D + 1
    paths, lens, toks = [], [], []
    for b in range(Bn):
        t, par = random_tree(rng, n, V)
        # a root-to-node path of random length
        node, pth = 0, [0]
        for _ in range(int(rng.integers(0, D + 1))):
            kids = [c for c in range(n) if par[c] == node]
            if not kids:
                break
            node = kids[int(rng.integers(len(kids)))]
            pth.append(node)
        paths.append(pth + [-1] * (maxp - len(pth)))
        lens.append(len(pth))
        toks.append(t)
    seq = to_dev(P)
    nroot = to_dev(rng.integers(0, V, Bn))
    aux_tree = torch.randn(Bn, n, 3 * eng.ms.d, device="cuda").to(eng.tdt)
    aux_new = torch.zeros(Bn, maxp, 3 * eng.ms.d, device="cuda").to(eng.tdt)
    ntok = torch.zeros(Bn, maxp, dtype=torch.int32, device="cuda")
    nlen = torch.zeros(Bn, dtype=torch.int32, device="cuda")
    keep = [to_dev(paths), to_dev(lens), to_dev(toks)]
    src_dst = torch.full((Bn, maxp, 2), 12345, dtype=torch.int32, device="cuda")
    B.eagle3_compact_kv(eng.ctx, Bn, _p(seq), n, _p(keep[0]), _p(keep[1]), _p(keep[2]), _p(nroot),
                        _p(aux_tree), _p(aux_new), _p(ntok), _p(nlen), _p(src_dst))
    torch.cuda.synchronize()
    _status_clear(eng)
    moves = src_dst.cpu().numpy()
    for b in range(Bn):
        ref = compaction_moves(P[b], paths[b][:lens[b]])
        assert [tuple(m) for m in moves[b, :lens[b]]] == ref, b
        assert (moves[b, lens[b]:] == -1).all(), b
    after = kv
    for b in range(Bn):
        L = lens[b]
        for j in range(L):
            assert torch.equal(after[:, :, b, :, P[b] + j], before[:, :, b, :, P[b] + paths[b][j]])
        assert torch.equal(after[:, :, b, :, :P[b]], before[:, :, b, :, :P[b]])
        assert seq[b].item() == P[b] + L and nlen[b].item() == L
        for j in range(L):
            assert torch.equal(aux_new[b, j], aux_tree[b, paths[b][j]])
        want = [toks[b][paths[b][j + 1]] for j in range(L - 1)] + [int(nroot[b].item())]
        assert list(ntok[b].cpu().numpy()[:L]) == want
    eng.close()


def test_device_status_flags_bad_inputs():
    """Capacity overflow and a malformed path raise device flags; nothing faults."""
    D, k, N, V = 4, 2, 6, 100
    eng = _tree_engine(D, k, N, V, batch=1)
    n = N + 1
    seq = to_dev([eng.max_seq - 2])            # no room for 7 tree rows
    toks = to_dev(np.arange(n)[None])
    logits = torch.zeros(n, V, device="cuda")
    zmask = torch.zeros(1, n, dtype=torch.int64, device="cuda")
    B.eagle3_verify_tree(eng.ctx, 0, 1, _p(seq), n, _p(toks), None, _p(zmask), B.LM_ALL, _p(logits), None, None, None)
    assert eng.device_status() & B.DEV_KV_OVERFLOW
    bad_path = to_dev([[0, 3, 2, -1, -1]])     # not increasing
    aux = torch.zeros(1, n, 3 * eng.ms.d, device="cuda").to(eng.tdt)
    keep = [to_dev([5]), to_dev([3]), to_dev([1]), torch.zeros(1, D + 1, 3 * eng.ms.d, device="cuda").to(eng.tdt),
            torch.zeros(1, D + 1, dtype=torch.int32, device="cuda"), torch.zeros(1, dtype=torch.int32, device="cuda")]
    moves = torch.zeros(1, D + 1, 2, dtype=torch.int32, device="cuda")
    B.eagle3_compact_kv(eng.ctx, 1, _p(keep[0]), n, _p(bad_path), _p(keep[1]), _p(toks), _p(keep[2]),
                        _p(aux), _p(keep[3]), _p(keep[4]), _p(keep[5]), _p(moves))
    assert eng.device_status() & B.DEV_BAD_PATH
    assert (moves.cpu().numpy() == -1).all() and keep[0].item() == 5     # nothing moved, length unchanged
    with pytest.raises(B.Eagle3Error):
        B.eagle3_verify_tree(eng.ctx, 0, 1, _p(seq), 65, _p(toks), None, _p(toks), B.LM_ALL, None, None, None, None)
    eng.close()


@pytest.mark.gpu
@pytest.mark.parametrize("N,K", [(16, 128), (48, 384), (4096, 1024), (7, 256), (5000, 128)])
def test_pack_linear_bit_exact(N, K):
    """eagle3_pack_linear moves every bf16 bit pattern to the index eagle3.h
    states and zero-fills the padding rows of a partial last 16-row block."""
    from test_abi_cpu import packed_index
    R16 = (N + 15) // 16 * 16
    rng = np.random.default_rng(N + K)
    w = rng.integers(0, 1 << 16, size=(N, K), dtype=np.uint16)
    src = torch.as_tensor(w.view(np.int16), device="cuda")
    dst = torch.full((R16 * K,), -1, dtype=torch.int16, device="cuda")
    B.eagle3_pack_linear(B.BF16, src.data_ptr(), dst.data_ptr(), N, K, torch.cuda.current_stream().cuda_stream)
    got = dst.cpu().numpy().view(np.uint16)
    ref = np.zeros(R16 * K, np.uint16)
    ref[packed_index(N, K).ravel()] = w.ravel()
    assert np.array_equal(got, ref)
