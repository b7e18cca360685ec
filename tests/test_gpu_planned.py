"""Attention launches over many sequences of different lengths, against the oracle.

When one attention launch covers several sequences in more than one round of
workgroups, a small kernel first orders its work items (query block, KV head,
key chunk) by their number of key tiles and deals them over the XCDs; the
launches of every layer then run in that order.  When one chunk per (query
block, KV head) covers every key and still makes a full round of work items,
each item writes its rows' normalised output itself (no partials, no merge);
otherwise the chunks are 3,072 keys and the plan marks the partials of items
without keys as empty.  Neither changes what is computed, so each sequence's
tree logits must still equal the oracle's ("Advanced speculative decoding: tree
drafts and EAGLE", Implementation: the logits of a tree node equal those of its
path recomputed; "EAGLE-3: Engineering Implementation of LLM Inference
Acceleration", VIII.1 the draft layer's attention).  These tests check every
sequence of 64, with lengths from a few tokens to the cache's end, several on
or next to a chunk or tile boundary, on the verify (chunked and one-chunk
launches, one and two query blocks per sequence, head sizes 64 and 128, a paged
cache with chunks of more than 64 tiles) and on the draft stage.
"""
import numpy as np
import pytest
import torch

from gpu_util import logits_close, make_engine, margin_tol, oracle_weights, random_tree, to_dev, toy_shape, top2_margin
from oracle.llama import KVCache, target_forward, draft_logits
from oracle.step import OracleSequence, SpecConfig, f32
from oracle.tree import build_dynamic_tree, mask_words, tree_mask
from speculative_decoding_step_amd import binding as B
from speculative_decoding_step_amd import synth
from speculative_decoding_step_amd.engine import Spec

pytestmark = pytest.mark.gpu

def _lengths(n_rows, top):
    """64 prompt lengths up to top: short ones, 64-key tile and 3,072-key chunk boundaries from both sides
    (the tree rows end on or just past them), and the rest spread up to top."""
    edges = [2, 3, 7, 64 - n_rows, 64, 65, 1024 - n_rows, 1024, top]
    if top > 3072 + n_rows:
        edges += [3072 - n_rows, 3072 - n_rows + 1, 3072, 3073]
    rest = np.linspace(40, top - 10, 64 - len(edges)).astype(int).tolist()
    lens = np.array(edges + rest, dtype=np.int64)
    return lens[np.random.default_rng(3).permutation(64)]


def _policy(n_seq, rows, ms, max_seq, paged=False):
    """The launch policy this file exercises (bf16 attention at head size 64 or 128), mirrored: several
    sequences whose launch at 256-key chunks has at least 2,048 work items are planned; with one chunk per
    (query block, KV head) when that covers every key (at most 128 tiles) in at least 512 work items (direct
    output), else at 3,072-key chunks when those give at least 512.  Returns (planned, direct, qblocks)."""
    G = ms.n_heads // ms.n_kv_heads
    nq = rows * G
    nw = min(8, max(4, -(-nq // 16)))
    qblocks = -(-nq // (16 * nw))
    w1 = n_seq * qblocks * ms.n_kv_heads
    if not (n_seq > 1 and w1 * -(-max_seq // 256) >= 2048):
        return False, False, qblocks
    one = -(-max_seq // 64) * 64
    if one <= 128 * 64 and w1 >= 512:
        return True, True, qblocks
    return 512 <= w1 * -(-max_seq // 3072) <= 16384, False, qblocks


# (heads, KV heads, head size, d, cache length, paged block size): chunked plans at head sizes 128 (two query
# vectors per KV head: one query block) and 64 (four: two query blocks); one-chunk plans (direct output) at
# head sizes 64 and 128, and on a paged cache whose one chunk spans more than 64 tiles
VERIFY_CASES = [(4, 4, 128, 512, 3200, 0, False), (8, 2, 64, 512, 3200, 0, False), (8, 8, 64, 512, 2100, 0, False),
                (8, 8, 128, 1024, 2100, 0, False), (8, 8, 64, 512, 4300, 64, False),
                (4, 4, 128, 512, 3200, 0, True), (8, 8, 64, 512, 2100, 0, True)]


@pytest.mark.parametrize("heads,kv,hd,d,max_seq,bs,lengths", VERIFY_CASES)
def test_planned_verify_ragged_vs_oracle(heads, kv, hd, d, max_seq, bs, lengths):
    """64 sequences, each with its own random 40-node tree, verified in one call: every
    sequence's tree logits within 2e-2 of the oracle's over the GPU prefill's K/V, argmax
    wherever the oracle's top-2 margin clears twice that, and the tree rows' K/V.  With
    per-request draft lengths (0 .. 39 nodes, several 0) only each request's first nodes
    take part: those rows are checked, the others (padding rows in the planned launches)
    write no K/V."""
    ms = toy_shape(dtype="bf16", vocab=1000, layers=2, d=d, heads=heads, kv=kv, hd=hd, ffn=512)
    n, Bn = 40, 64
    planned, direct, qblocks = _policy(Bn, n, ms, max_seq, bs > 0)
    assert planned
    spec = Spec("greedy_tree", 4, 13, n - 1)
    lens = _lengths(n, max_seq - n - 3 * 13)  # the longest prompt a step of this tree budget fits
    print(f"\n[planned verify: {Bn} sequences, {lens.min()}..{lens.max()} tokens, {heads}/{kv} heads x {hd}, "
          f"{qblocks} query block(s) per sequence, {'one chunk' if direct else 'chunked'}"
          f"{f', paged ({bs}-key blocks)' if bs else ''}{', draft lengths' if lengths else ''}]", flush=True)
    eng = make_engine(ms, spec, batch=Bn, max_seq=max_seq, sigma=0.02, block_size=bs, page_seed=5 if bs else 0)
    nd = np.full(Bn, n - 1)
    if lengths:
        nd = np.random.default_rng(23).integers(0, n, size=Bn)
        nd[::7] = 0
        eng.set_draft_lengths(nd)
    shp, W, H = oracle_weights(ms, sigma=0.02)
    prompts = [synth.tokens_np(71, f"r{b}", int(lens[b]), ms.vocab) for b in range(Bn)]
    eng.prefill(prompts)
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    kv_before = eng.kv_logical("target").cpu() if lengths else None
    rng = np.random.default_rng(17)
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
    B.eagle3_verify_tree(eng.ctx, 0, Bn, seq_lens.data_ptr(), n, tok_d.data_ptr(), pos_d.data_ptr(),
                         mw.data_ptr(), B.LM_ALL, logits.data_ptr(), am.data_ptr(), mg.data_ptr(), None)
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    g_all, am_all = logits.cpu().numpy().reshape(Bn, n, -1), am.cpu().numpy().reshape(Bn, n)
    # [L, 2, B, Hkv, S, hd] bf16 on the host: the prefill's K/V at [0, P) (the verify writes only P..P+n-1)
    # and the tree rows' K/V
    kv = eng.kv_logical("target").cpu()
    eng.close()

    worst = 0.0
    for b in range(Bn):
        P = int(lens[b])
        cache = KVCache(shp.n_layers, max_seq, shp.n_kv_heads, shp.head_dim)
        kvb = kv[:, :, b, :, :P + n].double().numpy()  # [L, 2, Hkv, P + n, hd]
        for l in range(shp.n_layers):
            cache.k[l][:P] = kvb[l, 0, :, :P].transpose(1, 0, 2)
            cache.v[l][:P] = kvb[l, 1, :, :P].transpose(1, 0, 2)
        cache.length = P
        tokens, parents = trees[b]
        m = tree_mask(parents)
        ref, rk, rv, _ = target_forward(W, shp, cache, tokens, P + deps[b],
                                        [list(np.nonzero(m[i])[0]) for i in range(n)])
        nr = int(nd[b]) + 1  # the rows that take part
        err, ok = logits_close(g_all[b][:nr], ref[:nr], "bf16")
        worst = max(worst, err)
        assert ok, (b, P, err)
        for i in range(nr):
            if top2_margin(ref[i]) > 2 * margin_tol("bf16", ref[i]):
                assert am_all[b, i] == int(np.argmax(ref[i])), (b, i)
        for l in range(shp.n_layers):
            assert np.abs(kvb[l, 0, :, P:P + nr].transpose(1, 0, 2) - rk[l][:nr]).max() < 2e-2
            assert np.abs(kvb[l, 1, :, P:P + nr].transpose(1, 0, 2) - rv[l][:nr]).max() < 2e-2
        if lengths:  # the other rows wrote no K/V
            assert torch.equal(kv[:, :, b, :, P + nr:P + n], kv_before[:, :, b, :, P + nr:P + n]), b
    print(f"  tree logits: largest error over all sequences {worst:.3g}", flush=True)


@pytest.mark.parametrize("heads,kv,hd,max_seq", [(8, 8, 64, 2100), (4, 4, 128, 3200)])
def test_planned_draft_ragged_vs_oracle(heads, kv, hd, max_seq):
    """The draft stage of 64 sequences (catch-up and three tree levels of 4 rows per
    sequence, each attention launch planned: one chunk per item, then 3,072-key chunks):
    every sequence's draft logits table within 2e-2 of the oracle's draft stage over the
    same frontiers, started from the GPU prefill's outputs (tap row, root, committed
    draft K/V), and each tree exactly the one the oracle's builder makes from the GPU's
    own table."""
    ms = toy_shape(dtype="bf16", vocab=1000, layers=2, d=512, heads=heads, kv=kv, hd=hd, ffn=512)
    D, k, N, Bn = 4, 4, 12, 64
    p1, p2 = _policy(Bn, 1, ms, max_seq), _policy(Bn, k, ms, max_seq)
    assert p1[0] and p2[0] and p1[1] == p2[1]
    spec = Spec("greedy_tree", D, k, N)
    lens = _lengths(N + 1, max_seq - (N + 1) - (D - 1) * k)
    print(f"\n[planned draft: {Bn} sequences, {lens.min()}..{lens.max()} tokens, "
          f"{'one chunk' if p1[1] else 'chunked'}]", flush=True)
    eng = make_engine(ms, spec, batch=Bn, max_seq=max_seq, sigma=0.02)
    shp, W, H = oracle_weights(ms, sigma=0.02)
    prompts = [synth.tokens_np(73, f"d{b}", int(lens[b]), ms.vocab) for b in range(Bn)]
    eng.prefill(prompts)
    aux_rows = eng.aux_new[:, :1].to(torch.float64).cpu().numpy()
    roots = eng.next_tok[:, 0].cpu().numpy()
    dkv = eng.kv_logical("draft")[0].cpu()  # [2, B, Hkv, S, hd] bf16 on the host
    eng.record_draft_logits()
    eng.draft()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    table = eng.draft_table.cpu().numpy()
    g_tok, g_par = eng.tokens.cpu().numpy(), eng.parents.cpu().numpy()
    g_score = eng.score.cpu().numpy()
    eng.close()

    worst = 0.0
    for b in range(Bn):
        P = int(lens[b])
        root = int(roots[b])
        frontiers = []
        nxt = [1]

        def from_table(d, info):
            frontiers.append(info)
            out = [table[b, nxt[0] + i] for i in range(len(info))]
            nxt[0] += len(info)
            return out

        implied = build_dynamic_tree(root, table[b, 0], from_table, D, k, N)
        assert list(g_tok[b]) == implied.tokens and list(g_par[b]) == implied.parents, b
        assert np.array_equal(g_score[b], np.array(implied.score, dtype=np.float32)), b

        seq = OracleSequence(W, H, shp, SpecConfig("greedy_tree", D, k, N), max_seq)
        seq.cache.length = P
        seq.root, seq.aux_new, seq.next_tok = root, aux_rows[b], [root]
        dkb = dkv[:, b, :, :P - 1].double().numpy()
        seq.dcache.k[0][:P - 1] = dkb[0].transpose(1, 0, 2)
        seq.dcache.v[0][:P - 1] = dkb[1].transpose(1, 0, 2)
        seq.dcache.length = P - 1
        a_last = seq.draft_catchup()
        rows = [f32(draft_logits(H, W, shp, a_last))]
        expand = seq._expander(a_last)
        for d, info in enumerate(frontiers):
            rows.extend(expand(d + 1, info))
        assert len(rows) == 1 + (D - 1) * k
        err = max(float(np.abs(table[b, r].astype(np.float64) - rows[r]).max()) for r in range(len(rows)))
        worst = max(worst, err)
        assert err <= 2e-2, (b, P, err)
    print(f"  draft logits: largest error over all sequences {worst:.3g}", flush=True)


@pytest.mark.parametrize("heads,kv,hd,max_seq", [(8, 8, 64, 2100), (4, 4, 128, 3200)])
def test_planned_graph_replay_matches_eager(heads, kv, hd, max_seq):
    """A step over 64 ragged sequences captured into a graph (its draft levels and verify
    planned: one chunk per item, then 3,072-key chunks) and replayed four times equals
    four eager steps bit for bit: the work order is recomputed inside the graph from the
    lengths each replay finds."""
    ms = toy_shape(dtype="bf16", vocab=1000, layers=2, d=512, heads=heads, kv=kv, hd=hd, ffn=512)
    D, k, N, Bn, steps = 4, 4, 12, 64, 4
    assert _policy(Bn, N + 1, ms, max_seq)[0] and _policy(Bn, k, ms, max_seq)[0]
    spec = Spec("greedy_tree", D, k, N)
    lens = _lengths(N + 1, max_seq - (N + 1) - (D - 1) * k - steps * (D + 1))
    print(f"\n[planned graph replay: {Bn} sequences, {lens.min()}..{lens.max()} tokens]", flush=True)
    prompts = [synth.tokens_np(75, f"g{b}", int(lens[b]), ms.vocab) for b in range(Bn)]
    a = make_engine(ms, spec, batch=Bn, max_seq=max_seq, seed=31, sigma=0.3)
    b = make_engine(ms, spec, batch=Bn, max_seq=max_seq, seed=31, sigma=0.3)
    a.prefill(prompts)
    b.prefill(prompts)
    b.capture()
    for i in range(steps):
        a.step()
        b.replay()
        torch.cuda.synchronize()
        for name in ("tokens", "parents", "path", "path_len", "next_root", "seq_lens", "next_tok"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (i, name)
    assert a.device_status() == 0 and b.device_status() == 0
    plen = a.path_len.cpu().numpy()
    ka, kb = a.kv_logical(), b.kv_logical()
    for s in (int(np.argmin(lens)), int(np.argmax(lens))):
        P = int(a.seq_lens[s])
        assert torch.equal(ka[:, :, s, :, :P], kb[:, :, s, :, :P]), s
    print(f"  last step's path lengths {np.bincount(plen).tolist()}", flush=True)
    a.close()
    b.close()
