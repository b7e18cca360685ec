"""Full-size parity at the 8B shape, in the launch configurations bench.py times.

The oracle cannot run all 32 layers at this size in a test, so the checks take
the outputs it can compute one by one: K/V written by layers 0 and 1 and the
tap entering layer 2 (hidden_states[2]) are compared with the oracle run on the
model's first two layers (same seeded weights), and every integer result of a
step (tree topology and masks, accepted paths, rejection-sampling decisions,
compaction) is checked bit-exactly against the oracle given the GPU's own
logits, over every sequence of the batch."""
import functools

import numpy as np
import pytest
import torch

from gpu_util import kv_view, random_tree, to_dev
from oracle.accept import chain_rejection, greedy_walk, tree_rejection
from oracle.llama import KVCache, Shape, causal_visible, target_forward
from oracle.numerics import probs_f32, sample_inverse_cdf
from oracle.tree import mask_words, tree_mask
from speculative_decoding_step_amd import binding as B
from speculative_decoding_step_amd import configs, synth
from speculative_decoding_step_amd.engine import Engine, Spec

pytestmark = pytest.mark.gpu


def _p(t):
    return None if t is None else t.data_ptr()


def _gen(seed, name, shape):
    return synth.normal_t(seed, name, shape, "cuda", 0.02, "bf16").to(torch.float64).cpu().numpy()


@functools.lru_cache(maxsize=1)
def _two_layer_weights(seed):
    ms = configs.L8B
    d = ms.d
    qd, kvd = ms.n_heads * ms.head_dim, ms.n_kv_heads * ms.head_dim
    layers = []
    for l in range(2):
        L = {"attn_norm": np.ones(d), "ffn_norm": np.ones(d)}
        for key, shape in [("wq", (qd, d)), ("wk", (kvd, d)), ("wv", (kvd, d)), ("wo", (d, qd)),
                           ("w_gate", (ms.ffn, d)), ("w_up", (ms.ffn, d)), ("w_down", (d, ms.ffn))]:
            L[key] = _gen(seed, f"l{l}.{key}", shape)
        layers.append(L)
    return layers


def _two_layer_oracle(seed, prompt, tokens, parents):
    """Oracle on target layers 0 and 1 for a prompt and a tree after it.

    Returns (prompt K [2][P, Hkv, hd], tree K, tree V [2][n, Hkv, hd], tree rows
    of hidden_states[2] [n, d]).  Tokens are remapped onto the embedding rows
    they use so that only those rows are materialised."""
    ms = configs.L8B
    d, P, n = ms.d, len(prompt), len(tokens)
    used = sorted(set(int(t) for t in prompt) | set(int(t) for t in tokens))
    remap = {t: i for i, t in enumerate(used)}
    emb = synth.normal_t(seed, "embed", (ms.vocab, d), "cuda", 0.02, "bf16")
    W = {"embed": emb[torch.as_tensor(used, device="cuda")].to(torch.float64).cpu().numpy(),
         "final_norm": np.ones(d), "lm_head": np.zeros((1, d)), "layers": _two_layer_weights(seed)}
    del emb
    shp = Shape(2, d, ms.n_heads, ms.n_kv_heads, ms.head_dim, ms.ffn, 1, ms.rope_theta, ms.eps, "bf16", (2, 2, 2))
    cache = KVCache(2, P + n + 1, ms.n_kv_heads, ms.head_dim)
    _, k, v, _ = target_forward(W, shp, cache, [remap[int(t)] for t in prompt], np.arange(P), causal_visible(P))
    for l in range(2):
        cache.k[l][:P], cache.v[l][:P] = k[l], v[l]
    cache.length = P
    dep = [0] * n
    for i in range(1, n):
        dep[i] = dep[parents[i]] + 1
    m = tree_mask(parents)
    _, tk, tv, aux = target_forward(W, shp, cache, [remap[int(t)] for t in tokens], P + np.array(dep),
                                    [list(np.nonzero(m[i])[0]) for i in range(n)])
    return k, tk, tv, aux[:, :d]


def _close(g, ref, what):
    e = np.abs(np.asarray(g, dtype=np.float64) - ref).max()
    scale = np.abs(ref).max()
    assert e <= 1e-2 * scale, (what, e, scale)
    return e, scale


def _check_tree(P, tokens, parents, depth, pos, mask, D):
    """Topology of one drafted tree: BFS order, depths, positions, ancestry masks, distinct siblings."""
    n = len(tokens)
    assert parents[0] == -1 and depth[0] == 0 and pos[0] == P
    for i in range(1, n):
        assert 0 <= parents[i] < i
        assert depth[i] == depth[parents[i]] + 1 <= D
        assert depth[i] >= depth[i - 1]
        assert pos[i] == P + depth[i]
    assert np.array_equal(np.asarray(mask, dtype=np.uint64), mask_words(list(parents)))
    for i in range(n):
        kids = [tokens[c] for c in range(n) if parents[c] == i]
        assert len(kids) == len(set(kids))


def test_8b_tree_verify_first_two_layers_vs_oracle():
    w = configs.WORKLOADS["llama8b_tree_b1"]
    ms = w.shape
    P, n, d = w.prompt_len, w.rows, ms.d
    print(f"\n[8B verify parity] P={P} rows={n}", flush=True)
    prompt = configs.prompts_np(w)[0]
    eng = Engine(ms, Spec.of(w), 1, P + 256, w.target_seed, w.head_seed, prefill_chunk=512)
    eng.prefill([prompt])
    rng = np.random.default_rng(12)
    tokens, parents = random_tree(rng, n, ms.vocab)
    dep = [0] * n
    for i in range(1, n):
        dep[i] = dep[parents[i]] + 1
    seq = to_dev([P])
    tok_d, pos_d = to_dev(tokens), to_dev(P + np.array(dep))
    mw = torch.as_tensor(mask_words(parents).view(np.int64), device="cuda")
    am = torch.zeros(n, dtype=torch.int32, device="cuda")
    auxo = torch.zeros(n, 3 * d, dtype=torch.bfloat16, device="cuda")
    B.eagle3_verify_tree(eng.ctx, 0, 1, _p(seq), n, _p(tok_d), _p(pos_d), _p(mw), B.LM_ALL, None, _p(am), None,
                         _p(auxo))
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    g_aux = auxo[:, :d].float().cpu().numpy()                       # taps[0] = 2
    kv = kv_view(eng)
    g_tree_k = kv[:2, 0, 0, :, P:P + n].float().cpu().numpy()       # [2, Hkv, n, hd]
    g_tree_v = kv[:2, 1, 0, :, P:P + n].float().cpu().numpy()
    sample_pos = [0, 1, 777, P - 1]
    g_pre_k = kv[:2, 0, 0, :, sample_pos].float().cpu().numpy()
    eng.close()
    del eng
    torch.cuda.empty_cache()

    k, tk, tv, aux = _two_layer_oracle(w.target_seed, prompt, tokens, parents)
    e, scale = _close(g_aux, aux, "tap 2")
    print(f"  tap-2 max err {e:.3g} (scale {scale:.3g})", flush=True)
    for l in range(2):
        _close(g_tree_k[l].transpose(1, 0, 2), tk[l], ("tree K", l))
        _close(g_tree_v[l].transpose(1, 0, 2), tv[l], ("tree V", l))
        _close(g_pre_k[l].transpose(1, 0, 2), k[l][sample_pos], ("prompt K", l))


def test_8b_batch64_ragged_tree_step():
    """Batch 64 with ragged prompts in [128, 4096] and a depth-4, top-4, 16-node
    tree (1088 verify rows): one whole step.  All 64 trees, accepted paths and
    compactions are checked exactly; verify K/V and taps of the shortest and
    the longest sequence against the two-layer oracle."""
    w = configs.WORKLOADS["llama8b_tree_b64"]
    ms, Bn, n, D = w.shape, w.batch, w.rows, w.depth
    prompts = configs.prompts_np(w)
    lens = np.array([len(p) for p in prompts])
    print(f"\n[8B batch {Bn}] prompt lengths {lens.min()}..{lens.max()} rows {Bn * n}", flush=True)
    eng = Engine(ms, Spec.of(w), Bn, int(lens.max()) + 64, w.target_seed, w.head_seed, prefill_chunk=512)
    eng.prefill(prompts)
    torch.cuda.synchronize()
    print("  prefill done", flush=True)
    eng.logits = torch.zeros(Bn * n, ms.vocab, dtype=torch.float32, device="cuda")  # verify writes every row's logits
    hid = torch.zeros(ms.n_layers + 1, Bn * n, ms.d, dtype=torch.float32, device="cuda")
    B.eagle3_set_hidden_out(eng.ctx, hid.data_ptr())
    eng.draft()
    eng.verify()
    B.eagle3_set_hidden_out(eng.ctx, None)
    eng.accept()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    tokens, parents = eng.tokens.cpu().numpy(), eng.parents.cpu().numpy()
    depth, pos = eng.depth.cpu().numpy(), eng.pos.cpu().numpy()
    mask = eng.mask.cpu().numpy().view(np.uint64)
    am = eng.argmax.cpu().numpy().reshape(Bn, n)
    path, plen = eng.path.cpu().numpy(), eng.path_len.cpu().numpy()
    nroot, emitted = eng.next_root.cpu().numpy(), eng.emitted.cpu().numpy()
    aux_tree = eng.aux_tree[:, :, :ms.d].float().cpu().numpy()
    kv = kv_view(eng)
    layers = [0, 1, ms.n_layers - 1]
    pre = [kv[layers, :, b, :, int(lens[b]):int(lens[b]) + n].clone() for b in range(Bn)]
    s0 = int(np.argmin(lens))
    P0 = int(lens[s0])
    kv_s0 = kv[:, :, s0, :, :P0].to(torch.float64).cpu().numpy()             # committed prefix, all layers
    tkv_s0 = kv[:, :, s0, :, P0:P0 + n].float().cpu().numpy()               # the tree rows' K/V, all layers
    hid_s0 = hid[:, s0 * n:(s0 + 1) * n].cpu().numpy()
    g_logits = eng.logits[s0 * n:(s0 + 1) * n].cpu().numpy()
    del hid
    eng.compact()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    seq_after = eng.seq_lens.cpu().numpy()
    for b in range(Bn):
        P = int(lens[b])
        _check_tree(P, tokens[b], parents[b], depth[b], pos[b], mask[b], D)
        walk, nxt = greedy_walk(list(tokens[b]), list(parents[b]), list(am[b]))
        assert list(path[b, :plen[b]]) == walk and nroot[b] == nxt
        assert list(emitted[b, :plen[b]]) == [int(tokens[b][i]) for i in walk]
        assert seq_after[b] == P + plen[b]
        moved = kv[layers, :, b, :, P:P + int(plen[b])]
        assert torch.equal(moved, pre[b][..., torch.as_tensor(walk, device="cuda"), :])
    print(f"  path lengths {np.bincount(plen)}", flush=True)
    checks = [int(np.argmin(lens)), int(np.argmax(lens))]
    g_tree = {b: pre[b][:2].float().cpu().numpy() for b in checks}    # [2 layers, K/V, Hkv, n, hd]
    eng.close()
    del eng, pre, kv
    torch.cuda.empty_cache()
    from test_gpu_8b_logits import per_layer_parity
    per_layer_parity(ms, w.target_seed, kv_s0, hid_s0, tkv_s0, tokens[s0], [int(x) for x in parents[s0]], P0,
                     g_logits, f"batch-64 seq {s0} (P={P0}, large-M GEMMs)")
    for b in checks:
        k, tk, tv, aux = _two_layer_oracle(w.target_seed, prompts[b], tokens[b], list(parents[b]))
        e, _ = _close(aux_tree[b], aux, ("tap 2", b))
        for l in range(2):
            _close(g_tree[b][l, 0].transpose(1, 0, 2), tk[l], ("tree K", b, l))
            _close(g_tree[b][l, 1].transpose(1, 0, 2), tv[l], ("tree V", b, l))
        print(f"  seq {b} (P={lens[b]}): tap-2 err {e:.3g}", flush=True)


def test_8b_sampling_chain_b4_steps():
    """Temperature-1 chain (K = 5) at batch 4, prompts of 64: two whole steps.
    Each draft token must be the inverse-CDF draw from the q row the draft
    produced, and every acceptance decision, resample and bonus must equal the
    oracle's rejection sampler given the GPU's p (from its verify logits), q and
    uniforms; the chain rows' layer-0/1 K/V match the two-layer oracle."""
    w = configs.WORKLOADS["llama8b_sample_chain_b4"]
    ms, Bn, K = w.shape, w.batch, w.depth
    prompts = configs.prompts_np(w)
    eng = Engine(ms, Spec.of(w), Bn, w.max_len, w.target_seed, w.head_seed, prefill_chunk=512)
    print(f"\n[8B sampling chain] batch {Bn} K={K}", flush=True)
    eng.prefill(prompts, synth.uniform24_t(5000, "u_root", Bn, "cuda"))
    seen = set()
    for s in range(2):
        u_d = synth.uniform24_t(5000, f"u_draft{s}", Bn * K, "cuda").view(Bn, K)
        u_a = synth.uniform24_t(5000, f"u_accept{s}", Bn * (K + 1), "cuda").view(Bn, K + 1)
        eng.set_uniforms(u_d, u_a)
        P = eng.seq_lens.cpu().numpy()
        eng.draft()
        eng.verify()
        eng.accept()
        torch.cuda.synchronize()
        assert eng.device_status() == 0
        toks, par = eng.tokens.cpu().numpy(), eng.parents.cpu().numpy()
        q = eng.q.cpu().numpy()
        lg = eng.logits.cpu().numpy().reshape(Bn, K + 1, ms.vocab)
        ud, ua = u_d.cpu().numpy(), u_a.cpu().numpy()
        plen, nroot, em = eng.path_len.cpu().numpy(), eng.next_root.cpu().numpy(), eng.emitted.cpu().numpy()
        if s == 0:
            chain_kv = kv_view(eng)[:2, :, 0, :, int(P[0]):int(P[0]) + K + 1].float().cpu().numpy()
            chain0 = [int(t) for t in toks[0]]
        for b in range(Bn):
            assert list(par[b]) == list(range(-1, K))
            assert list(eng.pos[b].cpu().numpy()) == [int(P[b]) + i for i in range(K + 1)]
            for i in range(K):
                assert abs(float(q[b, i].astype(np.float64).sum()) - 1.0) < 1e-4
                assert toks[b, i + 1] == sample_inverse_cdf(q[b, i], ud[b, i])
            p = np.stack([probs_f32(lg[b, i], 1.0) for i in range(K + 1)])
            n_acc, tok = chain_rejection(toks[b, 1:], q[b], p, ua[b])
            seen.add(n_acc)
            assert plen[b] == n_acc + 1 and nroot[b] == tok
            assert list(em[b]) == [int(x) for x in toks[b, :n_acc + 1]] + [-1] * (K - n_acc)
        eng.compact()
        torch.cuda.synchronize()
        assert list(eng.seq_lens.cpu().numpy()) == [int(P[b]) + int(plen[b]) for b in range(Bn)]
    print(f"  accepted counts seen {sorted(seen)}", flush=True)
    eng.close()
    del eng
    torch.cuda.empty_cache()
    k, tk, tv, _ = _two_layer_oracle(w.target_seed, prompts[0], chain0, list(range(-1, K)))
    for l in range(2):
        _close(chain_kv[l, 0].transpose(1, 0, 2), tk[l], ("chain K", l))
        _close(chain_kv[l, 1].transpose(1, 0, 2), tv[l], ("chain V", l))


def test_8b_sample_tree_b1_steps():
    """The batch-1 8B tree accepted by level-by-level rejection sampling at T = 1: three
    whole steps.  Each step's accepted path and next token must equal the oracle's tree
    rejection sampler given the GPU's tree, its verify logits (p over all 128,256 ids at
    every tree row) and the uniforms; compaction advances the sequence by the path."""
    w = configs.WORKLOADS["llama8b_sample_tree_b1"]
    ms, D, k = w.shape, w.depth, w.topk
    prompts = configs.prompts_np(w)
    eng = Engine(ms, Spec.of(w), 1, w.prompt_len + 256, w.target_seed, w.head_seed, prefill_chunk=512)
    print(f"\n[8B sampled tree] P={w.prompt_len} D{D} k{k} N{w.n_nodes} T={w.temperature}", flush=True)
    eng.prefill(prompts, synth.uniform24_t(5000, "u_root", 1, "cuda"))
    na = eng.n_u_accept
    lens = []
    for s in range(3):
        u_a = synth.uniform24_t(5000, f"u_accept{s}", na, "cuda").view(1, na)
        eng.set_uniforms(None, u_a)
        P = int(eng.seq_lens[0])
        eng.draft()
        eng.verify()
        eng.accept()
        torch.cuda.synchronize()
        assert eng.device_status() == 0
        toks, par = eng.tokens[0].cpu().numpy(), eng.parents[0].cpu().numpy()
        lg = eng.logits.cpu().numpy()
        p = np.stack([probs_f32(lg[i], w.temperature) for i in range(w.rows)])
        path, nxt = tree_rejection([int(t) for t in toks], [int(x) for x in par], p, u_a.cpu().numpy()[0], k, D)
        n = int(eng.path_len[0])
        assert list(eng.path[0].cpu().numpy()[:n]) == path and int(eng.next_root[0]) == nxt, s
        eng.compact()
        torch.cuda.synchronize()
        assert int(eng.seq_lens[0]) == P + n
        lens.append(n)
    print(f"  accepted path lengths {lens}", flush=True)
    eng.close()


def _seq_kv(eng, s, P, layers):
    """Target K/V of sequence s, positions [0, P), selected layers: [len(layers), 2, Hkv, P, hd]."""
    ms = eng.ms
    if not eng.block_size:
        return eng.kv_target.view(eng.tdt).view(ms.n_layers, 2, eng.B, ms.n_kv_heads, eng.max_seq,
                                                ms.head_dim)[layers, :, s, :, :P]
    bs = eng.block_size
    pool = eng.kv_target.view(eng.tdt).view(ms.n_layers, 2, eng.n_blocks, ms.n_kv_heads, bs, ms.head_dim)
    blocks = eng.block_table[s, :(P + bs - 1) // bs].long()
    g = pool[layers][:, :, blocks]                                   # [l, 2, nb, Hkv, bs, hd]
    return g.permute(0, 1, 3, 2, 4, 5).reshape(len(layers), 2, ms.n_kv_heads, -1, ms.head_dim)[..., :P, :]


def test_8b_batch64_paged_step_with_draft_lengths():
    """The batch-64 ragged workload on a paged cache (64-position blocks shuffled over the
    pool) with per-request draft lengths 0..16, against the same step on a contiguous
    cache: trees, verify argmax, paths and next tokens bit-identical where both verify a
    row; every path equals the greedy walk over the request's truncated tree; committed
    K/V identical for the shortest, a middle and the longest sequence (all layers' first
    and last)."""
    w = configs.WORKLOADS["llama8b_tree_b64_paged"]
    ms, Bn, n = w.shape, w.batch, w.rows
    prompts = configs.prompts_np(w)
    lens = np.array([len(p) for p in prompts])
    print(f"\n[8B batch {Bn} paged, block {w.block_size}] prompt lengths {lens.min()}..{lens.max()}", flush=True)
    a = Engine(ms, Spec.of(w), Bn, int(lens.max()) + 64, w.target_seed, w.head_seed, prefill_chunk=512)
    b = Engine(ms, Spec.of(w), Bn, int(lens.max()) + 64, w.target_seed, w.head_seed, prefill_chunk=512,
               weights=a.w, block_size=w.block_size, page_seed=w.cid)
    nd = np.random.default_rng(13).integers(0, n, size=Bn)
    nd[:4] = [0, n - 1, 1, 0]
    for e in (a, b):
        e.prefill(prompts)
        e.set_draft_lengths(nd)
        e.step()
    torch.cuda.synchronize()
    print("  prefill + one step on both caches done", flush=True)
    assert a.device_status() == 0 and b.device_status() == 0
    for name in ("tokens", "parents", "path", "path_len", "next_root", "seq_lens", "next_tok"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    am_a, am_b = a.argmax.view(Bn, n).cpu().numpy(), b.argmax.view(Bn, n).cpu().numpy()
    tokens, parents = b.tokens.cpu().numpy(), b.parents.cpu().numpy()
    path, plen = b.path.cpu().numpy(), b.path_len.cpu().numpy()
    for s in range(Bn):
        r = int(nd[s]) + 1
        assert (am_a[s, :r] == am_b[s, :r]).all(), s
        walk, nxt = greedy_walk(list(tokens[s, :r]), list(parents[s, :r]), list(am_b[s, :r]))
        assert list(path[s, :plen[s]]) == walk and b.next_root[s].item() == nxt, s
    order = np.argsort(lens)
    layers = [0, ms.n_layers - 1]
    for s in (int(order[0]), int(order[Bn // 2]), int(order[-1])):
        P = int(b.seq_lens[s])
        assert torch.equal(_seq_kv(a, s, P, layers), _seq_kv(b, s, P, layers)), s
    print(f"  path lengths {np.bincount(plen)}; zero-draft requests emitted "
          f"{sorted(set(plen[nd == 0].tolist()))} token(s)", flush=True)
    assert (plen[nd == 0] == 1).all()
    a.close()
    b.close()


def test_8b_graph_replay_matches_eager_steps():
    """Config 3 in the form the measurement times it: the whole step (draft,
    verify, accept, compact) captured once as a HIP graph and replayed, with
    eager work and synchronisations between the replays, gives bit-identical
    trees, accepted paths, next tokens and target K/V to eager steps of a
    second engine built from the same seeds."""
    w = configs.WORKLOADS["llama8b_tree_b1"]
    ms = w.shape
    prompt = configs.prompts_np(w)[0]
    print(f"\n[8B graph replay] P={len(prompt)}", flush=True)
    a = Engine(ms, Spec.of(w), 1, w.prompt_len + 256, w.target_seed, w.head_seed, prefill_chunk=512)
    b = Engine(ms, Spec.of(w), 1, w.prompt_len + 256, w.target_seed, w.head_seed, prefill_chunk=512)
    a.prefill([prompt])
    b.prefill([prompt])
    torch.cuda.synchronize()
    assert torch.equal(a.kv_target, b.kv_target) and torch.equal(a.next_tok, b.next_tok)
    b.capture()
    for i in range(4):
        a.step()
        b.replay()
        torch.cuda.synchronize()
        _ = b.seq_lens.sum().item()            # eager work between replays
        for name in ("tokens", "parents", "mask", "path", "path_len", "next_root", "seq_lens", "next_tok",
                     "argmax"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (i, name)
        assert torch.equal(a.kv_target, b.kv_target), i
        print(f"  step {i}: path length {int(a.path_len[0])}, next root {int(a.next_root[0])}", flush=True)
    assert a.device_status() == 0 and b.device_status() == 0
    a.close()
    b.close()


def test_8b_batch64_graph_replay_matches_eager_steps():
    """Config 5 (64 ragged prompts, planned attention with one chunk per item) as
    the measurement times it: the captured step graph, replayed twice, equals two
    eager steps of a second engine bit for bit (trees, paths, next tokens, caches)."""
    w = configs.WORKLOADS["llama8b_tree_b64"]
    ms, Bn = w.shape, w.batch
    prompts = configs.prompts_np(w)
    max_seq = int(max(len(p) for p in prompts)) + 64
    print(f"\n[8B batch {Bn} graph replay]", flush=True)
    a = Engine(ms, Spec.of(w), Bn, max_seq, w.target_seed, w.head_seed, prefill_chunk=512)
    b = Engine(ms, Spec.of(w), Bn, max_seq, w.target_seed, w.head_seed, prefill_chunk=512)
    a.prefill(prompts)
    b.prefill(prompts)
    torch.cuda.synchronize()
    print("  prefill done", flush=True)
    b.capture()
    for i in range(2):
        a.step()
        b.replay()
        torch.cuda.synchronize()
        _ = b.seq_lens.sum().item()
        for name in ("tokens", "parents", "mask", "path", "path_len", "next_root", "seq_lens", "next_tok",
                     "argmax"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (i, name)
        assert torch.equal(a.kv_target, b.kv_target) and torch.equal(a.kv_draft, b.kv_draft), i
        print(f"  step {i}: path lengths {np.bincount(a.path_len.cpu().numpy()).tolist()}", flush=True)
    assert a.device_status() == 0 and b.device_status() == 0
    a.close()
    b.close()
