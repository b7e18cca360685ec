"""End-to-end GPU speculative decoding against the oracle's vanilla decoding.

Greedy speculative decoding is lossless ("EAGLE-3: Engineering Implementation
of LLM Inference Acceleration", XI.6's token-for-token check; "Advanced
speculative decoding: tree drafts and EAGLE", Implementation), so the GPU's
speculative output must equal the oracle's plain greedy output token for token
up to the first position whose oracle top-2 logit margin is within the logits
tolerance (beyond it either token is a correct rounding of the model).
"""
import numpy as np
import pytest
import torch
from scipy.stats import chi2

from conftest import oracle_shape
from gpu_util import logits_close, make_engine, margin_tol, oracle_weights, toy_shape, top2_margin
from oracle.llama import KVCache, causal_visible, target_forward
from oracle.numerics import probs_f32
from oracle.step import OracleSequence, SpecConfig, vanilla_generate
from speculative_decoding_step_amd import configs, synth
from speculative_decoding_step_amd.engine import Engine, Spec

pytestmark = pytest.mark.gpu


def _teacher_forced_check(W, shp, prompt, gpu_out):
    """Every generated position, teacher-forced on the GPU's own prefix: where the
    oracle's top-2 margin exceeds twice the logits tolerance the GPU token must be
    the oracle's argmax, elsewhere it must be within that tolerance of the top
    logit.  Returns the number of positions checked strictly."""
    full = list(prompt) + list(gpu_out)
    cache = KVCache(shp.n_layers, len(full) + 1, shp.n_kv_heads, shp.head_dim)
    lg, _, _, _ = target_forward(W, shp, cache, full[:-1], np.arange(len(full) - 1), causal_visible(len(full) - 1))
    rows = lg[len(prompt) - 1:]
    strict = 0
    for i, (row, tok) in enumerate(zip(rows, gpu_out)):
        tol = 2 * margin_tol(shp.dtype, row)
        if top2_margin(row) > tol:
            assert tok == int(np.argmax(row)), (i, tok, int(np.argmax(row)))
            strict += 1
        else:
            assert row[tok] >= row.max() - tol, (i, tok)
    return strict


def _compare(gpu, ref, W, shp, prompt):
    """Exact agreement with the oracle's own greedy run up to the first low-margin
    position, then the teacher-forced check over the whole output."""
    strict = _teacher_forced_check(W, shp, prompt, gpu)
    upto = next((i for i in range(len(ref)) if gpu[i] != ref[i]), len(ref))
    return upto, strict


def test_tiny_f32_chain_config_end_to_end():
    w = configs.WORKLOADS["tiny_f32_chain"]
    print(f"\n[e2e {w.name}]", flush=True)
    shp = oracle_shape(w.shape)
    W, H = configs.weights_np(w.shape, w.target_seed, w.head_seed)
    prompt = configs.prompts_np(w)[0]
    ref = vanilla_generate(W, shp, prompt, w.max_new)
    eng = Engine(w.shape, Spec.of(w), 1, 32 + w.max_new + 16, w.target_seed, w.head_seed)
    out, lens = eng.generate([prompt], w.max_new)
    assert eng.device_status() == 0
    n, strict = _compare(out[0], ref, W, shp, prompt)
    print(f"  identical to oracle greedy for {n}/{w.max_new}; strict {strict}; steps {len(lens)}", flush=True)
    assert strict >= w.max_new // 2
    eng.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_toy_tree_end_to_end_with_acceptance(dtype):
    ms = toy_shape(dtype=dtype, vocab=64, layers=2)
    spec = Spec("greedy_tree", 4, 3, 10)
    shp, W, H = oracle_weights(ms, seed=21, sigma=0.3)
    prompt = synth.tokens_np(41, "p", 20, ms.vocab)
    ref = vanilla_generate(W, shp, prompt, 40)
    eng = make_engine(ms, spec, max_seq=128, seed=21, sigma=0.3)
    out, lens = eng.generate([prompt], 40)
    assert eng.device_status() == 0
    n, strict = _compare(out[0], ref, W, shp, prompt)
    pl = [int(x[0]) for x in lens]
    print(f"\n  toy {dtype}: identical for {n}/40, strict {strict}, path lengths {pl}", flush=True)
    assert strict >= 20 and max(pl) >= 2
    eng.close()


@pytest.mark.parametrize("D,k,N", [(1, 3, 3), (2, 1, 1), (6, 1, 6), (2, 8, 12)])
def test_degenerate_trees_end_to_end(D, k, N):
    """Trees at the edges of the budget: one level (the root's children only), a
    single draft node, a chain of single children, and a wide shallow tree whose N is
    not a multiple of k.  Greedy speculative output is vanilla greedy output and every
    accepted path fits the tree ("Advanced speculative decoding: tree drafts and
    EAGLE", Implementation: the accepted path is the longest prefix the target agrees
    with, so the output is the target's own greedy sequence)."""
    ms = toy_shape(dtype="f32", vocab=64, layers=2)
    spec = Spec("greedy_tree", D, k, N)
    shp, W, H = oracle_weights(ms, seed=21, sigma=0.3)
    prompt = synth.tokens_np(43, "p", 20, ms.vocab)
    ref = vanilla_generate(W, shp, prompt, 30)
    eng = make_engine(ms, spec, max_seq=128, seed=21, sigma=0.3)
    out, lens = eng.generate([prompt], 30)
    assert eng.device_status() == 0
    n, strict = _compare(out[0], ref, W, shp, prompt)
    pl = [int(x[0]) for x in lens]
    print(f"\n  D{D} k{k} N{N}: identical for {n}/30, strict {strict}, path lengths {pl}", flush=True)
    assert strict >= 15 and max(pl) <= D + 1
    eng.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_toy_tree_reduced_draft_vocab_end_to_end(dtype):
    """A draft head over 40 of the 64 ids (own head, d2t): greedy speculative output is
    still vanilla greedy output (a token outside the draft vocabulary can only come from
    the target's own argmax), and the tree tokens stay inside the draft vocabulary."""
    import dataclasses
    ms = dataclasses.replace(toy_shape(dtype=dtype, vocab=64, layers=2), draft_vocab=40)
    spec = Spec("greedy_tree", 4, 3, 10)
    shp, W, H = oracle_weights(ms, seed=21, sigma=0.3)
    prompt = synth.tokens_np(41, "p", 20, ms.vocab)
    ref = vanilla_generate(W, shp, prompt, 40)
    eng = make_engine(ms, spec, max_seq=128, seed=21, sigma=0.3)
    out, lens = eng.generate([prompt], 40)
    assert eng.device_status() == 0
    n, strict = _compare(out[0], ref, W, shp, prompt)
    inside = set(H["d2t"].tolist())
    assert all(int(t) in inside for t in eng.tokens[0, 1:].cpu().numpy())
    pl = [int(x[0]) for x in lens]
    outside = sum(1 for t in out[0] if t not in inside)
    print(f"\n  toy {dtype} V_d 40: identical for {n}/40, strict {strict}, path lengths {pl}, "
          f"{outside} tokens outside the draft vocabulary", flush=True)
    assert strict >= 20
    eng.close()


def test_draft_tree_reduced_vocab_matches_oracle_f32():
    """The whole draft stage with a draft-owned head over a reduced vocabulary (fp32)."""
    import dataclasses
    ms = dataclasses.replace(toy_shape(dtype="f32", vocab=96, layers=2), draft_vocab=57)
    spec = Spec("greedy_tree", 4, 3, 10)
    shp, W, H = oracle_weights(ms, seed=23, sigma=0.3)
    prompt = synth.tokens_np(42, "p", 30, ms.vocab)
    eng = make_engine(ms, spec, max_seq=96, seed=23, sigma=0.3)
    eng.prefill([prompt])
    eng.draft()
    torch.cuda.synchronize()
    seq = OracleSequence(W, H, shp, SpecConfig("greedy_tree", 4, 3, 10), 96)
    seq.prefill(prompt)
    t, _ = seq.draft_tree()
    assert eng.device_status() == 0
    sc = eng.score[0].cpu().numpy()
    ref_sc = np.array(t.score, dtype=np.float32)
    np.testing.assert_allclose(sc, ref_sc, atol=1e-4)
    # the seed's candidate scores are at least 1e-3 apart, ten times the score tolerance, so the
    # topology must agree exactly
    ordered = np.sort(ref_sc)
    assert np.min(np.diff(ordered)[ordered[1:] < 0]) > 1e-3
    assert list(eng.tokens[0].cpu().numpy()) == t.tokens
    assert list(eng.parents[0].cpu().numpy()) == t.parents
    eng.close()


def test_small_bf16_config_short_run():
    w = configs.scaled(configs.WORKLOADS["small_bf16_tree"], prompt_len=128, max_new=24)
    print(f"\n[e2e {w.name} short]", flush=True)
    shp = oracle_shape(w.shape)
    W, H = configs.weights_np(w.shape, w.target_seed, w.head_seed)
    prompt = configs.prompts_np(w)[0]
    ref = vanilla_generate(W, shp, prompt, w.max_new)
    eng = Engine(w.shape, Spec.of(w), 1, 128 + w.max_new + 64, w.target_seed, w.head_seed)
    out, lens = eng.generate([prompt], w.max_new)
    assert eng.device_status() == 0
    n, strict = _compare(out[0], ref, W, shp, prompt)
    print(f"  identical for {n}/{w.max_new}, strict {strict}", flush=True)
    assert strict >= 8
    eng.close()


def test_draft_tree_matches_oracle_f32():
    """The whole draft stage (catch-up, expansions, re-rank) on an fp32 toy model."""
    ms = toy_shape(dtype="f32", vocab=96, layers=2)
    spec = Spec("greedy_tree", 4, 3, 10)
    shp, W, H = oracle_weights(ms, seed=23, sigma=0.3)
    prompt = synth.tokens_np(42, "p", 30, ms.vocab)
    eng = make_engine(ms, spec, max_seq=96, seed=23, sigma=0.3)
    eng.prefill([prompt])
    eng.draft()
    torch.cuda.synchronize()
    seq = OracleSequence(W, H, shp, SpecConfig("greedy_tree", 4, 3, 10), 96)
    seq.prefill(prompt)
    t, _ = seq.draft_tree()
    assert eng.device_status() == 0
    assert eng.tokens[0, 0].item() == seq.root
    sc = eng.score[0].cpu().numpy()
    ref_sc = np.array(t.score, dtype=np.float32)
    np.testing.assert_allclose(sc, ref_sc, atol=1e-4)
    # the seed's candidate scores are at least 1e-3 apart, ten times the score tolerance, so the
    # topology must agree exactly
    ordered = np.sort(ref_sc)
    assert np.min(np.diff(ordered)[ordered[1:] < 0]) > 1e-3
    assert list(eng.tokens[0].cpu().numpy()) == t.tokens
    assert list(eng.parents[0].cpu().numpy()) == t.parents
    eng.close()


def test_sampled_chain_first_token_distribution_v64():
    """Vocab-64 variant of the sampling workload: chain K=5 at T=1, rejection + bonus.
    The first token the step decides after a fixed root is distributed as the
    target p(. | prompt, root): chi-square over 1e5 seeded draws."""
    ms = configs.ModelShape(2, 256, 4, 2, 64, 512, 64, 1e4, (0, 1, 1), dtype="f32")
    K, Bn, reps = 5, 1000, 100
    spec = Spec("sample_chain", K, 1, K, 1.0)
    shp, W, H = oracle_weights(ms, seed=31, sigma=0.1)
    prompt = list(synth.tokens_np(43, "p", 8, ms.vocab))
    eng = make_engine(ms, spec, batch=Bn, max_seq=32, seed=31, sigma=0.1, prefill_chunk=16)
    u_root = synth.uniform24_t(5000, "u_root", Bn, "cuda")
    eng.prefill([prompt] * Bn, u_root)
    root = 5
    eng.next_tok[:, 0] = root
    saved = [t.clone() for t in (eng.seq_lens, eng.new_len, eng.aux_new, eng.next_tok)]
    counts = np.zeros(ms.vocab)
    for s in range(reps):
        for t, v in zip((eng.seq_lens, eng.new_len, eng.aux_new, eng.next_tok), saved):
            t.copy_(v)
        eng.set_uniforms(synth.uniform24_t(5000, f"u_draft{s}", Bn * K, "cuda").view(Bn, K),
                         synth.uniform24_t(5000, f"u_accept{s}", Bn * (K + 1), "cuda").view(Bn, K + 1))
        eng.step()
        em = eng.emitted.cpu().numpy()
        pl = eng.path_len.cpu().numpy()
        nr = eng.next_root.cpu().numpy()
        first = np.where(pl >= 2, em[:, 1], nr)
        counts += np.bincount(first, minlength=ms.vocab)
    assert eng.device_status() == 0
    cache = KVCache(shp.n_layers, 16, shp.n_kv_heads, shp.head_dim)
    full = prompt + [root]
    lg, _, _, _ = target_forward(W, shp, cache, full, np.arange(len(full)), causal_visible(len(full)))
    p = probs_f32(lg[-1].astype(np.float32), 1.0).astype(np.float64)
    exp = p * counts.sum()
    keep = exp >= 5
    obs_m = np.append(counts[keep], counts[~keep].sum())
    exp_m = np.append(exp[keep], exp[~keep].sum())
    if exp_m[-1] < 5:
        obs_m, exp_m = obs_m[:-1], exp_m[:-1]
    stat = ((obs_m - exp_m) ** 2 / exp_m).sum()
    pval = chi2.sf(stat, len(obs_m) - 1)
    print(f"\n  chi-square {stat:.1f} dof {len(obs_m) - 1} p={pval:.3g}", flush=True)
    assert pval > 1e-3
    eng.close()


def test_sampled_tree_first_token_distribution_v64():
    """Vocab-64 tree under sampling (depth 3, top-3, 8 nodes, T = 1): the first token the
    step decides after a fixed root is distributed as the target p(. | prompt, root),
    whatever the draft tree: chi-square over 1e5 seeded draws."""
    ms = configs.ModelShape(2, 256, 4, 2, 64, 512, 64, 1e4, (0, 1, 1), dtype="f32")
    D, k, N, Bn, reps = 3, 3, 8, 1000, 100
    spec = Spec("sample_tree", D, k, N, 1.0)
    shp, W, H = oracle_weights(ms, seed=37, sigma=0.1)
    prompt = list(synth.tokens_np(47, "p", 8, ms.vocab))
    eng = make_engine(ms, spec, batch=Bn, max_seq=40, seed=37, sigma=0.1, prefill_chunk=16)
    eng.prefill([prompt] * Bn, synth.uniform24_t(5000, "u_root", Bn, "cuda"))
    root = 11
    eng.next_tok[:, 0] = root
    saved = [t.clone() for t in (eng.seq_lens, eng.new_len, eng.aux_new, eng.next_tok)]
    nu = eng.n_u_accept
    counts = np.zeros(ms.vocab)
    lens = np.zeros(D + 2)
    for s in range(reps):
        for t, v in zip((eng.seq_lens, eng.new_len, eng.aux_new, eng.next_tok), saved):
            t.copy_(v)
        eng.set_uniforms(None, synth.uniform24_t(5000, f"u_tree{s}", Bn * nu, "cuda").view(Bn, nu))
        eng.step()
        em = eng.emitted.cpu().numpy()
        pl = eng.path_len.cpu().numpy()
        nr = eng.next_root.cpu().numpy()
        counts += np.bincount(np.where(pl >= 2, em[:, 1], nr), minlength=ms.vocab)
        lens += np.bincount(pl, minlength=D + 2)
    assert eng.device_status() == 0
    cache = KVCache(shp.n_layers, 16, shp.n_kv_heads, shp.head_dim)
    full = prompt + [root]
    lg, _, _, _ = target_forward(W, shp, cache, full, np.arange(len(full)), causal_visible(len(full)))
    p = probs_f32(lg[-1].astype(np.float32), 1.0).astype(np.float64)
    exp = p * counts.sum()
    keep = exp >= 5
    obs_m = np.append(counts[keep], counts[~keep].sum())
    exp_m = np.append(exp[keep], exp[~keep].sum())
    if exp_m[-1] < 5:
        obs_m, exp_m = obs_m[:-1], exp_m[:-1]
    stat = ((obs_m - exp_m) ** 2 / exp_m).sum()
    pval = chi2.sf(stat, len(obs_m) - 1)
    print(f"\n  chi-square {stat:.1f} dof {len(obs_m) - 1} p={pval:.3g}; path lengths {lens[1:].astype(int)}",
          flush=True)
    assert pval > 1e-3
    eng.close()


@pytest.mark.parametrize("D,k,N", [(3, 3, 8), (1, 4, 4)])
def test_sampled_tree_steps_match_oracle_f32(D, k, N):
    """Tree drafts accepted by rejection sampling, eight steps on an fp32 toy model: every
    step's tree, accepted path and next token equal the oracle's for the same uniforms
    (also for a one-level tree, whose root children are the only candidates)."""
    ms = toy_shape(dtype="f32", vocab=96, layers=2)
    T = 0.8
    spec = Spec("sample_tree", D, k, N, T)
    shp, W, H = oracle_weights(ms, seed=29, sigma=0.3)
    prompt = synth.tokens_np(52, "p", 24, ms.vocab)
    eng = make_engine(ms, spec, max_seq=96, seed=29, sigma=0.3)
    u_root = synth.uniform24_t(5000, "u_root", 1, "cuda")
    eng.prefill([prompt], u_root)
    seq = OracleSequence(W, H, shp, SpecConfig("sample_tree", D, k, N, T), 96)
    seq.prefill(prompt, np.float32(u_root.cpu().numpy()[0]))
    assert eng.next_tok[0, 0].item() == seq.root
    nu = eng.n_u_accept
    lens = []
    for s in range(8):
        u = synth.uniform24_t(5000, f"u_acc{s}", nu, "cuda").view(1, nu)
        if s % 2:  # uniforms scaled by 2^-24 (exact): acceptances under the peaked toy target, longer paths
            u = u * 2.0 ** -24
        eng.set_uniforms(None, u)
        eng.step()
        tree, path, nxt = seq.step(u_accept=u.cpu().numpy()[0])
        assert eng.device_status() == 0
        assert list(eng.tokens[0].cpu().numpy()) == tree.tokens
        n = eng.path_len[0].item()
        assert list(eng.path[0].cpu().numpy()[:n]) == path
        assert eng.next_root[0].item() == nxt
        lens.append(n)
    print(f"\n  accepted path lengths {lens}", flush=True)
    assert max(lens) >= 2
    eng.close()


def test_graph_replay_matches_eager_steps():
    """The captured step graph, replayed with eager work and synchronisations in
    between, gives bit-identical tokens, paths and KV to eager steps."""
    ms = toy_shape(dtype="bf16", vocab=64, layers=2)
    spec = Spec("greedy_tree", 4, 3, 10)
    prompt = synth.tokens_np(44, "p", 24, ms.vocab)
    a = make_engine(ms, spec, max_seq=160, seed=21, sigma=0.3)
    b = make_engine(ms, spec, max_seq=160, seed=21, sigma=0.3)
    a.prefill([prompt])
    b.prefill([prompt])
    b.capture()
    for i in range(8):
        a.step()
        b.replay()
        torch.cuda.synchronize()
        _ = b.seq_lens.sum().item()            # eager work between replays
        for name in ("tokens", "parents", "mask", "path", "path_len", "next_root", "seq_lens", "next_tok",
                     "argmax"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (i, name)
        assert torch.equal(a.kv_target, b.kv_target), i
    assert a.device_status() == 0 and b.device_status() == 0
    a.close()
    b.close()
