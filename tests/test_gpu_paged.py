"""Paged KV caches, per-request draft lengths and the verify batch's index
bookkeeping on the GPU ("Speculative Decoding (EAGLE3) in the vLLM Neuron
Framework", The propose() Method, Design Choices, SpecDecodeMetadata: Index
Bookkeeping), through the C ABI, against the oracle."""
import json
import os

import numpy as np
import pytest
import torch

from gpu_util import make_engine, oracle_weights, toy_shape
from oracle.paged import spec_decode_metadata
from oracle.step import OracleSequence, SpecConfig, vanilla_generate
from speculative_decoding_step_amd import binding as B
from speculative_decoding_step_amd import synth
from speculative_decoding_step_amd.engine import Spec

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _i32(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device="cuda")


GUARD = 16  # extra entries past each capacity that the call must leave alone


def _metadata_gpu(cu, nd, ids, max_drafts):
    batch = len(cu)
    outs = {k: torch.full((n + GUARD,), -7, dtype=torch.int32, device="cuda") for k, n in
            (("cu", batch), ("li", batch + max_drafts), ("tli", max_drafts), ("bli", batch),
             ("dti", max_drafts), ("err", 1))}
    keep = [_i32(cu), _i32(nd), _i32(ids)]
    B.eagle3_spec_decode_metadata(batch, max_drafts, keep[0].data_ptr(), keep[1].data_ptr(), keep[2].data_ptr(),
                                  outs["cu"].data_ptr(), outs["li"].data_ptr(), outs["tli"].data_ptr(),
                                  outs["bli"].data_ptr(), outs["dti"].data_ptr(), outs["err"].data_ptr(), None)
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy().tolist() for k, v in outs.items()}
    for k, n in (("cu", batch), ("li", batch + max_drafts), ("tli", max_drafts), ("bli", batch),
                 ("dti", max_drafts), ("err", 1)):
        assert all(v == -7 for v in got[k][n:]), k          # nothing written past the capacity
        got[k] = got[k][:n]
    return got


def test_spec_decode_metadata_matches_oracle():
    print("\n[spec decode metadata]", flush=True)
    g = json.load(open(os.path.join(GOLDEN, "spec_decode_metadata_neuron.json")))
    cu, nd = g["cu_num_scheduled_tokens"], g["num_draft_tokens"]
    got = _metadata_gpu(cu, nd, np.arange(cu[-1]), sum(nd))
    assert got["cu"] == g["cu_num_draft_tokens"] and got["li"] == g["logits_indices"]
    assert got["dti"] == [cu[b] - nd[b] + t for b in range(5) for t in range(nd[b])]  # ids = positions here
    assert got["tli"] == g["target_logits_indices"] and got["bli"] == g["bonus_logits_indices"]
    assert got["err"] == [0]
    rng = np.random.default_rng(12)
    for B_ in (1, 7, 1023, 1024, 1025, 2500):            # chunks of the 1024-thread scan and their carries
        nd = rng.integers(0, 8, size=B_)
        ctx = rng.integers(1, 40, size=B_) * (rng.random(B_) < 0.3) + 1
        cu = np.cumsum(nd + ctx)
        ids = rng.integers(0, 128256, size=int(cu[-1]))
        ref = spec_decode_metadata(cu, nd, ids)
        got = _metadata_gpu(cu, nd, ids, int(nd.sum()))
        assert got["err"] == [0], B_
        assert got["cu"] == ref["cu_num_draft_tokens"], B_
        assert got["li"] == ref["logits_indices"], B_
        assert got["tli"] == ref["target_logits_indices"], B_
        assert got["bli"] == ref["bonus_logits_indices"], B_
        assert got["dti"] == ref["draft_token_ids"], B_
    # malformed requests raise the error word and stay inside the given capacities
    for cu, nd, cap in (([4, 6], [4, 0], 4), ([4, 6], [-1, 1], 1), ([3, 3, 5], [1, 0, 1], 2), ([4, 8], [3, 3], 2)):
        got = _metadata_gpu(cu, nd, np.arange(cu[-1]), cap)   # (the guard zones are checked inside)
        assert got["err"] == [1], (cu, nd)


def _ragged_prompts(ms, lens, seed):
    return [synth.tokens_np(seed, f"p{b}", n, ms.vocab) for b, n in enumerate(lens)]


@pytest.mark.parametrize("dtype,bs", [("bf16", 64), ("f32", 64), ("bf16", 128)])
def test_paged_steps_equal_contiguous(dtype, bs):
    """The same steps on a contiguous cache and on a paged one whose blocks are a shuffle
    of the pool: identical trees, paths and next tokens, and the same K/V position by
    position (target and draft), bit for bit."""
    print(f"\n[paged {dtype} block {bs}]", flush=True)
    ms = toy_shape(dtype=dtype, vocab=64, layers=2)
    spec = Spec("greedy_tree", 4, 3, 10)
    prompts = _ragged_prompts(ms, [70, 5, 130], 61)
    a = make_engine(ms, spec, batch=3, max_seq=200, seed=21, sigma=0.3)
    b = make_engine(ms, spec, batch=3, max_seq=200, seed=21, sigma=0.3, block_size=bs, page_seed=3)
    assert b.max_seq >= 200 and b.block_table.shape == (3, -(-200 // bs))
    a.prefill(prompts)
    b.prefill(prompts)
    for i in range(8):
        a.step()
        b.step()
        for name in ("tokens", "parents", "mask", "path", "path_len", "next_root", "seq_lens", "next_tok", "argmax"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (i, name)
    assert a.device_status() == 0 and b.device_status() == 0
    ka, kb = a.kv_logical("target"), b.kv_logical("target")
    da, db = a.kv_logical("draft"), b.kv_logical("draft")
    for s in range(3):
        P = int(a.seq_lens[s])
        assert torch.equal(ka[:, :, s, :, :P], kb[:, :, s, :, :P]), s
        Pd = P - int(a.new_len[s])                      # draft positions already caught up
        assert torch.equal(da[:, :, s, :, :Pd], db[:, :, s, :, :Pd]), s
    print(f"  lengths {a.seq_lens.tolist()}", flush=True)
    a.close()
    b.close()


def test_paged_tree_end_to_end_is_vanilla_greedy():
    """A paged toy model decodes the oracle's plain greedy continuation."""
    ms = toy_shape(dtype="f32", vocab=64, layers=2)
    spec = Spec("greedy_tree", 4, 3, 10)
    shp, W, H = oracle_weights(ms, seed=21, sigma=0.3)
    prompt = synth.tokens_np(41, "p", 90, ms.vocab)
    ref = vanilla_generate(W, shp, prompt, 40)
    eng = make_engine(ms, spec, max_seq=192, seed=21, sigma=0.3, block_size=64, page_seed=5)
    out, lens = eng.generate([prompt], 40)
    assert eng.device_status() == 0
    n = next((i for i in range(40) if out[0][i] != ref[i]), 40)
    print(f"\n  paged f32: identical to vanilla greedy for {n}/40", flush=True)
    assert n == 40
    eng.close()


def _oracle_seqs(W, H, shp, cfg, prompts, cap, u_root=None):
    seqs = []
    for b, p in enumerate(prompts):
        s = OracleSequence(W, H, shp, cfg, cap)
        s.prefill(p, None if u_root is None else np.float32(u_root[b]))
        seqs.append(s)
    return seqs


@pytest.mark.parametrize("bs", [0, 64])
def test_draft_lengths_greedy_match_oracle_f32(bs):
    """Random per-request draft lengths (0 .. N) each step: every request's tree, accepted
    path and next token equal the oracle's step over its truncated draft."""
    print(f"\n[draft lengths greedy, block {bs}]", flush=True)
    ms = toy_shape(dtype="f32", vocab=64, layers=2)
    D, k, N = 4, 3, 10
    spec = Spec("greedy_tree", D, k, N)
    shp, W, H = oracle_weights(ms, seed=21, sigma=0.3)
    prompts = _ragged_prompts(ms, [30, 12, 65], 62)
    eng = make_engine(ms, spec, batch=3, max_seq=160, seed=21, sigma=0.3, block_size=bs, page_seed=7)
    eng.prefill(prompts)
    seqs = _oracle_seqs(W, H, shp, SpecConfig("greedy_tree", D, k, N), prompts, 160)
    rng = np.random.default_rng(9)
    for step in range(8):
        nd = rng.integers(0, N + 1, size=3)
        nd[step % 3] = 0                                # plain decoding for one request each step
        eng.set_draft_lengths(nd)
        eng.step()
        assert eng.device_status() == 0
        for s in range(3):
            tree, path, nxt = seqs[s].step(n_draft=int(nd[s]))
            assert list(eng.tokens[s].cpu().numpy()[:len(tree.tokens)]) == tree.tokens, (step, s)
            n = eng.path_len[s].item()
            assert list(eng.path[s].cpu().numpy()[:n]) == path, (step, s, nd[s])
            assert eng.next_root[s].item() == nxt, (step, s)
            assert n <= nd[s] + 1
    eng.close()


@pytest.mark.parametrize("K", [4, 1])
def test_draft_lengths_sampled_chain_match_oracle_f32(K):
    """Sampled chains with per-request draft lengths: the accepted count and the
    resampled or bonus token equal the oracle's for the same uniforms (K = 1: a
    one-draft chain, lengths 0 or 1)."""
    ms = toy_shape(dtype="f32", vocab=96, layers=2)
    T = 0.8
    spec = Spec("sample_chain", K, 1, K, T)
    shp, W, H = oracle_weights(ms, seed=29, sigma=0.3)
    prompts = _ragged_prompts(ms, [24, 40], 63)
    eng = make_engine(ms, spec, batch=2, max_seq=128, seed=29, sigma=0.3, block_size=64, page_seed=2)
    u_root = synth.uniform24_t(5000, "u_root", 2, "cuda")
    eng.prefill(prompts, u_root)
    seqs = _oracle_seqs(W, H, shp, SpecConfig("sample_chain", K, 1, K, T), prompts, 128, u_root.cpu().numpy())
    rng = np.random.default_rng(10)
    lens = []
    for step in range(8):
        nd = rng.integers(0, K + 1, size=2)
        ud = synth.uniform24_t(5001, f"d{step}", 2 * K, "cuda").view(2, K)
        ua = synth.uniform24_t(5002, f"a{step}", 2 * (K + 1), "cuda").view(2, K + 1)
        if step % 2:  # acceptance uniforms scaled by 2^-24 (exact): the peaked toy target then accepts drafts
            ua = ua * 2.0 ** -24
        eng.set_uniforms(ud, ua)
        eng.set_draft_lengths(nd)
        eng.step()
        assert eng.device_status() == 0
        for s in range(2):
            tree, path, nxt = seqs[s].step(ud[s].cpu().numpy(), ua[s].cpu().numpy(), n_draft=int(nd[s]))
            n = eng.path_len[s].item()
            assert list(eng.path[s].cpu().numpy()[:n]) == path, (step, s, nd[s])
            assert eng.next_root[s].item() == nxt, (step, s)
            lens.append(n)
    print(f"\n  path lengths {lens}", flush=True)
    assert max(lens) >= 2
    eng.close()


def test_paged_graph_replay_sees_current_table_and_lengths():
    """A captured paged step replayed with new draft lengths and a rewritten block table
    (blocks moved to spare ids between replays) matches eager steps bit for bit."""
    ms = toy_shape(dtype="bf16", vocab=64, layers=2)
    spec = Spec("greedy_tree", 4, 3, 10)
    prompts = _ragged_prompts(ms, [40, 70], 64)
    a = make_engine(ms, spec, batch=2, max_seq=160, seed=21, sigma=0.3, block_size=64, page_seed=1)
    b = make_engine(ms, spec, batch=2, max_seq=160, seed=21, sigma=0.3, block_size=64, page_seed=1)
    a.prefill(prompts)
    b.prefill(prompts)
    a.set_draft_lengths([10, 10])
    b.set_draft_lengths([10, 10])
    b.capture()
    rng = np.random.default_rng(11)
    for i in range(6):
        nd = rng.integers(0, 11, size=2)
        a.set_draft_lengths(nd)
        b.set_draft_lengths(nd)
        if i == 3:  # move sequence 1's last block to a spare block in both engines (copying its contents)
            for e in (a, b):
                old = int(e.block_table[1, -1])
                used = set(e.block_table.flatten().tolist())
                new = next(x for x in range(e.n_blocks) if x not in used)
                for buf, L in ((e.kv_target, ms.n_layers), (e.kv_draft, 1)):
                    pool = buf.view(e.tdt).view(L, 2, e.n_blocks, -1)
                    pool[:, :, new] = pool[:, :, old]
                e.block_table[1, -1] = new
        a.step()
        b.replay()
        torch.cuda.synchronize()
        for name in ("tokens", "path", "path_len", "next_root", "seq_lens", "next_tok"):
            assert torch.equal(getattr(a, name), getattr(b, name)), (i, name)
    ka, kb = a.kv_logical(), b.kv_logical()
    for s in range(2):
        P = int(a.seq_lens[s])
        assert torch.equal(ka[:, :, s, :, :P], kb[:, :, s, :, :P]), s
    assert a.device_status() == 0 and b.device_status() == 0
    a.close()
    b.close()


def test_draft_lengths_sampled_tree_match_oracle_f32():
    """Tree rejection sampling with per-request draft lengths on a paged cache: every
    request's accepted path and next token equal the oracle's sampler over its truncated
    draft (children past the budget are never tested)."""
    ms = toy_shape(dtype="f32", vocab=96, layers=2)
    D, k, N, T = 3, 3, 8, 0.8
    spec = Spec("sample_tree", D, k, N, T)
    shp, W, H = oracle_weights(ms, seed=29, sigma=0.3)
    prompts = _ragged_prompts(ms, [24, 50], 65)
    eng = make_engine(ms, spec, batch=2, max_seq=128, seed=29, sigma=0.3, block_size=64, page_seed=4)
    u_root = synth.uniform24_t(5000, "u_root", 2, "cuda")
    eng.prefill(prompts, u_root)
    seqs = _oracle_seqs(W, H, shp, SpecConfig("sample_tree", D, k, N, T), prompts, 128, u_root.cpu().numpy())
    rng = np.random.default_rng(14)
    nu = eng.n_u_accept
    for step in range(6):
        nd = rng.integers(0, N + 1, size=2)
        ua = synth.uniform24_t(5003, f"a{step}", 2 * nu, "cuda").view(2, nu)
        eng.set_uniforms(None, ua)
        eng.set_draft_lengths(nd)
        eng.step()
        assert eng.device_status() == 0
        for s in range(2):
            tree, path, nxt = seqs[s].step(u_accept=ua[s].cpu().numpy(), n_draft=int(nd[s]))
            assert list(eng.tokens[s].cpu().numpy()[:len(tree.tokens)]) == tree.tokens, (step, s)
            n = eng.path_len[s].item()
            assert list(eng.path[s].cpu().numpy()[:n]) == path, (step, s, nd[s])
            assert eng.next_root[s].item() == nxt, (step, s)
    eng.close()
