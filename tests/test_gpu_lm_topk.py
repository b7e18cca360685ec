"""The LM heads with the top-k in the GEMM epilogue, at their edges.

Passes of at most 64 rows take the head's top-k per 128-id slice in the
GEMM's epilogue and merge the slices in one more kernel ("EAGLE-3:
Engineering Implementation of LLM Inference Acceleration", VIII.6 LM head;
"Advanced speculative decoding: tree drafts and EAGLE", Implementation: the
children of a node are the top-k of its logits, the verify reads the argmax).
These tests drive a bf16 toy model whose vocabulary (9,000 ids) ends in a
partial slice, at the largest top-k (16), at draft passes of 16 and 32 rows,
at verify passes of 21 and 64 rows (and 66 on the large-M path) and under sampling at
T = 0.7, and check the outputs against the oracle's definitions applied to the
GPU's own logits: ranked ids and values, tree scores and the draws' q rows
(which carry the log-sum-exp) exactly, argmax and top-2 margin exactly.
"""
import numpy as np
import pytest
import torch

from gpu_util import make_engine, toy_shape
from oracle.numerics import logsumexp_f64, sample_inverse_cdf, topk_desc
from oracle.tree import build_dynamic_tree
from speculative_decoding_step_amd import synth
from speculative_decoding_step_amd.engine import Spec

pytestmark = pytest.mark.gpu

VOCAB = 9000  # 70 full 128-id slices and one of 40


def _implied_tree(table, root, D, k, N):
    nxt = [1]

    def from_table(d, info):
        out = [table[nxt[0] + i] for i in range(len(info))]
        nxt[0] += len(info)
        return out

    return build_dynamic_tree(root, table[0], from_table, D, k, N)


@pytest.mark.parametrize("Bn,D,k,N,V", [(1, 3, 16, 20, VOCAB), (1, 5, 15, 63, VOCAB), (2, 4, 8, 32, VOCAB),
                                        (3, 1, 6, 6, VOCAB), (2, 3, 8, 20, 140000)])
def test_fused_head_topk_tree_and_verify_argmax(Bn, D, k, N, V):
    """Greedy trees with top-k up to 16 over a vocabulary ending in a partial slice:
    each sequence's tree (ids, parents, fp32 scores) equals the oracle's builder over
    the GPU's own draft logits table, so every draft row's ranked top-k and
    log-sum-exp are exact (draft passes of 16 and 32 rows); the verify's argmax and
    top-2 margin equal the oracle's on the GPU's verify logits for every row (21
    and 64 rows in the fused kernels, 2 x 33 rows on the large-M path).  Depth 1
    (the root's children only) keeps one table row per sequence.  A vocabulary of
    140,000 ids (over the 1,024 slices the fused epilogue takes) runs the heads
    with a separate top-k pass over their logits."""
    ms = toy_shape(dtype="bf16", vocab=V, layers=2)
    spec = Spec("greedy_tree", D, k, N)
    eng = make_engine(ms, spec, batch=Bn, max_seq=192, seed=57, sigma=0.07)
    prompts = [list(synth.tokens_np(58 + b, "p", 40 - 3 * b, ms.vocab)) for b in range(Bn)]
    eng.prefill(prompts)
    roots = [int(eng.next_tok[b, 0]) for b in range(Bn)]
    eng.record_draft_logits()
    eng.logits = torch.zeros(Bn * eng.rows, ms.vocab, dtype=torch.float32, device="cuda")  # verify logits out
    eng.draft()
    eng.verify()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    table = eng.draft_table.cpu().numpy()
    g_tok, g_par = eng.tokens.cpu().numpy(), eng.parents.cpu().numpy()
    g_score = eng.score.cpu().numpy()
    assert table.shape == (Bn, 1 + (D - 1) * k, ms.vocab) and not np.isnan(table).any()
    rows = Bn * (N + 1)
    lg = eng.logits.cpu().numpy().reshape(-1, ms.vocab)[:rows]
    am = eng.argmax.cpu().numpy()[:rows]
    mg = eng.margin.cpu().numpy()[:rows]
    eng.close()

    for b in range(Bn):
        implied = _implied_tree(table[b], roots[b], D, k, N)
        assert list(g_tok[b]) == implied.tokens and list(g_par[b]) == implied.parents
        assert np.array_equal(g_score[b], np.array(implied.score, dtype=np.float32))
    for r in range(rows):
        t2 = topk_desc(lg[r], 2)
        assert am[r] == int(t2[0]), (r, am[r], t2)
        assert mg[r] == np.float32(lg[r][t2[0]] - lg[r][t2[1]]), (r, mg[r])


@pytest.mark.parametrize("Bn,D,k,N", [(2, 3, 8, 20), (1, 4, 5, 17)])
def test_fused_head_exact_ties(Bn, D, k, N):
    """LM-head rows planted in groups of four equal rows (ids 2m, 2m + 1, 2m + 4500,
    2m + 4501: two in one 128-id slice, two in another), so every logit value occurs
    exactly four times: each top-k pick ties across and within slices, and the order
    must be the lower id first (the tie rule of "Advanced speculative decoding: tree
    drafts and EAGLE", Implementation, argmax: the first maximal index).  Trees
    equal the oracle's builder over the GPU's own draft logits; verify argmax is
    the lowest id of the top group and the top-2 margin is zero."""
    ms = toy_shape(dtype="bf16", vocab=VOCAB, layers=2)
    eng = make_engine(ms, Spec("greedy_tree", D, k, N), batch=Bn, max_seq=160, seed=67, sigma=0.07)
    t = eng._tensor(67, "lm_head", (VOCAB, ms.d), "mat", 0.07)
    half = 4500
    src = (torch.arange(VOCAB, device="cuda") % half) // 2 * 2
    eng.w["lm_head"].copy_(eng._pack(t[src].contiguous()))
    torch.cuda.synchronize()
    prompts = [list(synth.tokens_np(68 + b, "p", 30 + 4 * b, ms.vocab)) for b in range(Bn)]
    eng.prefill(prompts)
    roots = [int(eng.next_tok[b, 0]) for b in range(Bn)]
    eng.record_draft_logits()
    eng.logits = torch.zeros(Bn * eng.rows, ms.vocab, dtype=torch.float32, device="cuda")
    eng.draft()
    eng.verify()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    table = eng.draft_table.cpu().numpy()
    g_tok, g_par = eng.tokens.cpu().numpy(), eng.parents.cpu().numpy()
    g_score = eng.score.cpu().numpy()
    rows = Bn * (N + 1)
    lg = eng.logits.cpu().numpy().reshape(-1, ms.vocab)[:rows]
    am = eng.argmax.cpu().numpy()[:rows]
    mg = eng.margin.cpu().numpy()[:rows]
    eng.close()
    ids = np.arange(VOCAB)
    grp = (ids % half) // 2 * 2
    # the ties are exact in the GPU's own logits
    assert np.array_equal(table[..., ids], table[..., grp]) and np.array_equal(lg[:, ids], lg[:, grp])
    for b in range(Bn):
        implied = _implied_tree(table[b], roots[b], D, k, N)
        assert list(g_tok[b]) == implied.tokens and list(g_par[b]) == implied.parents
        assert np.array_equal(g_score[b], np.array(implied.score, dtype=np.float32))
        kids = [int(x) for x in g_tok[b][1:k + 1]]
        assert kids[:4] == sorted(kids[:4]) and len({grp[x] for x in kids[:4]}) == 1  # one tied group, ids ascending
    for r in range(rows):
        t2 = topk_desc(lg[r], 2)
        assert am[r] == int(t2[0]) == grp[am[r]] and mg[r] == 0.0, (r, am[r], t2, mg[r])


@pytest.mark.parametrize("K", [4, 1])
def test_fused_head_sampled_chain_q_rows(K):
    """Sampled chain (K = 4 and the one-draft chain, T = 0.7, batch 3) on the fused
    draft head: every q row the draft outputs equals exp(z / T - lse) with the
    log-sum-exp taken by the oracle (float64, by definition) over the GPU's own
    draft logits row z, and every draft token is the inverse-CDF draw from that
    row."""
    ms = toy_shape(dtype="bf16", vocab=VOCAB, layers=2)
    Bn, T = 3, 0.7
    spec = Spec("sample_chain", K, 1, K, T)
    eng = make_engine(ms, spec, batch=Bn, max_seq=96, seed=61, sigma=0.07)
    prompts = [list(synth.tokens_np(62 + b, "p", 24 + 5 * b, ms.vocab)) for b in range(Bn)]
    eng.prefill(prompts, synth.uniform24_t(6000, "u_root", Bn, "cuda"))
    u_d = synth.uniform24_t(6000, "u_draft", Bn * K, "cuda").view(Bn, K)
    u_a = synth.uniform24_t(6000, "u_accept", Bn * (K + 1), "cuda").view(Bn, K + 1)
    eng.set_uniforms(u_d, u_a)
    eng.record_draft_logits()
    eng.draft()
    torch.cuda.synchronize()
    assert eng.device_status() == 0
    table = eng.draft_table.cpu().numpy()
    q = eng.q.cpu().numpy()
    toks = eng.tokens.cpu().numpy()
    ud = u_d.cpu().numpy()
    eng.close()
    assert table.shape == (Bn, K, ms.vocab) and not np.isnan(table).any()

    worst, mism = 0.0, 0
    for b in range(Bn):
        for j in range(K):
            z = table[b, j].astype(np.float32).astype(np.float64) / np.float64(np.float32(T))
            ref = np.exp(z - logsumexp_f64(z)).astype(np.float32)
            d = np.abs(q[b, j].astype(np.float64) - ref) / np.maximum(ref, 1e-30)
            worst = max(worst, float(d.max()))
            mism += int(np.count_nonzero(q[b, j] != ref))
            assert toks[b, j + 1] == sample_inverse_cdf(q[b, j], ud[b, j])
    print(f"\n  q rows: largest relative difference {worst:.3g}, entries not bit-equal {mism} of "
          f"{Bn * K * ms.vocab}", flush=True)
    assert worst <= 2.4e-7 and mism <= 4
