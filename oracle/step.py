"""The speculative step and its driver loops, one sequence at a time.

Sources (page title, section):
  * "EAGLE-3: Engineering Implementation of LLM Inference Acceleration",
    XI.1-XI.6 (prefill; catch-up of the draft over (g_i, e_{t_{i+1}}) for the
    newly committed positions; drafting from the last catch-up row's a;
    verify; accept; commit; the draft keeps K/V only for positions built from
    real g; the pending token becomes the next root) and VI.5-VI.6.
  * "Advanced speculative decoding: tree drafts and EAGLE", Implementation
    (tree verify at prefix + depth; the accepted path's K/V are appended to
    the cache, the rest discarded; the next root is the argmax at the end of
    the path) and the vanilla greedy decode it is compared with.
  * "Speculative Decoding (EAGLE3) in the vLLM Neuron Framework", Design
    Choices (speculation stops near the length limit; a request may verify
    fewer drafts, see paged.truncate_tree) and The propose()
    Method (prefill phase, then recurrent phase at increasing positions).

Readings (the pages leave these open):
  * A node at depth d sits at target position P + d; the draft row that
    expands it sits at draft position P + d - 1; the catch-up row of
    committed position i sits at i.
  * The draft's speculative K/V entries (one per expanded node) are visible to
    that node's descendants only, like the target's tree mask.
  * Sampled drafting draws each d_j from q_j = softmax(draft logits / T)
    (or takes the argmax when draft_greedy is set, making q_j one-hot).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .accept import argmax_rows_f32, chain_rejection, greedy_walk, tree_rejection
from .llama import (KVCache, Shape, causal_visible, draft_fuse, draft_layer, draft_logits,
                    target_forward)
from .numerics import argmax_first, probs_f32, sample_inverse_cdf
from .paged import truncate_tree
from .tree import Tree, build_dynamic_tree, tree_mask


@dataclass
class SpecConfig:
    mode: str               # "greedy_tree", "sample_chain" or "sample_tree"
    depth: int              # D (chain length K in sample_chain mode)
    topk: int               # k (1 in sample_chain mode)
    n_nodes: int            # N, draft nodes excluding the root
    temperature: float = 0.0
    draft_greedy: bool = False


def f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def build_sampled_chain(root: int, root_logits32, expand, K: int, temperature: float,
                        u_draft, draft_greedy: bool, d2t=None, vocab: int = None):
    """Chain draft by sampling: d_j ~ q_j, q_j = softmax(logits_j / T) (fp32).

    expand(d, [(token, parent_row)]) follows the same contract as in
    build_dynamic_tree.  Returns (tokens [K+1] root first, q [K, V] float32).
    With a reduced draft vocabulary (d2t, ascending target ids) the draw is over
    the draft ids, the token is d2t[id], and q is scattered into the target
    vocabulary of size `vocab` so that p and q share a support ("EAGLE-3:
    Engineering Implementation of LLM Inference Acceleration", VIII.6, X.2).
    """
    toks, qs = [root], []
    logits = f32(root_logits32)
    for j in range(K):
        if draft_greedy:
            t = argmax_first(logits)
            qd = np.zeros(logits.shape, dtype=np.float32)
            qd[t] = 1.0
        else:
            qd = probs_f32(logits, temperature)
            t = sample_inverse_cdf(qd, u_draft[j])
        if d2t is None:
            q = qd
        else:
            t = int(d2t[t])
            q = np.zeros(vocab, dtype=np.float32)
            q[np.asarray(d2t)] = qd
        toks.append(int(t))
        qs.append(q)
        if j + 1 < K:
            logits = f32(expand(j + 1, [(t, j - 1)])[0])
    return toks, np.stack(qs)


def compaction_moves(P: int, path):
    """The cache update over an accepted path as explicit moves ("Advanced
    speculative decoding: tree drafts and EAGLE", Implementation: the accepted
    nodes' K/V are appended to the cache in path order, the rest discarded).
    Tree row r of a step verified at committed length P was written at slot
    P + r; the j-th node of the path ends at slot P + j.  Returns [(source
    slot, destination slot)] in path order."""
    return [(int(P) + int(r), int(P) + j) for j, r in enumerate(path)]


class OracleSequence:
    """One sequence's full speculative state: target KV, draft KV, pending inputs."""

    def __init__(self, W: dict, H: dict, shp: Shape, spec: SpecConfig, capacity: int):
        self.W, self.H, self.shp, self.spec = W, H, shp, spec
        self.cache = KVCache(shp.n_layers, capacity, shp.n_kv_heads, shp.head_dim)
        self.dcache = KVCache(1, capacity, shp.n_kv_heads, shp.head_dim)
        self.root = None
        self.aux_new = None        # [c, 3d] aux of positions [P - c, P)
        self.next_tok = None       # [c] tokens at positions P - c + 1 .. P (last = root)
        self.emitted = []
        self.stats = []

    @property
    def P(self):
        return self.cache.length

    # ---------------------------------------------------------------- prefill
    def prefill(self, prompt, u_root=None):
        prompt = [int(t) for t in prompt]
        n = len(prompt)
        logits, k, v, aux = target_forward(self.W, self.shp, self.cache, prompt,
                                           np.arange(n), causal_visible(n))
        self._commit_rows(k, v, list(range(n)))
        row = f32(logits[-1])
        if self.spec.temperature == 0:
            self.root = argmax_first(row)
        else:
            self.root = sample_inverse_cdf(probs_f32(row, self.spec.temperature), u_root)
        self.aux_new = aux
        self.next_tok = prompt[1:] + [self.root]
        return logits

    def _commit_rows(self, k, v, rows):
        P = self.cache.length
        for l in range(self.shp.n_layers):
            for j, r in enumerate(rows):
                self.cache.k[l][P + j] = k[l][r]
                self.cache.v[l][P + j] = v[l][r]
        self.cache.length = P + len(rows)

    # ------------------------------------------------------------------ draft
    def draft_catchup(self):
        """Draft over the newly committed positions; returns a at position P - 1."""
        c = len(self.next_tok)
        P, dl = self.P, self.dcache.length
        assert dl == P - c
        g = draft_fuse(self.H, self.aux_new)
        base_k, base_v = self.dcache.k[0][:dl], self.dcache.v[0][:dl]

        def ctx(i, k, v):
            return (np.concatenate([base_k, k[:i + 1]]), np.concatenate([base_v, v[:i + 1]]))

        a, k, v = draft_layer(self.H, self.W, self.shp, self.next_tok, g, np.arange(dl, P), ctx)
        self.dcache.k[0][dl:P] = k
        self.dcache.v[0][dl:P] = v
        self.dcache.length = P
        return a[-1]

    def _expander(self, a_last):
        """expand() for the tree builders: runs the draft layer on frontier rows."""
        P = self.P
        rows_a, rows_k, rows_v, rows_anc = [], [], [], []   # per expansion row
        H, W, shp = self.H, self.W, self.shp

        def expand(d, info):
            first = len(rows_a)
            toks = [t for t, _ in info]
            xs = np.stack([a_last if pr < 0 else rows_a[pr] for _, pr in info])
            ancs = [([] if pr < 0 else rows_anc[pr] + [pr]) for _, pr in info]
            ck, cv = self.dcache.k[0][:P], self.dcache.v[0][:P]

            def ctx(i, k, v):
                anc = ancs[i]
                ks = [ck] + [rows_k[r][None] for r in anc] + [k[i:i + 1]]
                vs = [cv] + [rows_v[r][None] for r in anc] + [v[i:i + 1]]
                return np.concatenate(ks), np.concatenate(vs)

            a, k, v = draft_layer(H, W, shp, toks, xs, np.full(len(info), P + d - 1), ctx)
            for i in range(len(info)):
                rows_a.append(a[i])
                rows_k.append(k[i])
                rows_v.append(v[i])
                rows_anc.append(ancs[i])
            assert len(rows_a) == first + len(info)
            return [f32(draft_logits(H, W, shp, a[i])) for i in range(len(info))]

        return expand

    def draft_tree(self, u_draft=None):
        """The draft stage: catch-up, then the tree (or sampled chain).

        Returns (Tree, q) where q is [K, V] float32 in sample_chain mode, else None
        (sample_tree drafts the greedy mode's tree: its candidates are top-k picks).
        """
        a_last = self.draft_catchup()
        root_logits = f32(draft_logits(self.H, self.W, self.shp, a_last))
        expand = self._expander(a_last)
        s = self.spec
        if s.mode in ("greedy_tree", "sample_tree"):
            return build_dynamic_tree(self.root, root_logits, expand, s.depth, s.topk, s.n_nodes,
                                      self.H.get("d2t")), None
        toks, q = build_sampled_chain(self.root, root_logits, expand, s.depth, s.temperature,
                                      u_draft, s.draft_greedy, self.H.get("d2t"), self.shp.vocab)
        K = s.depth
        tree = Tree(toks, [-1] + list(range(K)), list(range(K + 1)), [np.float32(0)] * (K + 1),
                    [-2] + list(range(K - 1)) + [-1])
        return tree, q

    # ----------------------------------------------------------------- verify
    def verify(self, tree: Tree):
        """One target pass over the tree rows (prefix + ancestors + self)."""
        m = tree_mask(tree.parents)
        vis = [list(np.nonzero(m[i])[0]) for i in range(len(tree.tokens))]
        pos = self.P + np.asarray(tree.depth)
        return target_forward(self.W, self.shp, self.cache, tree.tokens, pos, vis)

    # ----------------------------------------------------------- accept+commit
    def accept(self, tree: Tree, logits, q=None, u_accept=None):
        if self.spec.mode == "greedy_tree":
            return greedy_walk(tree.tokens, tree.parents, argmax_rows_f32(logits))
        if self.spec.mode == "sample_tree":
            p = np.stack([probs_f32(f32(logits[i]), self.spec.temperature) for i in range(len(tree.tokens))])
            return tree_rejection(tree.tokens, tree.parents, p, u_accept, self.spec.topk, self.spec.depth)
        K = len(tree.tokens) - 1  # the request's draft length (the chain's full depth unless truncated)
        p = np.stack([probs_f32(f32(logits[i]), self.spec.temperature) for i in range(K + 1)])
        u = list(u_accept[:K]) + [u_accept[self.spec.depth]]  # the final draw keeps the row's last uniform
        n_acc, nxt = chain_rejection(tree.tokens[1:], q[:K], p, u)
        return list(range(n_acc + 1)), nxt

    def compact(self, tree: Tree, path, next_root, k, v, aux):
        """Commit the path: K/V of node path[j] -> slot P + j, aux and next tokens for the catch-up."""
        self._commit_rows(k, v, path)
        self.aux_new = aux[path]
        self.next_tok = [tree.tokens[i] for i in path[1:]] + [int(next_root)]
        self.emitted += [tree.tokens[i] for i in path]
        self.root = int(next_root)

    def step(self, u_draft=None, u_accept=None, tree=None, n_draft=None):
        """One speculative step.  A given ``tree`` replaces the drafted one (the draft's
        catch-up still runs so its cache stays consistent); tests inject trees that hold
        a known continuation to exercise multi-token acceptance.  ``n_draft`` limits the
        request's verified draft to its first n_draft nodes (paged.truncate_tree)."""
        if tree is None:
            tree, q = self.draft_tree(u_draft)
        else:
            self.draft_catchup()
            q = None
        if n_draft is not None:
            tree = truncate_tree(tree, n_draft)
        logits, k, v, aux = self.verify(tree)
        path, nxt = self.accept(tree, logits, q, u_accept)
        self.compact(tree, path, nxt, k, v, aux)
        self.stats.append(len(path))
        return tree, path, nxt


def vanilla_generate(W: dict, shp: Shape, prompt, max_new: int, temperature: float = 0.0,
                     uniforms=None, capacity: int = None):
    """Plain autoregressive decoding with a KV cache: one target pass per token."""
    prompt = [int(t) for t in prompt]
    cap = capacity or (len(prompt) + max_new + 1)
    cache = KVCache(shp.n_layers, cap, shp.n_kv_heads, shp.head_dim)
    toks = list(prompt)
    out = []
    feed = prompt
    for s in range(max_new):
        n0 = cache.length
        T = len(feed)
        logits, k, v, _ = target_forward(W, shp, cache, feed, np.arange(n0, n0 + T), causal_visible(T))
        for l in range(shp.n_layers):
            cache.k[l][n0:n0 + T] = k[l]
            cache.v[l][n0:n0 + T] = v[l]
        cache.length = n0 + T
        row = f32(logits[-1])
        if temperature == 0:
            t = argmax_first(row)
        else:
            t = sample_inverse_cdf(probs_f32(row, temperature), uniforms[s])
        out.append(t)
        toks.append(t)
        feed = [t]
    return out


def spec_generate(W: dict, H: dict, shp: Shape, spec: SpecConfig, prompt, max_new: int,
                  u_root=None, u_draft=None, u_accept=None, capacity: int = None):
    """Speculative decoding until max_new tokens exist; returns (tokens, per-step path lengths)."""
    rows = spec.n_nodes + 1
    cap = capacity or (len(prompt) + max_new + 2 * rows + spec.depth * spec.topk + 2)
    seq = OracleSequence(W, H, shp, spec, cap)
    seq.prefill(prompt, u_root)
    s = 0
    while len(seq.emitted) + 1 < max_new:
        ud = None if u_draft is None else u_draft[s]
        ua = None if u_accept is None else u_accept[s]
        seq.step(ud, ua)
        s += 1
    out = (seq.emitted + [seq.root])[:max_new]
    return out, seq.stats
