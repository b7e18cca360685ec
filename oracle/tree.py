"""Draft trees: ancestry mask, depths, and the two builders.

Sources (page title, section):
  * "Advanced speculative decoding: tree drafts and EAGLE", Why trees and
    Implementation (tree_mask: a node sees itself and all its ancestors;
    depths; positions are prefix length + depth; node 0 is the root with
    parent -1; build_draft_tree expands each frontier node into its
    top-branching[l] tokens) and Exercises (node counts of static trees).
  * "EAGLE-3: Engineering Implementation of LLM Inference Acceleration",
    VI.7 Draft Sequence, and "EAGLE-3: Training-Time Test for Speculative
    Decoding", Dynamic Draft Trees Spend Verification Where It Can Pay Off
    (EAGLE-2's tree: expand by draft confidence, prune after drafting).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .numerics import draft_logprobs_f32, topk_desc


def tree_mask(parents) -> np.ndarray:
    """[n, n] bool; row i is true at i and at every ancestor of i (walk to the root)."""
    n = len(parents)
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j != -1:
            m[i, j] = True
            j = parents[j]
    return m


def depths(parents) -> list:
    d = []
    for p in parents:
        d.append(0 if p == -1 else d[p] + 1)
    return d


def mask_words(parents) -> np.ndarray:
    """tree_mask packed one uint64 per row: bit j of row i set iff mask[i, j] (n <= 64)."""
    m = tree_mask(parents)
    n = len(parents)
    assert n <= 64
    out = np.zeros(n, dtype=np.uint64)
    for i in range(n):
        for j in range(n):
            if m[i, j]:
                out[i] |= np.uint64(1) << np.uint64(j)
    return out


def build_static_tree(root: int, branching, children_of):
    """Static tree with a fixed branching count per level ("Advanced speculative
    decoding: tree drafts and EAGLE", Implementation and Exercises).

    Level 0 is the root; every node of level l has branching[l] children.  The
    rows of a level are contiguous and the children of a node are contiguous
    in its level, so level l + 1 has prod(branching[:l + 1]) rows and its j-th
    row hangs under row j // branching[l] of level l.  children_of(path_tokens,
    width) gives the `width` tokens under the node reached by path_tokens
    (root first).  Returns (tokens, parents).
    """
    sizes = [1]
    for width in branching:
        sizes.append(sizes[-1] * int(width))
    first = [0]
    for n in sizes[:-1]:
        first.append(first[-1] + n)
    total = first[-1] + sizes[-1]
    parents = [-1] * total
    tokens = [int(root)] + [None] * (total - 1)
    prefix = {0: [int(root)]}                       # row -> tokens from the root down to the row
    for lvl, width in enumerate(branching):
        for j in range(sizes[lvl + 1]):
            parents[first[lvl + 1] + j] = first[lvl] + j // int(width)
        for i in range(sizes[lvl]):
            row = first[lvl] + i
            kids = list(children_of(list(prefix[row]), int(width)))
            for r in range(int(width)):
                child = first[lvl + 1] + i * int(width) + r
                tokens[child] = int(kids[r])
                prefix[child] = prefix[row] + [int(kids[r])]
    return tokens, parents


@dataclass
class Tree:
    tokens: list      # [N+1], root first
    parents: list     # [N+1], root -1
    depth: list       # [N+1]
    score: list       # [N+1] float32 cumulative draft log-prob, root 0
    expanded_as: list  # [N+1] index of the expansion row that produced the node's
                       # children, -1 if never expanded (the root is expanded by
                       # the catch-up row, reported as -2)


def build_dynamic_tree(root: int, root_logits32, expand, depth: int, topk: int, n_nodes: int,
                       d2t=None) -> Tree:
    """Dynamic draft tree ranked by cumulative draft log-probability.  The pages
    name EAGLE-2's confidence-driven expansion and final pruning but do not
    spell it out; this is a reading of it, pinned against itself by an
    independent enumeration of the candidates and against the pages by its
    k = 1 (greedy chain) and depth-1 (top-k) reductions.  The reading:

    * score(root) = 0; a child's score is fl32(score(parent) + logp(child)),
      with logp from :func:`draft_logprobs_f32` of the expanded row's logits.
    * Depth 1: the top-k tokens of the root's draft row (logit descending,
      lower token id on ties), in that order.
    * Depth 2..D: the frontier is the k best depth-(d-1) candidates by
      (score descending, creation index ascending); each frontier node, in
      frontier order, gets its top-k tokens as children.
    * Creation index: candidates are numbered in creation order (depth, then
      parent's frontier rank, then child rank).
    * After depth D: keep the N best of all candidates by (score desc,
      creation index asc) -- an ancestor-closed set because logp <= 0 -- and
      number them root first, then by (depth, creation index).

    expand(d, frontier) is called once per depth d = 1..D-1 with the frontier
    as a list of (token, parent_row), where parent_row is the expansion row of
    the node's parent (-1 when the parent is the root); the frontier nodes
    themselves become expansion rows numbered consecutively from 0 in call
    order.  It returns the float32 draft logits of each frontier row.

    d2t: with a reduced draft vocabulary the rows are over the draft ids and a
    child's token is d2t[draft id] (ascending target ids), ranked and scored in
    draft space ("EAGLE-3: Engineering Implementation of LLM Inference
    Acceleration", VIII.6); None is the identity.
    """
    cand_tok, cand_par, cand_dep, cand_score = [], [], [], []   # indexed by creation index
    row_of = {}                                                  # creation index -> expansion row

    def add_children(parent_cid, parent_score, logits32):
        lp = draft_logprobs_f32(logits32)
        for t in topk_desc(np.asarray(logits32, dtype=np.float32), topk):
            cand_tok.append(int(t) if d2t is None else int(d2t[t]))
            cand_par.append(parent_cid)
            cand_dep.append(1 if parent_cid < 0 else cand_dep[parent_cid] + 1)
            cand_score.append(np.float32(np.float32(parent_score) + lp[t]))

    add_children(-1, np.float32(0.0), root_logits32)
    for d in range(2, depth + 1):
        level = [c for c in range(len(cand_tok)) if cand_dep[c] == d - 1]
        level.sort(key=lambda c: (-float(cand_score[c]), c))
        frontier = level[:topk]
        info = [(cand_tok[c], row_of.get(cand_par[c], -1)) for c in frontier]
        for c in frontier:
            row_of[c] = len(row_of)
        rows = expand(d - 1, info)
        for rank, c in enumerate(frontier):
            add_children(c, cand_score[c], rows[rank])
    order = sorted(range(len(cand_tok)), key=lambda c: (-float(cand_score[c]), c))
    keep = order[:n_nodes]
    keep.sort(key=lambda c: (cand_dep[c], c))
    index = {c: i + 1 for i, c in enumerate(keep)}
    tokens, parents, dep, score, exp_as = [root], [-1], [0], [np.float32(0)], [-2]
    for c in keep:
        p = cand_par[c]
        assert p < 0 or p in index, "selected set must be ancestor-closed"
        tokens.append(cand_tok[c])
        parents.append(0 if p < 0 else index[p])
        dep.append(cand_dep[c])
        score.append(cand_score[c])
        exp_as.append(row_of.get(c, -1))
    return Tree(tokens, parents, dep, score, exp_as)


def tree_from_table(root: int, table32, depth: int, topk: int, n_nodes: int, d2t=None) -> Tree:
    """build_dynamic_tree with draft logits taken from a table instead of a draft model.

    table32[0] is the root's draft row; table32[1 + r] is expansion row r's
    (expansion rows are numbered in creation order across depths).  With a reduced
    draft vocabulary the rows are over draft ids and d2t maps them to tokens.
    """
    table32 = np.asarray(table32, dtype=np.float32)
    count = [0]

    def expand(d, info):
        rows = [table32[1 + count[0] + i] for i in range(len(info))]
        count[0] += len(info)
        return rows

    return build_dynamic_tree(root, table32[0], expand, depth, topk, n_nodes, d2t)
