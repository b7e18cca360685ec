"""Pins of the oracle's tree code against the pages and against brute force."""
import itertools
import json
import os

import numpy as np
import pytest

from oracle.tree import (build_dynamic_tree, build_static_tree, depths, mask_words, tree_from_table,
                         tree_mask)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_p3_mask():
    rows, parents = [], None
    for line in open(os.path.join(GOLDEN, "p3_tree_mask.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("parents:"):
            parents = [int(x) for x in line.split(":")[1].split()]
        else:
            rows.append([int(x) for x in line.split()])
    return parents, np.array(rows, dtype=bool)


def test_tree_mask_matches_printed_example():
    parents, expect = _read_p3_mask()
    assert np.array_equal(tree_mask(parents), expect)


def test_depths_of_printed_example():
    parents, _ = _read_p3_mask()
    assert depths(parents) == [0, 1, 1, 2, 2, 2]


def _all_parent_arrays(n):
    """Every parent array with parent[0] = -1 and 0 <= parent[i] < i."""
    for rest in itertools.product(*[range(i) for i in range(1, n)]):
        yield [-1] + list(rest)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
def test_mask_brute_force(n):
    """Ancestry by set closure (brute force) == tree_mask == packed words == recurrence."""
    count = 0
    for parents in _all_parent_arrays(n):
        count += 1
        # brute force: the ancestor relation is the reflexive-transitive closure of child->parent
        anc = np.eye(n, dtype=bool)
        for i in range(n):
            if parents[i] >= 0:
                anc[i, parents[i]] = True
        for _ in range(n):
            anc = anc | ((anc.astype(np.int64) @ anc.astype(np.int64)) > 0)
        m = tree_mask(parents)
        assert np.array_equal(m, anc)
        words = mask_words(parents)
        rec = []
        for i in range(n):
            rec.append((0 if parents[i] < 0 else rec[parents[i]]) | (1 << i))
        assert [int(w) for w in words] == rec
        d = depths(parents)
        assert list(m.sum(1)) == [x + 1 for x in d]
    assert count == int(np.prod(range(1, n))) if n > 1 else count == 1


def test_static_tree_node_counts():
    """Exercise answer: [2, 2, 1, 1] has 14 nodes besides the root, [3, 3, 2] has 30."""
    def children(path, width):
        return list(range(width))

    for branching, expect in [([2, 2, 1, 1], 14), ([3, 3, 2], 30)]:
        toks, parents = build_static_tree(7, branching, children)
        assert len(toks) - 1 == expect
        assert parents[0] == -1 and all(0 <= p < i for i, p in enumerate(parents) if i)


def test_dynamic_tree_hand_worked():
    g = json.load(open(os.path.join(GOLDEN, "dynamic_tree_hand.json")))
    table = np.log(np.array(g["probs"], dtype=np.float64)).astype(np.float32)
    for n, exp in g["expect"].items():
        t = tree_from_table(g["root"], table, g["depth"], g["topk"], int(n))
        assert t.tokens == exp["tokens"]
        assert t.parents == exp["parents"]
        assert t.depth == exp["depth"]
        np.testing.assert_allclose(np.exp(np.array(t.score, dtype=np.float64)), exp["prob"], rtol=1e-5)


def _check_invariants(t, n_nodes, topk, D):
    n = len(t.tokens)
    assert n == n_nodes + 1
    assert t.parents[0] == -1 and t.depth[0] == 0
    for i in range(1, n):
        p = t.parents[i]
        assert 0 <= p < i
        assert t.depth[i] == t.depth[p] + 1 <= D
        assert t.score[i] <= t.score[p]
        assert t.depth[i] >= t.depth[i - 1]
    for p in range(n):
        kids = [t.tokens[c] for c in range(n) if t.parents[c] == p]
        assert len(kids) == len(set(kids)) <= topk


@pytest.mark.parametrize("D,k,N,V", [(3, 2, 5, 8), (4, 3, 10, 16), (6, 4, 32, 64), (6, 10, 60, 256),
                                     (4, 4, 16, 64), (2, 5, 3, 9)])
def test_dynamic_tree_invariants_random(D, k, N, V):
    rng = np.random.default_rng(D * 100 + k * 10 + N)
    for trial in range(5):
        table = rng.normal(0, 2, size=(1 + (D - 1) * k, V)).astype(np.float32)
        t = tree_from_table(int(rng.integers(V)), table, D, k, N)
        _check_invariants(t, N, k, D)


def test_dynamic_tree_selects_best_candidates_by_enumeration():
    """The kept nodes are the N best of every candidate the frontier rule creates,
    enumerated here independently by re-walking the same table."""
    rng = np.random.default_rng(5)
    D, k, N, V = 4, 3, 9, 12
    table = rng.normal(0, 2, size=(1 + (D - 1) * k, V)).astype(np.float32)
    t = tree_from_table(0, table, D, k, N)

    def logp(row):
        r = table[row].astype(np.float64)
        lse = np.float32(np.log(np.sum(np.exp(r - r.max()))) + r.max())
        return (table[row] - lse).astype(np.float32)

    # enumerate: level lists of (score, creation, token, parent creation)
    cands = []
    lp = logp(0)
    for t0 in np.argsort(-table[0], kind="stable")[:k]:
        cands.append((lp[t0], len(cands), int(t0), -1, 1))
    row = 1
    for d in range(2, D + 1):
        level = sorted([c for c in cands if c[4] == d - 1], key=lambda c: (-c[0], c[1]))[:k]
        for par in level:
            lp = logp(row)
            row += 1
            for tk in np.argsort(-table[row - 1], kind="stable")[:k]:
                cands.append((np.float32(par[0] + lp[tk]), len(cands), int(tk), par[1], d))
    best = sorted(cands, key=lambda c: (-c[0], c[1]))[:N]
    got = sorted(zip(t.score[1:], t.tokens[1:], t.depth[1:]), key=lambda x: (-x[0], x[2], x[1]))
    want = sorted([(c[0], c[2], c[4]) for c in best], key=lambda x: (-x[0], x[2], x[1]))
    assert [(float(a), b, c) for a, b, c in got] == [(float(a), b, c) for a, b, c in want]


def test_topk1_tree_is_the_greedy_chain():
    """With k = 1 the tree reduces to iterated argmax (a chain of depth D)."""
    rng = np.random.default_rng(9)
    D, V = 5, 20
    table = rng.normal(0, 1, size=(D, V)).astype(np.float32)
    t = tree_from_table(3, table, D, 1, D)
    assert t.parents == [-1] + list(range(D))
    assert t.tokens[1:] == [int(np.argmax(table[i])) for i in range(D)]


def test_depth1_tree_is_topk():
    rng = np.random.default_rng(10)
    V = 50
    row = rng.normal(0, 1, size=(1, V)).astype(np.float32)
    t = tree_from_table(0, row, 1, 7, 7)
    assert t.tokens[1:] == list(np.argsort(-row[0])[:7])
    assert t.parents == [-1] + [0] * 7


# ------------------------------------------------ reduced draft vocabulary
# ("EAGLE-3: Engineering Implementation of LLM Inference Acceleration", VIII.6: a
# draft-owned head over V_d ids, d2t back to target ids, ascending)

def _subset(rng, V, Vd):
    return np.sort(rng.choice(V, Vd, replace=False))


def test_reduced_vocab_tree_equals_masked_full_vocab_tree():
    """A tree drafted over V_d draft ids and mapped through d2t is the tree the full
    vocabulary would give if every non-draft token's logit were -inf: the same
    tokens, parents and scores (softmax over the draft ids only)."""
    rng = np.random.default_rng(12)
    V, Vd, D, k, N = 200, 57, 4, 3, 12
    d2t = _subset(rng, V, Vd)
    n_exp = (D - 1) * k
    small = rng.normal(0, 2, size=(1 + n_exp, Vd)).astype(np.float32)
    full = np.full((1 + n_exp, V), -np.inf, dtype=np.float32)
    full[:, d2t] = small
    t_red = tree_from_table(7, small, D, k, N, d2t)
    t_full = tree_from_table(7, full, D, k, N)
    assert t_red.tokens == t_full.tokens
    assert t_red.parents == t_full.parents
    assert [float(x) for x in t_red.score] == [float(x) for x in t_full.score]
    assert all(t in set(d2t.tolist()) for t in t_red.tokens[1:])


def test_reduced_vocab_identity_map_is_the_full_tree():
    rng = np.random.default_rng(13)
    V, D, k, N = 90, 3, 3, 8
    table = rng.normal(0, 2, size=(1 + (D - 1) * k, V)).astype(np.float32)
    a = tree_from_table(3, table, D, k, N, np.arange(V))
    b = tree_from_table(3, table, D, k, N)
    assert (a.tokens, a.parents) == (b.tokens, b.parents)
