"""Pins of acceptance: the greedy walk, and rejection sampling against its closed form
(the emitted token is distributed exactly as the target p, Leviathan et al. A.1 as cited
by "EAGLE-3: Engineering Implementation of LLM Inference Acceleration", III.5)."""
import numpy as np
from scipy.stats import chi2

from oracle.accept import chain_rejection, emitted_row, greedy_walk
from oracle.numerics import sample_inverse_cdf


def test_greedy_walk_hand_cases():
    tokens = [5, 1, 2, 3, 4, 7]
    parents = [-1, 0, 0, 1, 1, 2]
    # root predicts 2 -> node 2; node 2 predicts 7 -> node 5; node 5 predicts 9 (no child)
    argmax = [2, 0, 7, 0, 0, 9]
    assert greedy_walk(tokens, parents, argmax) == ([0, 2, 5], 9)
    # nothing matches: path is the root only, next root is the root's argmax
    assert greedy_walk(tokens, parents, [8, 0, 0, 0, 0, 0]) == ([0], 8)
    assert emitted_row([5, 2, 7], 5) == [5, 2, 7, -1, -1]


def _rand_dist(rng, V, conc=1.0):
    p = rng.gamma(conc, 1.0, V)
    return (p / p.sum()).astype(np.float32)


def _draws(rng, n, K, V, p_rows, q_rows):
    """First emitted token after the root for n independent cycles (drafts drawn from q)."""
    out = np.empty(n, dtype=np.int64)
    for s in range(n):
        u = (rng.integers(0, 1 << 24, K + 1 + K) * 2.0 ** -24).astype(np.float32)
        d = [sample_inverse_cdf(q_rows[j], u[K + 1 + j]) for j in range(K)]
        n_acc, nxt = chain_rejection(d, q_rows, p_rows, u[:K + 1])
        out[s] = d[0] if n_acc >= 1 else nxt
    return out


def _chi2_pvalue(counts, probs):
    exp = probs * counts.sum()
    order = np.argsort(exp)
    # merge small bins until every expected count is >= 5
    obs_m, exp_m, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += exp[i]
        if acc_e >= 5:
            obs_m.append(acc_o)
            exp_m.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        obs_m[-1] += acc_o
        exp_m[-1] += acc_e
    obs_m, exp_m = np.array(obs_m), np.array(exp_m)
    stat = np.sum((obs_m - exp_m) ** 2 / exp_m)
    return chi2.sf(stat, len(obs_m) - 1)


def test_rejection_marginal_chi_square_v64():
    rng = np.random.default_rng(1234)
    V, K = 64, 1
    p = np.stack([_rand_dist(rng, V) for _ in range(K + 1)])
    q = np.stack([_rand_dist(rng, V) for _ in range(K)])
    draws = _draws(rng, 100_000, K, V, p, q)
    assert _chi2_pvalue(np.bincount(draws, minlength=V).astype(float), p[0].astype(np.float64)) > 1e-3


def test_rejection_total_variation_v8():
    rng = np.random.default_rng(77)
    V, K = 8, 1
    p = np.stack([_rand_dist(rng, V) for _ in range(K + 1)])
    q = np.stack([_rand_dist(rng, V) for _ in range(K)])
    draws = _draws(rng, 200_000, K, V, p, q)
    tv = 0.5 * np.abs(np.bincount(draws, minlength=V) / len(draws) - p[0]).sum()
    assert tv < 0.005


def test_rejection_two_token_joint_v8():
    """Chain of two drafts over a toy conditional model: the first two emitted tokens
    follow p1(t1) p2(t2 | t1).  When a cycle stops after one token the next token is
    drawn from the target directly (what the next cycle's root would be)."""
    rng = np.random.default_rng(99)
    V = 8
    P1, Q1 = _rand_dist(rng, V), _rand_dist(rng, V)
    P2 = np.stack([_rand_dist(rng, V) for _ in range(V)])
    Q2 = np.stack([_rand_dist(rng, V) for _ in range(V)])
    P3 = _rand_dist(rng, V)
    n = 100_000
    joint = np.zeros((V, V))
    for s in range(n):
        u = (rng.integers(0, 1 << 24, 6) * 2.0 ** -24).astype(np.float32)
        d1 = sample_inverse_cdf(Q1, u[3])
        d2 = sample_inverse_cdf(Q2[d1], u[4])
        n_acc, nxt = chain_rejection([d1, d2], np.stack([Q1, Q2[d1]]), np.stack([P1, P2[d1], P3]), u[:3])
        if n_acc == 0:
            t1 = nxt
            t2 = sample_inverse_cdf(P2[t1], u[5])
        elif n_acc == 1:
            t1, t2 = d1, nxt
        else:
            t1, t2 = d1, d2
        joint[t1, t2] += 1
    expect = (P1[:, None].astype(np.float64) * P2.astype(np.float64)).ravel()
    assert _chi2_pvalue(joint.ravel(), expect) > 1e-3


def test_acceptance_probability_worked_example():
    """p(d) = 0.6, q(d) = 0.8: accepted with probability 0.75; p = 0.6, q = 0.4: always.
    Exhaustive over the 2**24-point uniform grid."""
    V = 4
    grid = np.arange(1 << 24, dtype=np.float64) * 2.0 ** -24
    for pd, qd, expect in [(0.6, 0.8, 0.75), (0.6, 0.4, 1.0)]:
        p = np.array([pd, 1 - pd, 0, 0], np.float32)
        q = np.array([qd, 1 - qd, 0, 0], np.float32)
        ratio = np.float32(p[0] / q[0])
        frac = np.mean(grid.astype(np.float32) < ratio)
        assert abs(frac - expect) < 2e-7
        # the routine's decision agrees on sampled uniforms
        for u in grid[::1 << 18].astype(np.float32):
            n_acc, _ = chain_rejection([0], q[None], np.stack([p, p]), np.array([u, 0.5], np.float32))
            assert (n_acc == 1) == (u < ratio)


def test_greedy_draft_residual_zeroes_the_draft_token():
    """Greedy drafts (q one-hot): a rejected draft token can never be the replacement."""
    rng = np.random.default_rng(8)
    V = 16
    p = _rand_dist(rng, V)
    for d in range(V):
        q = np.zeros(V, np.float32)
        q[d] = 1
        for u_final in np.linspace(0, 1 - 2.0 ** -24, 50).astype(np.float32):
            u = np.array([0.9999, u_final], np.float32)
            n_acc, nxt = chain_rejection([d], q[None], np.stack([p, p]), u)
            if n_acc == 0:
                assert nxt != d


# ---------------------------------------------------------------- trees under sampling
# Pins of oracle.accept.tree_rejection ("Advanced speculative decoding: tree drafts and
# EAGLE", Exercises, trees under sampling): at every level the emitted token must be
# distributed exactly as the target p of the node the walk stands on, whatever the
# (deterministic) candidates are.

from oracle.accept import tree_rejection  # noqa: E402
from oracle.numerics import int_weights  # noqa: E402


def _u_grid(rng, n):
    return (rng.integers(0, 1 << 24, n) * 2.0 ** -24).astype(np.float32)


def _first_token(path, nxt, tokens):
    return int(tokens[path[1]]) if len(path) > 1 else int(nxt)


def test_tree_rejection_first_token_chi_square_v64():
    """Fixed tree (root with 4 candidates, each with 2 children), fixed target rows, random
    uniforms: the first emitted token follows p at the root.  The candidates hold most of
    the root's mass (as a draft's top-k would), so a missing renormalisation after a
    rejection or a residual that keeps rejected tokens moves their frequencies by tens of
    percent."""
    rng = np.random.default_rng(2024)
    V, k, D = 64, 4, 2
    tokens = [0, 5, 17, 3, 40, 1, 2, 9, 8, 33, 34, 60, 61]
    parents = [-1, 0, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4]
    p = np.stack([_rand_dist(rng, V, 0.7) for _ in tokens])
    root = 0.2 * _rand_dist(rng, V).astype(np.float64)
    root[[5, 17, 3, 40]] += [0.30, 0.25, 0.15, 0.10]
    p[0] = (root / root.sum()).astype(np.float32)
    n = 60_000
    first = np.empty(n, dtype=np.int64)
    for s in range(n):
        path, nxt = tree_rejection(tokens, parents, p, _u_grid(rng, D * k + 1), k, D)
        first[s] = _first_token(path, nxt, tokens)
    assert _chi2_pvalue(np.bincount(first, minlength=V).astype(float), p[0].astype(np.float64)) > 1e-3


def test_tree_rejection_two_token_joint_v8():
    """Toy conditional model: the target row of a node holding token t is P2[t] (the root's
    is P1).  The first two emitted tokens follow P1(t1) P2(t2 | t1); when a cycle emits only
    one token the second is drawn from the target directly (what the next cycle's root
    would be)."""
    rng = np.random.default_rng(31)
    V, k, D = 8, 3, 2
    P1 = _rand_dist(rng, V)
    P2 = np.stack([_rand_dist(rng, V) for _ in range(V)])
    P3 = _rand_dist(rng, V)
    # root -> P1's three most likely tokens; each of them -> its row's two most likely
    # (the candidates a draft close to the target would propose)
    top1 = [int(t) for t in np.argsort(-P1, kind="stable")[:3]]
    tokens, parents = [7] + top1, [-1, 0, 0, 0]
    for j, t in enumerate(top1):
        for c in np.argsort(-P2[t], kind="stable")[:2]:
            tokens.append(int(c))
            parents.append(1 + j)
    rows = [P1] + [P2[t] for t in top1] + [P3] * 6
    p = np.stack(rows)
    joint = np.zeros((V, V))
    n = 80_000
    for s in range(n):
        u = _u_grid(rng, D * k + 2)
        path, nxt = tree_rejection(tokens, parents, p, u[:D * k + 1], k, D)
        if len(path) == 1:
            t1, t2 = nxt, sample_inverse_cdf(P2[nxt], u[-1])
        elif len(path) == 2:
            t1, t2 = tokens[path[1]], nxt
        else:
            t1, t2 = tokens[path[1]], tokens[path[2]]
        joint[t1, t2] += 1
    expect = (P1[:, None].astype(np.float64) * P2.astype(np.float64)).ravel()
    assert _chi2_pvalue(joint.ravel(), expect) > 1e-3


def test_tree_rejection_candidate_probabilities_closed_form():
    """Root with three candidates: over the whole 2**24 grid of each candidate's uniform,
    candidate i is accepted with probability W_i / (S - sum of earlier W) (the residual
    after the earlier rejections), so the candidate emitted is x_i with total probability
    p(x_i) and the residual draw covers the rest."""
    V = 6
    p = np.array([0.05, 0.30, 0.10, 0.25, 0.20, 0.10], np.float32)
    W = int_weights(p).astype(object)
    S = sum(W)
    cand = [3, 1, 4]
    grid = np.arange(1 << 24, dtype=np.uint64)
    total, reach = 0.0, 1.0
    rem = S
    for x in cand:
        # fraction of the grid accepted: floor(u * rem) < W_x, computed exactly
        hi, lo = np.uint64(int(rem) >> 24), np.uint64(int(rem) & 0xFFFFFF)
        r = grid * hi + ((grid * lo) >> np.uint64(24))
        frac = float(np.mean(r < np.uint64(int(W[x]))))
        assert abs(frac - float(W[x]) / float(rem)) < 2 ** -23
        total += reach * frac
        assert abs(reach * frac - float(p[x])) < 1e-6
        reach *= 1 - frac
        rem -= W[x]
    assert abs(reach - (1 - float(p[cand].sum()))) < 1e-6
    # the routine itself, on a few uniforms: accepts the first candidate exactly when u is
    # below its residual share
    tokens, parents = [0] + cand, [-1, 0, 0, 0]
    prow = np.stack([p] * 4)
    for u0 in np.linspace(0, 1 - 2.0 ** -24, 41).astype(np.float32):
        u = np.array([u0, 0.999, 0.999, 0.5], np.float32)
        path, _ = tree_rejection(tokens, parents, prow, u, 3, 1)
        assert (path == [0, 1]) == (u0 < float(W[3]) / float(S))


def test_tree_rejection_special_cases():
    rng = np.random.default_rng(5)
    V = 16
    p = _rand_dist(rng, V)
    tokens, parents = [0, 4, 9, 2], [-1, 0, 0, 0]
    # a rejected candidate never comes back as the residual token
    for s in range(400):
        u = _u_grid(rng, 4)
        u[:3] = np.maximum(u[:3], np.float32(0.999))  # reject everything
        path, nxt = tree_rejection(tokens, parents, np.stack([p] * 4), u, 3, 1)
        if len(path) == 1:
            assert nxt not in (4, 9, 2)
    # point mass on the second candidate: the first is always rejected, the second accepted
    pm = np.zeros(V, np.float32)
    pm[9] = 1
    for s in range(100):
        path, _ = tree_rejection(tokens, parents, np.stack([pm] + [p] * 3), _u_grid(rng, 4), 3, 1)
        assert path == [0, 2]
    # a candidate with zero target mass is never accepted
    pz = p.copy()
    pz[4] = 0
    pz /= pz.sum()
    for s in range(200):
        path, nxt = tree_rejection(tokens, parents, np.stack([pz] + [p] * 3), _u_grid(rng, 4), 3, 1)
        assert path[1:] != [1] and nxt != 4
    # no candidates: the single draw from the root's p with the final uniform
    for s in range(50):
        u = _u_grid(rng, 4)
        assert tree_rejection([0], [-1], p[None], u, 3, 1) == ([0], sample_inverse_cdf(p, u[3]))
    # a chain whose target puts all mass on each draft: every draft accepted, bonus from the
    # last row (depth limit respected)
    toks, pars = [0, 3, 7, 11], [-1, 0, 1, 2]
    rows = []
    for t in toks[1:]:
        r = np.zeros(V, np.float32)
        r[t] = 1
        rows.append(r)
    rows.append(p)
    u = _u_grid(rng, 3 * 1 + 1)
    assert tree_rejection(toks, pars, np.stack(rows), u, 1, 3) == ([0, 1, 2, 3], sample_inverse_cdf(p, u[3]))


# ------------------------------------------------ reduced draft vocabulary

def test_reduced_vocab_chain_draw_is_the_scattered_draw():
    """Drawing over the draft ids and mapping through the ascending d2t picks the same
    token as drawing over q scattered into the target vocabulary (the nonzero entries
    keep their order, so the integer prefix sums agree); the scattered q sums to 1 on
    d2t and is 0 elsewhere."""
    from oracle.numerics import probs_f32
    from oracle.step import build_sampled_chain
    rng = np.random.default_rng(21)
    V, Vd, K = 300, 71, 3
    d2t = np.sort(rng.choice(V, Vd, replace=False))
    rows = rng.normal(0, 1.5, size=(K, Vd)).astype(np.float32)
    for s in range(60):
        u = (rng.integers(0, 1 << 24, K) * 2.0 ** -24).astype(np.float32)
        toks, q = build_sampled_chain(5, rows[0], lambda d, info: [rows[d]], K, 1.0, u, False, d2t, V)
        for j in range(K):
            assert q[j][np.setdiff1d(np.arange(V), d2t)].sum() == 0
            assert abs(float(q[j][d2t].astype(np.float64).sum()) - 1) < 1e-5
            assert toks[1 + j] == sample_inverse_cdf(q[j], u[j])
            assert toks[1 + j] == int(d2t[sample_inverse_cdf(probs_f32(rows[j], 1.0), u[j])])


def test_reduced_vocab_rejection_keeps_the_target_distribution_v64():
    """A draft that can only propose 40 of 64 tokens: the first emitted token still
    follows the target p (tokens outside the draft vocabulary come from the residual
    or bonus draw)."""
    rng = np.random.default_rng(61)
    V, Vd, K = 64, 40, 1
    d2t = np.sort(rng.choice(V, Vd, replace=False))
    p = np.stack([_rand_dist(rng, V) for _ in range(K + 1)])
    qd = _rand_dist(rng, Vd)
    q = np.zeros((K, V), np.float32)
    q[0, d2t] = qd
    n = 100_000
    first = np.empty(n, dtype=np.int64)
    for s in range(n):
        u = (rng.integers(0, 1 << 24, K + 2) * 2.0 ** -24).astype(np.float32)
        d = int(d2t[sample_inverse_cdf(qd, u[K + 1])])
        n_acc, nxt = chain_rejection([d], q, p, u[:K + 1])
        first[s] = d if n_acc >= 1 else nxt
    outside = np.setdiff1d(np.arange(V), d2t)
    counts = np.bincount(first, minlength=V).astype(float)
    assert counts[outside].sum() > 0
    assert _chi2_pvalue(counts, p[0].astype(np.float64)) > 1e-3
