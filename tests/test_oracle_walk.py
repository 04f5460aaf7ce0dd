"""Pins of the oracle's tree walk.

Greedy: brute force over all nodes (the accepted node is the deepest one whose
every path token is its parent's argmax and the first such sibling), and a chain
tree equals greedy acceptance on the same rows.  Sampling: the walk accepts
node v with probability prod over v's path of p_parent(token) (the tree
acceptance of the astralord page, section "Token trees"), checked by Monte
Carlo; the first emitted token follows the root's distribution.
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
import synth

GREEDY, SAMPLE = oracle.GREEDY, oracle.SAMPLE


def _sm(lg, tau):
    return special.softmax(np.asarray(lg, dtype=np.float64) / float(np.float32(tau)), axis=-1)


def _path(parents, v):
    out = []
    while v >= 0:
        out.append(v)
        v = parents[v]
    return out[::-1]


def _greedy_brute(logits, tokens, parents):
    n = len(parents)
    z = np.argmax(logits, axis=-1)
    good = np.zeros(n, dtype=bool)
    good[0] = True
    for v in range(1, n):
        p = parents[v]
        first = min(c for c in range(1, n) if parents[c] == p and tokens[c] == tokens[v])
        good[v] = good[p] and tokens[v] == z[p] and first == v
    deepest = max((v for v in range(n) if good[v]), key=lambda v: len(_path(parents, v)))
    path = _path(parents, deepest)
    return path, [tokens[u] for u in path[1:]] + [int(z[deepest])]


@pytest.mark.parametrize("seed,n,V,branch", [(0, 12, 16, 0.5), (1, 65, 50, 0.8), (2, 200, 30, 0.9),
                                              (3, 40, 8, 0.3)])
def test_greedy_walk_brute_force(seed, n, V, branch):
    parents = synth.random_tree(seed, n, branch_p=branch)
    B = 64
    lg = synth.tree_logits(seed, B, n, V, 3.0)
    toks = synth.node_tokens(seed, lg, parents)
    if seed == 3:
        toks[:, 5] = toks[:, 4]            # duplicate sibling tokens: the first index wins
    res = oracle.tree_walk(GREEDY, lg, toks, parents, 1.0, seed=0)
    depths = []
    for b in range(B):
        path, emitted = _greedy_brute(lg[b], toks[b], parents)
        J = len(path) - 1
        depths.append(J)
        assert res["accept_len"][b] == J
        assert list(res["path"][b, :J + 1]) == path
        assert list(res["out_tokens"][b, :J + 1]) == emitted
    assert max(depths) >= 2                # the walks do descend


def test_chain_tree_equals_greedy_accept():
    r = np.random.default_rng(3)
    B, gamma, V = 200, 5, 20
    tgt = r.standard_normal((B, gamma + 1, V)).astype(np.float32)
    z = np.argmax(tgt, -1)
    x = np.where(r.random((B, gamma)) < 0.75, z[:, :gamma], r.integers(0, V, (B, gamma)))
    parents = np.arange(gamma + 1) - 1
    toks = np.concatenate([np.zeros((B, 1), dtype=np.int64), x], axis=1)
    w = oracle.tree_walk(GREEDY, tgt, toks, parents, 1.0, seed=0)
    a = oracle.spec_accept(GREEDY, tgt, None, x, 1.0, seed=0)
    assert np.array_equal(w["accept_len"], a["accept_len"])
    assert np.array_equal(w["out_tokens"], a["out_tokens"])


def test_sampling_walk_node_acceptance_closed_form():
    n, V, tau = 15, 6, 0.7
    parents = synth.random_tree(7, n, branch_p=0.6)
    lg1 = synth.tree_logits(7, 1, n, V, 1.0)
    toks1 = synth.node_tokens(7, lg1, parents)
    N = 300_000
    lg = np.broadcast_to(lg1, (N, n, V))
    toks = np.broadcast_to(toks1, (N, n))
    res = oracle.tree_walk(SAMPLE, lg, toks, parents, tau, seed=5)
    p = _sm(lg1[0], tau)
    visits = np.zeros(n)
    for d in range(1, res["path"].shape[1]):
        col = res["path"][:, d]
        np.add.at(visits, col[col >= 0], 1)
    for v in range(1, n):
        pr = math.prod(p[parents[u], toks1[0, u]] for u in _path(parents, v)[1:])
        sd = math.sqrt(pr * (1 - pr) / N)
        assert abs(visits[v] / N - pr) < 4 * sd + 1e-12, (v, visits[v] / N, pr)
    # tree acceptance: E[J] = sum over drafted nodes of Pr(path accepted)
    want = sum(math.prod(p[parents[u], toks1[0, u]] for u in _path(parents, v)[1:]) for v in range(1, n))
    J = res["accept_len"]
    assert abs(J.mean() - want) < 4 * J.std() / math.sqrt(N)
    # the first emitted token is a draw from the root's distribution
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    assert stats.chisquare(counts, p[0] * N).pvalue > 1e-4


def test_walk_uses_depth_indexed_uniforms():
    n, V, tau, seed = 9, 40, 0.9, 13
    parents = np.array([-1, 0, 0, 1, 1, 2, 3, 3, 6])
    lg = synth.tree_logits(2, 8, n, V, 3.0)
    toks = synth.node_tokens(2, lg, parents)
    res = oracle.tree_walk(SAMPLE, lg, toks, parents, tau, seed=seed, stream_ids=np.arange(8) + 100)
    for b in range(8):
        J = res["accept_len"][b]
        for d in range(J + 1):
            v = res["path"][b, d]
            p = _sm(lg[b, v], tau)
            u = oracle.uniform(seed, d, 0, 100 + b, oracle.TAG_WALK)
            y = int(np.searchsorted(np.cumsum(p), u * p.sum(), side="right"))
            if res["flags"][b]:
                continue
            if d < J:
                assert toks[b, res["path"][b, d + 1]] == y
            else:
                assert res["out_tokens"][b, J] == y


def test_walk_rejects_too_deep_tree():
    parents = np.arange(4) - 1
    lg = np.zeros((1, 4, 3), dtype=np.float32)
    lg[0, :, 1] = 5.0
    toks = np.ones((1, 4), dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.tree_walk(GREEDY, lg, toks, parents, 1.0, seed=0, max_depth=2)
    ok = oracle.tree_walk(GREEDY, lg, toks, parents, 1.0, seed=0, max_depth=3)
    assert ok["accept_len"][0] == 3 and list(ok["path"][0]) == [0, 1, 2, 3]
