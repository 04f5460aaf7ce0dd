"""Pins of the oracle's token-tree mask and of the synthetic tree builders."""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def test_page_example_mask_and_depth():
    g = read_golden("tree_example.txt")
    parents = [int(x) for x in g["parents"]]
    want_mask = np.array(g["mask"], dtype=int).astype(bool)
    want_depth = np.array([int(x) for x in g["depth"]])
    P = 7
    bits, depth, pos = oracle.tree_mask(parents, P)
    dense = oracle.dense_mask(bits, len(parents), P)
    assert np.array_equal(dense[:, P:], want_mask)
    assert dense[:, :P].all()
    assert np.array_equal(depth, want_depth)
    assert np.array_equal(pos, P + want_depth)


@pytest.mark.parametrize("n,P", [(1, 0), (5, 3), (33, 10), (70, 0)])
def test_chain_is_bottom_right_causal(n, P):
    parents = np.arange(n) - 1
    bits, depth, pos = oracle.tree_mask(parents, P)
    dense = oracle.dense_mask(bits, n, P)
    want = np.tril(np.ones((n, P + n), dtype=bool), k=P)      # bottom-right aligned causal
    assert np.array_equal(dense, want)
    assert np.array_equal(depth, np.arange(n))


def _closure_mask(parents):
    """Independent construction: reachability by repeated boolean products of (A + I)."""
    n = len(parents)
    A = np.eye(n, dtype=np.int64)
    for i, p in enumerate(parents):
        if p >= 0:
            A[i, p] = 1
    R = A.copy()
    for _ in range(int(math.ceil(math.log2(max(n, 2)))) + 1):
        R = ((R @ R) > 0).astype(np.int64)
    return R.astype(bool)


@pytest.mark.parametrize("seed,n", [(0, 10), (1, 65), (2, 200), (3, 513)])
def test_random_tree_matches_transitive_closure(seed, n):
    parents = synth.random_tree(seed, n, branch_p=0.6)
    if seed == 3:
        parents[5] = -1                    # a forest: a second node following the prefix
    bits, depth, _ = oracle.tree_mask(parents, 0)
    dense = oracle.dense_mask(bits, n, 0)
    assert np.array_equal(dense, _closure_mask(parents))
    assert np.array_equal(depth, dense.sum(axis=1) - 1)     # ancestors = visible nodes minus self


@pytest.mark.parametrize("bad", [[0], [-1, 1], [-1, 0, 5], [-2]])
def test_bad_parents_rejected(bad):
    with pytest.raises(ValueError):
        oracle.tree_mask(bad, 4)


def test_cartesian_counts_from_page():
    g = read_golden("cartesian_counts.txt")
    K, s = int(g["K"][0]), int(g["s"][0])
    parents, paths = synth.tree_from_rank_paths(synth.cartesian_paths(K, s))
    n_drafted = len(parents) - 1
    assert n_drafted == int(g["tokens"][0])
    has_child = np.zeros(len(parents), dtype=bool)
    has_child[parents[parents >= 0]] = True
    assert int((~has_child).sum()) == int(g["paths"][0])
    _, depth, _ = oracle.tree_mask(parents, 0)
    assert [int((depth == d).sum()) for d in range(K + 1)] == [1, 8, 64, 512, 4096]


@pytest.mark.parametrize("s", [(3, 2, 4), (2, 5), (1, 1, 1, 1), (6,)])
def test_cartesian_count_formula(s):
    paths = [p for m in range(1, len(s) + 1) for p in itertools.product(*[range(1, x + 1) for x in s[:m]])]
    parents, _ = synth.tree_from_rank_paths(paths)
    want = sum(math.prod(s[: i + 1]) for i in range(len(s)))     # sum_i prod_{j<=i} s_j
    assert len(parents) - 1 == want


def test_medusa_greedy_equals_top_scores_and_is_closed():
    chosen = synth.medusa_greedy_paths(64, 4, 10)
    assert len(chosen) == 64
    assert len(set(chosen)) == 64
    # brute force: sort every candidate path by (score descending, rank path ascending)
    cands = [p for m in range(1, 5) for p in itertools.product(range(1, 11), repeat=m)]

    def score(p):
        return math.prod(synth.medusa_accuracy(k + 1, i) for k, i in enumerate(p))

    # exact ordering key: score = 0.7^A 0.6^B, larger score <=> smaller A ln(1/0.7) + B ln(1/0.6)
    def key(p):
        A = len(p) * (len(p) + 1) // 2
        Bx = sum(i - 1 for i in p)
        return (A * math.log(1 / 0.7) + Bx * math.log(1 / 0.6), p)

    top = sorted(cands, key=key)[:64]
    assert set(top) == set(chosen)
    for p in chosen:                                   # ancestor-closed
        assert len(p) == 1 or p[:-1] in set(chosen)
    # the 15-way tie at the cut does not change the objective: sum of path scores
    assert abs(sum(score(p) for p in chosen) - 4.6158) < 1e-4
    depth_hist = [sum(1 for p in chosen if len(p) == d) for d in range(1, 5)]
    assert depth_hist == [8, 28, 23, 5]


def test_medusa_tree_node_list():
    parents, paths = synth.build_tree(synth.WORKLOADS[3])
    assert len(parents) == 65 and parents[0] == -1
    d3 = sorted("".join(map(str, p)) for p in paths if len(p) == 3)
    assert d3 == sorted("111 112 113 114 115 121 122 123 124 131 132 133 141 211 212 213 221 222 "
                        "231 311 312 321 411".split())
    d4 = sorted("".join(map(str, p)) for p in paths if len(p) == 4)
    assert d4 == ["1111", "1112", "1121", "1211", "2111"]
