"""Pins of the oracle's tree verification by recursive rejection ("Speculative decoding"
textbook, box "Recursive rejection at a node with several children", its proof, and the
paragraph on the Sequoia variant).

* At a node whose k children were drawn i.i.d. from q, the emitted token follows p
  (chi-square) and some child is accepted with probability
  1 - prod_i (1 - sum_x min(R_i(x), q(x))), R_1 = p, R_{i+1} = (R_i - q)+ normalized --
  the box's formula, iterated here in NumPy -- for k = 1, 2, 4, 8.
* Children drawn without replacement (rejected tokens zeroed in q): the emitted token still
  follows p.
* The page's cell 8 uses p = (0.40, 0.25, 0.20, 0.10, 0.05): the output stays at p for every
  k and acceptance grows with k (its printed 0.55 and 0.86 depend on a q the page does not
  print: those two values are unpinned).
* A copy of the oracle that keeps R = p after a rejection fails the output-law test.
* A chain tree keeps sum_i prod_{j<=i} alpha_j drafts on average.
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
from test_oracle_accept import _draw_from, _logits_of


def _draw_children(q, k, N, r, without_replacement):
    out = np.zeros((N, k), dtype=np.int64)
    if not without_replacement:
        for i in range(k):
            out[:, i] = _draw_from(np.broadcast_to(q, (N, len(q))), r.random(N))
        return out
    w = np.broadcast_to(q, (N, len(q))).copy()
    for i in range(k):
        x = _draw_from(w / w.sum(1, keepdims=True), r.random(N))
        out[:, i] = x
        w[np.arange(N), x] = 0.0
    return out


def _one_node(p, q, k, N, seed, without_replacement, handle=None):
    """A root with k leaf children drawn from q; returns (first emitted token, J)."""
    V = len(p)
    r = np.random.default_rng(seed)
    kids = _draw_children(q, k, N, r, without_replacement)
    parents = np.array([-1] + [0] * k)
    toks = np.concatenate([np.zeros((N, 1), np.int64), kids], 1)
    tgt = np.broadcast_to(_logits_of(p), (N, k + 1, V))
    dr = np.broadcast_to(_logits_of(q), (N, k + 1, V))
    res = oracle.tree_rrs(tgt, dr, toks, parents, 1.0, seed=seed, without_replacement=without_replacement,
                          handle=handle)
    return res["out_tokens"][:, 0], res["accept_len"]


def _accept_formula(p, q, k):
    R, miss = p.copy(), 1.0
    for _ in range(k):
        a = np.minimum(R, q).sum()
        miss *= 1.0 - a
        z = np.maximum(R - q, 0.0)
        if z.sum() > 0:
            R = z / z.sum()
    return 1.0 - miss


P_CELL8 = np.array([0.40, 0.25, 0.20, 0.10, 0.05])
Q_CELL8 = np.array([0.15, 0.45, 0.15, 0.20, 0.05])     # not printed on the page: a stand-in


@pytest.mark.parametrize("k", [1, 2, 4, 8])
def test_output_law_and_acceptance_formula(k):
    N = 400_000 if k <= 4 else 200_000
    tok, J = _one_node(P_CELL8, Q_CELL8, k, N, seed=40 + k, without_replacement=False)
    assert stats.chisquare(np.bincount(tok, minlength=5), P_CELL8 * N).pvalue > 1e-4
    want = _accept_formula(P_CELL8, Q_CELL8, k)
    got = (J == 1).mean()
    assert abs(got - want) < 4 * math.sqrt(want * (1 - want) / N), (got, want)


@pytest.mark.parametrize("k", [2, 4])
def test_without_replacement_output_law(k):
    N = 300_000
    tok, J = _one_node(P_CELL8, Q_CELL8, k, N, seed=50 + k, without_replacement=True)
    assert stats.chisquare(np.bincount(tok, minlength=5), P_CELL8 * N).pvalue > 1e-4
    # at low temperature i.i.d. children repeat the draft's favourite; without replacement
    # they do not, and some child is accepted more often
    q_peaked = np.array([0.05, 0.85, 0.04, 0.03, 0.03])
    _, J_iid = _one_node(P_CELL8, q_peaked, k, N, seed=60 + k, without_replacement=False)
    _, J_wor = _one_node(P_CELL8, q_peaked, k, N, seed=60 + k, without_replacement=True)
    assert J_wor.mean() > J_iid.mean()


def test_acceptance_grows_with_children():
    rates = [(_one_node(P_CELL8, Q_CELL8, k, 100_000, seed=70 + k, without_replacement=False)[1] == 1).mean()
             for k in (1, 2, 4, 8)]
    assert all(a < b for a, b in zip(rates, rates[1:])), rates


def test_planted_residual_left_at_p_fails():
    bad = oracle.compile_variant({"for (int32_t x = 0; x < V; ++x) R[x] = fmax(0.0, R[x] - q[x]) / z;":
                                  "(void)z;"}, "rrs_no_residual")
    N = 400_000
    tok, _ = _one_node(P_CELL8, Q_CELL8, 4, N, seed=44, without_replacement=False, handle=bad)
    assert stats.chisquare(np.bincount(tok, minlength=5), P_CELL8 * N).pvalue < 1e-12


def test_chain_tree_expected_length():
    V, N, gamma = 8, 300_000, 3
    r = np.random.default_rng(45)
    tl = (r.standard_normal((gamma + 1, V)) * 1.3).astype(np.float32)
    dl = (tl + 0.8 * r.standard_normal((gamma + 1, V))).astype(np.float32)
    p, q = special.softmax(tl.astype(np.float64), -1), special.softmax(dl.astype(np.float64), -1)
    toks = np.zeros((N, gamma + 1), np.int64)
    for i in range(gamma):      # node i+1 is drafted from q at node i
        toks[:, i + 1] = _draw_from(np.broadcast_to(q[i], (N, V)), r.random(N))
    parents = np.arange(gamma + 1) - 1
    res = oracle.tree_rrs(np.broadcast_to(tl, (N, gamma + 1, V)), np.broadcast_to(dl, (N, gamma + 1, V)), toks,
                          parents, 1.0, seed=46)
    alpha = np.minimum(p[:gamma], q[:gamma]).sum(-1)
    J = res["accept_len"]
    assert abs(J.mean() - np.cumprod(alpha).sum()) < 4 * J.std() / math.sqrt(N)
