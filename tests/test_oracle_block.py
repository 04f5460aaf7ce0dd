"""Pins of the oracle's block verification ("Speculative Decoding: The Art of Guessing
Well", section "Block verification").

* The section's toy: p(a) = 1/3, p(b) = 2/3, q(a) = 2/3, q(b) = 1/3 at every position,
  gamma = 2: block verification keeps 11/9 tokens per round, token-wise 10/9 (the values the
  page prints), on the same drafts.
* Lossless: the first emitted token follows p on the toy, and the first two emitted tokens
  of a round over two bigram models follow the target's two-token law (chi-square over 10^6
  sequences); a copy of the oracle that draws the next token from p instead of the residual
  (w_n p - q)+ fails the same test.
* With one draft the rule is speculative sampling: same uniforms, same decisions.
* p = q keeps every draft; on random rows block verification keeps at least as many tokens
  as the token-wise rule on average (the section's optimality claim).
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
from conftest import read_golden
from test_oracle_accept import _bigram_models, _draw_from, _logits_of, _sm

SAMPLE = oracle.SAMPLE


def _toy():
    g = read_golden("block_toy.txt")
    p = np.array(g["p"], dtype=float)
    q = np.array(g["q"], dtype=float)
    return g, p, q, int(g["gamma"][0])


def test_toy_expected_tokens_printed_values():
    g, p, q, gamma = _toy()
    N = 400_000
    r = np.random.default_rng(20)
    x = np.stack([_draw_from(np.broadcast_to(q, (N, 2)), r.random(N)) for _ in range(gamma)], 1)
    tgt = np.broadcast_to(_logits_of(p), (N, gamma + 1, 2))
    dr = np.broadcast_to(_logits_of(q), (N, gamma, 2))
    blk = oracle.block_accept(tgt, dr, x, 1.0, seed=71)
    tok = oracle.spec_accept(SAMPLE, tgt, dr, x, 1.0, seed=71)
    for res, key in ((blk, "block"), (tok, "tokenwise")):
        want = int(g[key + "_EJ_num"][0]) / int(g[key + "_EJ_den"][0])
        J = res["accept_len"]
        assert abs(J.mean() - want) < 4 * J.std() / math.sqrt(N), (key, J.mean(), want)
    counts = np.bincount(blk["out_tokens"][:, 0], minlength=2)
    assert stats.chisquare(counts, p * N).pvalue > 1e-4


def _bigram_two_tokens_block(handle, N, seed, s0=0, gamma=2):
    """Two bigram models over six tokens, drafts conditioned on the drafts before them; the
    first two emitted tokens of each sequence (a second round when the first emits one)."""
    tl, dl = _bigram_models(seed)
    V = tl.shape[0]
    r = np.random.default_rng(seed + 100)
    qd = _sm(dl)
    x = np.zeros((N, gamma), dtype=np.int64)
    prev = np.full(N, s0)
    for i in range(gamma):
        x[:, i] = _draw_from(qd[prev], r.random(N))
        prev = x[:, i]
    ctx = np.concatenate([np.full((N, 1), s0), x], axis=1)
    res = oracle.block_accept(tl[ctx], dl[ctx[:, :gamma]], x, 1.0, seed=seed, step=0, handle=handle)
    J, out = res["accept_len"], res["out_tokens"]
    t1, t2 = out[:, 0].copy(), out[:, 1].copy()
    need = J == 0
    m = int(need.sum())
    if m:
        y = t1[need]
        x2 = np.zeros((m, gamma), dtype=np.int64)
        prev = y
        for i in range(gamma):
            x2[:, i] = _draw_from(qd[prev], r.random(m))
            prev = x2[:, i]
        ctx2 = np.concatenate([y[:, None], x2], axis=1)
        res2 = oracle.block_accept(tl[ctx2], dl[ctx2[:, :gamma]], x2, 1.0, seed=seed, step=1, handle=handle)
        t2[need] = res2["out_tokens"][:, 0]
    exact = np.outer(_sm(tl[s0]), np.ones(V)) * _sm(tl)
    counts = np.zeros((V, V))
    np.add.at(counts, (t1, t2), 1)
    return counts, exact * N


def test_bigram_two_token_law_chi_square():
    counts, expected = _bigram_two_tokens_block(None, 1_000_000, seed=22)
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert stats.chi2.sf(chi2, df=35) > 1e-4, chi2


def test_planted_draw_from_p_fails_chi_square():
    bad = oracle.compile_variant({"q[x] = fmax(0.0, w[n] * p[x] - q[x]);": "q[x] = p[x];"}, "block_from_p")
    counts, expected = _bigram_two_tokens_block(bad, 1_000_000, seed=22)
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert stats.chi2.sf(chi2, df=35) < 1e-12, chi2


def test_one_draft_is_speculative_sampling():
    r = np.random.default_rng(23)
    B, V = 3000, 40
    tgt = (r.standard_normal((B, 2, V)) * 2).astype(np.float32)
    dr = (tgt[:, :1] + r.standard_normal((B, 1, V))).astype(np.float32)
    x = np.array([_draw_from(_sm(dr[b, 0], 0.9)[None], r.random(1))[0] for b in range(B)]).reshape(B, 1)
    blk = oracle.block_accept(tgt, dr, x, 0.9, seed=5, step=2)
    tok = oracle.spec_accept(SAMPLE, tgt, dr, x, 0.9, seed=5, step=2)
    assert np.array_equal(blk["accept_len"], tok["accept_len"])
    assert np.array_equal(blk["out_tokens"], tok["out_tokens"])


def test_equal_distributions_keep_every_draft():
    r = np.random.default_rng(24)
    B, gamma, V = 500, 4, 30
    tgt = r.standard_normal((B, gamma + 1, V)).astype(np.float32)
    x = r.integers(0, V, (B, gamma))
    res = oracle.block_accept(tgt, tgt[:, :gamma].copy(), x, 0.9, seed=4)
    assert np.all(res["accept_len"] == gamma) and np.all(res["weights"] == 1.0)


def test_block_keeps_at_least_as_many_tokens_as_tokenwise():
    V, N, gamma = 8, 300_000, 4
    r = np.random.default_rng(25)
    tgt1 = (r.standard_normal((gamma + 1, V)) * 1.3).astype(np.float32)
    dr1 = (tgt1[:gamma] + 0.9 * r.standard_normal((gamma, V))).astype(np.float32)
    x = np.stack([_draw_from(np.broadcast_to(_sm(dr1[i]), (N, V)), r.random(N)) for i in range(gamma)], 1)
    tgt = np.broadcast_to(tgt1, (N, gamma + 1, V))
    dr = np.broadcast_to(dr1, (N, gamma, V))
    blk = oracle.block_accept(tgt, dr, x, 1.0, seed=41)["accept_len"]
    tok = oracle.spec_accept(SAMPLE, tgt, dr, x, 1.0, seed=41)["accept_len"]
    se = math.sqrt((blk.var() + tok.var()) / N)
    assert blk.mean() > tok.mean() - 3 * se, (blk.mean(), tok.mean())
    # the first emitted token still follows p_1
    counts = np.bincount(oracle.block_accept(tgt, dr, x, 1.0, seed=41)["out_tokens"][:, 0], minlength=V)
    assert stats.chisquare(counts, special.softmax(tgt1[0].astype(np.float64)) * N).pvalue > 1e-4
