"""Pins of the oracle's Gumbel-coupled verification ("Speculative Decoding: The Art of
Guessing Well", section "Sampling with shared noise").

* The noise: every target sample equals a NumPy recomputation with NumPy's own Philox
  (word x mod 4 of the block with counter (x div 4, step, stream, tag + 2^32 i)) and
  argmax(l / T - log(-log u)).
* Gumbel-max samples softmax(l / T) (chi-square over 10^6 draws).
* With shared noise the first draft matches the target's sample with probability
  sum_j 1 / sum_i max(p_i/p_j, q_i/q_j) -- the section's formula -- which lies between
  (1 - TV)/(1 + TV) and 1 - TV; with independent noise it is sum_i p_i q_i.
* Drafter invariance: two drafters sharing the noise emit the same tokens (the target's
  own samples) as far as both rounds reach; temperature 0 is greedy verification.
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
from np_philox import block as np_block, word_to_uniform
from test_oracle_accept import _draw_from

GREEDY = oracle.GREEDY


def _np_gumbel_argmax(logits, tau, seed, step, stream, pos):
    V = len(logits)
    words = [int(w) for c in range((V + 3) // 4)
             for w in np_block([c, step, stream, oracle.TAG_GUMBEL + (pos << 32)], [seed, 0])]
    u = np.array([word_to_uniform(w) for w in words[:V]])
    s = logits.astype(np.float64) / float(np.float32(tau)) - np.log(-np.log(u))
    return int(np.argmax(s))


def test_noise_recomputed_with_numpy_philox():
    r = np.random.default_rng(30)
    B, rows, V = 12, 3, 37
    lg = (r.standard_normal((B, rows, V)) * 2).astype(np.float32)
    streams = (np.arange(B) * 13 + 5).astype(np.uint64)
    got, gap = oracle.gumbel_argmax(lg, 0.7, seed=99, step=4, stream_ids=streams)
    for b in range(B):
        for i in range(rows):
            assert got[b, i] == _np_gumbel_argmax(lg[b, i], 0.7, 99, 4, int(streams[b]), i)
    assert np.all(gap > 0)


def test_gumbel_max_law():
    V, N = 8, 1_000_000
    lg1 = (np.random.default_rng(31).standard_normal(V) * 1.5).astype(np.float32)
    got, _ = oracle.gumbel_argmax(np.broadcast_to(lg1, (N, 1, V)), 0.8, seed=7)
    counts = np.bincount(got[:, 0], minlength=V)
    assert stats.chisquare(counts, special.softmax(lg1.astype(np.float64) / float(np.float32(0.8))) * N).pvalue > 1e-4


def _match_formula(p, q):
    return sum(1.0 / np.maximum(p / p[j], q / q[j]).sum() for j in range(len(p)))


@pytest.mark.parametrize("scale", [0.5, 1.5])
def test_shared_noise_match_probability(scale):
    V, N, gamma = 10, 400_000, 1
    r = np.random.default_rng(32)
    tl = (r.standard_normal(V) * 1.5).astype(np.float32)
    dl = (tl + scale * r.standard_normal(V)).astype(np.float32)
    p, q = special.softmax(tl.astype(np.float64)), special.softmax(dl.astype(np.float64))
    tgt = np.broadcast_to(np.stack([tl, tl]), (N, gamma + 1, V))
    drafts, _ = oracle.gumbel_argmax(np.broadcast_to(dl, (N, 1, V)), 1.0, seed=8)   # the drafter, same noise
    res = oracle.gumbel_accept(tgt, drafts, 1.0, seed=8)
    match = res["accept_len"].mean()
    want = _match_formula(p, q)
    tv = 0.5 * np.abs(p - q).sum()
    assert (1 - tv) / (1 + tv) - 1e-12 <= want <= 1 - tv + 1e-12
    assert abs(match - want) < 4 * math.sqrt(want * (1 - want) / N), (match, want)
    # independent noise: the drafter draws from q on its own
    indep = _draw_from(np.broadcast_to(q, (N, V)), r.random(N)).reshape(N, 1)
    m2 = oracle.gumbel_accept(tgt, indep, 1.0, seed=8)["accept_len"].mean()
    w2 = float((p * q).sum())
    assert abs(m2 - w2) < 4 * math.sqrt(w2 * (1 - w2) / N), (m2, w2)


def test_drafter_invariance():
    r = np.random.default_rng(33)
    B, gamma, V = 400, 5, 50
    tl = (r.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    outs = []
    for noise in (0.3, 2.0):
        dl = (tl[:, :gamma] + noise * r.standard_normal((B, gamma, V))).astype(np.float32)
        drafts, _ = oracle.gumbel_argmax(dl, 0.9, seed=9, step=3)
        outs.append(oracle.gumbel_accept(tl, drafts, 0.9, seed=9, step=3))
    y, _ = oracle.gumbel_argmax(tl, 0.9, seed=9, step=3)      # the target's own samples
    for res in outs:
        for b in range(B):
            J = res["accept_len"][b]
            assert list(res["out_tokens"][b, :J + 1]) == list(y[b, :J + 1])
    assert outs[0]["accept_len"].mean() > outs[1]["accept_len"].mean()


def test_temperature_zero_is_greedy():
    r = np.random.default_rng(34)
    B, gamma, V = 300, 4, 20
    tl = r.standard_normal((B, gamma + 1, V)).astype(np.float32)
    z = np.argmax(tl, -1)
    x = np.where(r.random((B, gamma)) < 0.7, z[:, :gamma], r.integers(0, V, (B, gamma)))
    g = oracle.gumbel_accept(tl, x, 0.0, seed=1)
    s = oracle.spec_accept(GREEDY, tl, None, x, 1.0, seed=1)
    assert np.array_equal(g["accept_len"], s["accept_len"]) and np.array_equal(g["out_tokens"], s["out_tokens"])
