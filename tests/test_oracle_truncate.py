"""Pins of the oracle's truncation (oracle.truncate: top-k, then top-p).

The pages ask that p and q be the distributions each model really samples from, after
temperature and truncation such as top-p ("Speculative decoding", section "When the target
samples, keep a guess with probability p over q"; box "The speculative sampling rule", case
"A processed target"), and warn that a q taken before the draft's own top-p cut makes the
ratio wrong (box "Four ways to lose exactness without noticing").  They do not define top-k
or top-p themselves; the oracle takes the usual definitions (top-k: the k most likely
tokens; top-p: the smallest set of most likely tokens whose probability reaches p, of the
top-k renormalized distribution when both are on; ties by the lower token id).

Pinned here against things other than the oracle's own loops: a library partial sort
(top-k on distinct logits), brute force over every subset of a small vocabulary (top-p is
the smallest set reaching the mass), hand-worked small rows, invariants (temperature as a
logit scale, per-row values, identity when off), and the pages' warning, by chi-square over
many rounds of speculative sampling.
"""
import itertools

import numpy as np
import pytest
from scipy import special, stats

import oracle
import synth

SAMPLE = oracle.SAMPLE


def kept_ids(out_row):
    return set(np.flatnonzero(out_row > -np.inf).tolist())


@pytest.mark.parametrize("k,p", [(0, 1.0), (-3, 1.0), (50, 1.0), (80, 1.0), (0, 1.5), (0, float("nan"))])
def test_identity_when_off(k, p):
    lg = synth.logit_rows(1, 4, 50, 4.0)
    r = oracle.truncate(lg, 0.7, top_k=k, top_p=p)
    assert np.array_equal(r["out"], lg)
    assert np.all(r["kept"] == 50) and not r["flags"].any()


@pytest.mark.parametrize("k", [1, 2, 17, 500, 999])
def test_top_k_is_the_k_largest(k):
    lg = synth.logit_rows(2, 3, 1000, 9.0)
    for row, out in zip(lg, oracle.truncate(lg, 1.0, top_k=k)["out"]):
        assert len(np.unique(row)) == row.size  # distinct logits: the k largest are unique
        assert kept_ids(out) == set(np.argpartition(-row, k - 1)[:k].tolist())
        keep = out > -np.inf
        assert np.array_equal(out[keep], row[keep])


def test_top_k_ties_go_to_the_lower_token_id():
    row = np.array([[1.0, 3.0, 3.0, 2.0, 3.0]], np.float32)
    want = {1: {1}, 2: {1, 2}, 3: {1, 2, 4}, 4: {1, 2, 3, 4}}
    for k, ids in want.items():
        assert kept_ids(oracle.truncate(row, 1.0, top_k=k)["out"][0]) == ids
    # -0 and +0 are one logit
    for row in ([0.0, -0.0, -1.0], [-0.0, 0.0, -1.0]):
        assert kept_ids(oracle.truncate(np.array([row], np.float32), 1.0, top_k=1)["out"][0]) == {0}


def test_top_p_worked_rows():
    # probabilities 0.5, 0.3, 0.2 (logits their logs, T = 1): prefix masses 0.5, 0.8, 1.0
    row = np.log(np.array([[0.2, 0.5, 0.3]])).astype(np.float32)
    for p, n, ids in [(0.45, 1, {1}), (0.55, 2, {1, 2}), (0.79, 2, {1, 2}), (0.81, 3, {0, 1, 2}),
                      (0.0, 1, {1}), (-1.0, 1, {1})]:
        r = oracle.truncate(row, 1.0, top_p=p)
        assert r["kept"][0] == n and kept_ids(r["out"][0]) == ids, p
        assert r["flags"][0] == 0, p
    # a cut that lands exactly on a prefix mass is flagged (other rounding could move it by a
    # token): four equal logits, prefix masses 1/4, 1/2, 3/4 exactly
    r = oracle.truncate(np.zeros((1, 4), np.float32), 1.0, top_p=0.5)
    assert r["flags"][0] == 1 and kept_ids(r["out"][0]) == {0, 1}


def test_top_p_is_the_smallest_set_reaching_the_mass():
    """Brute force over all subsets of 8 tokens: top-p keeps as few tokens as any set whose
    mass reaches top_p, and of those sets the heaviest."""
    lg = synth.logit_rows(3, 30, 8, 2.0)
    checked = 0
    for T in (0.5, 1.0, 2.0):
        for p in (0.1, 0.3, 0.5, 0.7, 0.9, 0.97):
            r = oracle.truncate(lg, T, top_p=p)
            for i, row in enumerate(lg):
                if r["flags"][i]:
                    continue
                pr = special.softmax(row.astype(np.float64) / T)
                best = None
                for m in range(1, 9):
                    sets = [s for s in itertools.combinations(range(8), m) if pr[list(s)].sum() >= p]
                    if sets:
                        best = (m, max(sets, key=lambda s: pr[list(s)].sum()))
                        break
                assert r["kept"][i] == best[0]
                assert kept_ids(r["out"][i]) == set(best[1])
                checked += 1
    assert checked > 500


def test_top_p_is_taken_over_the_top_k_set():
    # probabilities 0.4, 0.3, 0.2, 0.1: top-2 renormalized is (4/7, 3/7); 4/7 > 0.55, while
    # over the whole row 0.4 < 0.55 <= 0.7
    row = np.log(np.array([[0.1, 0.3, 0.4, 0.2]])).astype(np.float32)
    assert kept_ids(oracle.truncate(row, 1.0, top_k=2, top_p=0.55)["out"][0]) == {2}
    assert kept_ids(oracle.truncate(row, 1.0, top_k=0, top_p=0.55)["out"][0]) == {1, 2}
    assert kept_ids(oracle.truncate(row, 1.0, top_k=3, top_p=0.999)["out"][0]) == {1, 2, 3}


def test_temperature_is_a_logit_scale():
    """top-p at temperature T keeps what top-p at T = 1 keeps on logits / T (T a power of
    two, so the scaled logits are exact); top-k does not depend on T."""
    lg = synth.logit_rows(4, 8, 300, 4.0)
    for T in (0.25, 0.5, 2.0, 4.0):
        a = oracle.truncate(lg, T, top_k=100, top_p=0.8)
        b = oracle.truncate(lg / np.float32(T), 1.0, top_k=100, top_p=0.8)
        assert np.array_equal(a["kept"], b["kept"]) and np.array_equal(a["flags"], b["flags"])
        assert np.array_equal(a["out"] > -np.inf, b["out"] > -np.inf)
        k = oracle.truncate(lg, T, top_k=37)
        assert np.array_equal(k["out"], oracle.truncate(lg, 1.0, top_k=37)["out"])


def test_per_row_values_override_the_scalars():
    lg = synth.logit_rows(5, 7, 120, 3.0)
    ks = np.array([0, 1, 5, 119, 120, 60, -2], np.int32)
    ps = np.array([1.0, 0.5, 0.9, 0.2, 0.95, 2.0, 0.0], np.float32)
    r = oracle.truncate(lg, 0.8, top_k=3, top_p=0.1, top_k_rows=ks, top_p_rows=ps)
    for i in range(7):
        s = oracle.truncate(lg[i:i + 1], 0.8, top_k=int(ks[i]), top_p=float(ps[i]))
        assert np.array_equal(r["out"][i], s["out"][0]) and r["kept"][i] == s["kept"][0]


def test_rows_of_minus_infinity():
    lg = np.full((2, 9), -np.inf, np.float32)
    lg[1, [2, 5]] = [0.5, 1.5]
    r = oracle.truncate(lg, 1.0, top_p=0.5)
    assert r["kept"][0] == 9 and np.all(r["out"][0] == -np.inf)   # nothing to truncate
    assert r["kept"][1] == 1 and kept_ids(r["out"][1]) == {5}
    assert oracle.truncate(lg, 1.0, top_k=2)["kept"].tolist() == [2, 2]


# --------------------------------------------------------------------------------------
# The pages' warning: the q in the ratio must be the draft's truncated distribution.
P_TOY = np.array([0.30, 0.25, 0.20, 0.12, 0.08, 0.05])
Q_TOY = np.array([0.10, 0.15, 0.30, 0.25, 0.12, 0.08])


def _round(target_row, draft_row, x, seed):
    N = x.shape[0]
    target = np.broadcast_to(target_row, (N, 2, 6)).astype(np.float32)
    draft = np.broadcast_to(draft_row, (N, 1, 6)).astype(np.float32)
    r = oracle.spec_accept(SAMPLE, target, draft, x, 1.0, seed=seed, step=0)
    return np.bincount(r["out_tokens"][:, 0], minlength=6)


def test_ratio_needs_the_drafts_own_truncated_q():
    N = 200_000
    lp, lq = np.log(P_TOY).astype(np.float32), np.log(Q_TOY).astype(np.float32)
    tp = oracle.truncate(lp[None], 1.0, top_k=4, top_p=0.8)
    tq = oracle.truncate(lq[None], 1.0, top_k=4, top_p=0.8)
    assert tp["kept"][0] == 3 and tq["kept"][0] == 3 and not (tp["flags"][0] or tq["flags"][0])
    p_t = special.softmax(tp["out"][0].astype(np.float64))
    q_t = special.softmax(tq["out"][0].astype(np.float64))
    assert set(np.flatnonzero(p_t).tolist()) == {0, 1, 2} and set(np.flatnonzero(q_t).tolist()) == {1, 2, 3}
    x = np.random.default_rng(8).choice(6, size=N, p=q_t).astype(np.int32).reshape(N, 1)

    def fits(counts, law):
        s = law > 0
        if np.any(counts[~s]):
            return 0.0
        return stats.chisquare(counts[s], law[s] * N).pvalue

    # processed target and the draft's own truncated q: the output law is the processed p
    good = _round(tp["out"][0], tq["out"][0], x, 31)
    assert fits(good, p_t) > 1e-4, good / N
    # the draft's logits before its cut in the ratio: not p any more
    bad_q = _round(tp["out"][0], lq, x, 31)
    assert fits(bad_q, p_t) < 1e-12, bad_q / N
    # an unprocessed target: the output follows the untruncated p instead
    raw_p = _round(lp, tq["out"][0], x, 31)
    assert fits(raw_p, P_TOY) > 1e-4 and fits(raw_p, p_t) < 1e-12
