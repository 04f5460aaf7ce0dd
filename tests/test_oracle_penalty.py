"""Pins of the oracle's penalties (oracle.penalize: repetition, frequency, presence).

The pages ask that p and q be the distributions each model really samples from, after
temperature, truncation and penalties ("Speculative decoding", section "When the target
samples, keep a guess with probability p over q"), with the drafted prefix as context (box
"The speculative sampling rule", case "A processed target").  They name penalties without
defining them; the oracle takes the usual three: a token seen c > 0 times in the context has
its logit l divided by theta when positive, multiplied by theta otherwise, then lowered by
c * frequency + presence.

Pinned here: hand-worked rows; NumPy's own counting (np.unique) against the oracle's;
invariants (identity when off or with an empty context, history order, out-of-range
entries, row i = row 0 with the first i drafts appended to the history); and the pages'
rule, by chi-square on the law of two generated tokens: speculative rounds over rows
penalized with the drafted prefix reproduce sequential sampling, rows penalized without it
do not.
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle
import synth

SAMPLE = oracle.SAMPLE


def test_hand_worked_rows():
    lg = np.array([[[2.0, -1.0, 0.5, 3.0], [2.0, -1.0, 0.5, 3.0]]], np.float32)
    out = oracle.penalize(lg, history=np.array([[0, 1, 1]]), drafts=np.array([[3]]), repetition=2.0,
                          frequency=0.5, presence=0.25)
    # token 0 once: 2 / 2 - 0.5 - 0.25; token 1 twice: -1 * 2 - 1.0 - 0.25; token 2 unseen;
    # token 3 only in row 1's context (the draft before it): 3 / 2 - 0.5 - 0.25
    assert out[0, 0].tolist() == [0.25, -3.25, 0.5, 3.0]
    assert out[0, 1].tolist() == [0.25, -3.25, 0.5, 0.75]
    # repetition alone: positive logits shrink, negative ones grow in magnitude, zero stays
    z = oracle.penalize(np.array([[[4.0, -4.0, 0.0]]], np.float32), history=np.array([[0, 1, 2]]), repetition=4.0)
    assert z[0, 0].tolist() == [1.0, -16.0, 0.0]


def _numpy_penalize(lg, hist, drafts, theta, fr, pr):
    """The same definition with NumPy's own counting (np.unique), row by row (the parameters
    are fp32 values, as the library takes them)."""
    theta, fr, pr = (float(np.float32(v)) for v in (theta, fr, pr))
    B, n, V = lg.shape
    out = lg.copy()
    for b in range(B):
        for i in range(n):
            ctx = np.concatenate([hist[b], drafts[b, :min(i, drafts.shape[1])]])
            ctx = ctx[(ctx >= 0) & (ctx < V)]
            tok, cnt = np.unique(ctx, return_counts=True)
            x = lg[b, i, tok].astype(np.float64)
            r = np.where(x > 0, x / theta, x * theta)
            out[b, i, tok] = ((r - cnt * fr) - pr).astype(np.float32)
    return out


@pytest.mark.parametrize("theta,fr,pr", [(1.3, 0.0, 0.0), (1.0, 0.4, 0.0), (1.0, 0.0, 0.7), (1.2, 0.3, 0.5),
                                         (0.8, -0.2, -0.1)])
def test_counts_against_numpy(theta, fr, pr):
    B, n, V, H, g = 6, 5, 300, 80, 4
    lg = synth.logit_rows(7, B * n, V, 4.0).reshape(B, n, V)
    r = np.random.default_rng(3)
    hist = r.integers(-3, V + 3, (B, H)).astype(np.int32)   # some entries out of range
    hist[:, :20] = r.integers(0, 10, (B, 20))                # repeated tokens
    drafts = r.integers(0, 12, (B, g)).astype(np.int32)
    got = oracle.penalize(lg, history=hist, drafts=drafts, repetition=theta, frequency=fr, presence=pr)
    assert np.array_equal(got, _numpy_penalize(lg, hist, drafts, theta, fr, pr))


def test_identity_when_off_or_without_context():
    lg = synth.logit_rows(8, 12, 200, 4.0).reshape(3, 4, 200)
    hist = np.random.default_rng(1).integers(0, 200, (3, 50)).astype(np.int32)
    drafts = np.random.default_rng(2).integers(0, 200, (3, 3)).astype(np.int32)
    assert np.array_equal(oracle.penalize(lg, history=hist, drafts=drafts), lg)
    # no history: row 0 has an empty context
    out = oracle.penalize(lg, drafts=drafts, repetition=1.5, frequency=0.3, presence=0.2)
    assert np.array_equal(out[:, 0], lg[:, 0]) and not np.array_equal(out[:, 1], lg[:, 1])
    # history lengths: 0 is no history; beyond the stride is clamped to it
    out0 = oracle.penalize(lg, history=hist, hist_len=np.zeros(3, np.int32), repetition=1.5)
    assert np.array_equal(out0, lg)
    full = oracle.penalize(lg, history=hist, repetition=1.5)
    assert np.array_equal(oracle.penalize(lg, history=hist, hist_len=np.full(3, 999, np.int32), repetition=1.5), full)


def test_history_order_does_not_matter():
    lg = synth.logit_rows(9, 8, 150, 4.0).reshape(2, 4, 150)
    r = np.random.default_rng(4)
    hist = r.integers(0, 40, (2, 60)).astype(np.int32)
    drafts = r.integers(0, 40, (2, 3)).astype(np.int32)
    a = oracle.penalize(lg, history=hist, drafts=drafts, repetition=1.4, frequency=0.2, presence=0.3)
    b = oracle.penalize(lg, history=hist[:, r.permutation(60)], drafts=drafts, repetition=1.4, frequency=0.2,
                        presence=0.3)
    assert np.array_equal(a, b)


def test_row_i_has_the_first_i_drafts_as_context():
    B, g, V = 3, 5, 120
    lg = synth.logit_rows(10, B * (g + 1), V, 4.0).reshape(B, g + 1, V)
    r = np.random.default_rng(5)
    hist = r.integers(0, 30, (B, 25)).astype(np.int32)
    drafts = r.integers(0, 30, (B, g)).astype(np.int32)
    got = oracle.penalize(lg, history=hist, drafts=drafts, repetition=1.3, frequency=0.25, presence=0.1)
    for i in range(g + 1):
        h2 = np.concatenate([hist, drafts[:, :i]], axis=1)
        one = oracle.penalize(lg[:, i:i + 1], history=h2, repetition=1.3, frequency=0.25, presence=0.1)
        assert np.array_equal(got[:, i], one[:, 0]), i


# --------------------------------------------------------------------------------------
# The pages' rule: penalties applied with the drafted prefix as context keep the round exact.
LP = np.log(np.array([0.35, 0.25, 0.2, 0.12, 0.08])).astype(np.float32)
LQ = np.log(np.array([0.15, 0.3, 0.25, 0.2, 0.1])).astype(np.float32)
PEN = dict(repetition=1.5, frequency=0.6, presence=0.4)


def _soft(l):
    return special.softmax(l.astype(np.float64), axis=-1)


def _draw(r, probs):
    """One inverse-CDF draw per row of probs."""
    u = r.random(probs.shape[0])[:, None]
    return np.minimum((np.cumsum(probs, axis=1) <= u).sum(axis=1), probs.shape[1] - 1).astype(np.int32)


def _two_tokens(N, with_prefix, seed):
    """Two tokens generated by speculative rounds (gamma = 2) from a history [0]; a round that
    emits one token is followed by one draw from the target given it."""
    V = 5
    r = np.random.default_rng(seed)
    hist = np.zeros((N, 1), np.int32)
    # the drafter samples x0, x1 with its own penalized q (its context includes x0 for x1)
    q0 = _soft(oracle.penalize(LQ[None, None], history=hist[:1], **PEN)[0, 0])
    x0 = r.choice(V, size=N, p=q0).astype(np.int32)
    q1_all = np.stack([_soft(oracle.penalize(LQ[None, None], history=np.array([[0, t]], np.int32), **PEN)[0, 0])
                       for t in range(V)])
    x1 = _draw(r, q1_all[x0])
    drafts = np.stack([x0, x1], axis=1)
    target = np.broadcast_to(LP, (N, 3, V)).copy()
    draft = np.broadcast_to(LQ, (N, 2, V)).copy()
    if with_prefix:
        tp = oracle.penalize(target, history=hist, drafts=drafts, **PEN)
    else:   # every row penalized with the history only
        tp = oracle.penalize(target, history=hist, **PEN)
    dq = oracle.penalize(draft, history=hist, drafts=drafts, **PEN)
    res = oracle.spec_accept(SAMPLE, tp, dq, drafts, 1.0, seed=seed, step=0)
    y0 = res["out_tokens"][:, 0].copy()
    y1 = res["out_tokens"][:, 1].copy()
    one = res["accept_len"] == 0
    p1_all = np.stack([_soft(oracle.penalize(LP[None, None], history=np.array([[0, t]], np.int32), **PEN)[0, 0])
                       for t in range(V)])
    y1[one] = _draw(r, p1_all[y0[one]])
    return np.bincount(y0 * V + y1, minlength=V * V)


def _joint_law():
    V = 5
    p0 = _soft(oracle.penalize(LP[None, None], history=np.zeros((1, 1), np.int32), **PEN)[0, 0])
    law = np.zeros((V, V))
    for t in range(V):
        law[t] = p0[t] * _soft(oracle.penalize(LP[None, None], history=np.array([[0, t]], np.int32), **PEN)[0, 0])
    return law.reshape(-1)


def test_drafted_prefix_context_keeps_the_round_exact():
    N = 200_000
    law = _joint_law()
    good = _two_tokens(N, True, 11)
    assert stats.chisquare(good, law * N).pvalue > 1e-4, good / N
    bad = _two_tokens(N, False, 11)
    assert stats.chisquare(bad, law * N).pvalue < 1e-12, bad / N
