"""Pins of the oracle's near-threshold flags.

A decision the GPU may take differently from the fp64 oracle is one whose uniform lies
very close to its threshold: a ratio test u_i q_i(x_i) < p_i(x_i) with |u_i - p_i/q_i|
< 1e-6 (flag bit 0), or an inverse-CDF draw whose target u* Z lies within 1e-10 (in units
of probability mass) of a cumulative sum on either side of the chosen token (flag bit 1).
The GPU parity tests excuse flagged sequences, so a flag that fires too often would make
them vacuous and one that fires too rarely would let a real mismatch be excused as
rounding.

Here every flag is recomputed independently -- NumPy softmax, NumPy's own Philox for the
uniforms, the distances written out -- and compared bit for bit with the oracle's, on
inputs crafted so that the distances straddle each window (distances from a tenth of the
window to ten times it, on both sides) and on random inputs.  A copy of the oracle whose
ratio flag is forced on, and one whose draw flag is forced off, must fail the same checks
(negative controls).
"""
import numpy as np
import pytest
from scipy import special

import oracle
from np_philox import uniform as np_uniform

NEAR_RATIO = 1e-6
NEAR_DRAW = 1e-10
SAMPLE = oracle.SAMPLE
# distances from the threshold, in units of its window: half of them inside it
STEPS = [-10.0, -3.0, -1.5, -0.8, -0.4, -0.1, 0.1, 0.4, 0.8, 1.5, 3.0, 10.0]
DELTAS = [d * NEAR_RATIO for d in STEPS]
DRAW_DELTAS = [d * NEAR_DRAW for d in STEPS]


def _sm(lg, tau):
    return special.softmax(np.asarray(lg, np.float64) / float(np.float32(tau)), axis=-1)


def _cdf_flag(w, u):
    """(token, near) of the inverse-CDF draw: the smallest y with C_y > u Z; near when
    u Z is within 1e-10 of C_{y-1} or C_y (w in units of probability mass)."""
    c = np.cumsum(w)
    z = c[-1]
    target = u * z
    y = int(np.searchsorted(c, target, side="right"))
    if y >= len(w):  # rounding left the total at or below u Z: the last token with mass
        y = int(np.nonzero(w > 0)[0][-1])
        prev = c[-1]
    else:
        prev = c[y - 1] if y > 0 else 0.0
    return y, bool(abs(target - prev) < NEAR_DRAW or abs(c[y] - target) < NEAR_DRAW)


def accept_expected(tgt, dr, toks, tau, seed, step, streams):
    """Decisions and flags of speculative sampling, recomputed in NumPy."""
    B, g1, V = tgt.shape
    gamma = g1 - 1
    p, q = _sm(tgt, tau), _sm(dr, tau)
    J = np.zeros(B, np.int64)
    y = np.zeros(B, np.int64)
    flags = np.zeros(B, np.int64)
    for b in range(B):
        j = 0
        while j < gamma:
            u = np_uniform(seed, j, step, int(streams[b]), oracle.TAG_ACCEPT)
            px, qx = p[b, j, toks[b, j]], q[b, j, toks[b, j]]
            if qx > 0 and abs(u - px / qx) < NEAR_RATIO:
                flags[b] |= 1
            if not (u * qx < px):
                break
            j += 1
        J[b] = j
        w = np.maximum(p[b, j] - q[b, j], 0.0) if j < gamma else p[b, gamma]
        if not (w.sum() > 0):
            w = p[b, j]
        ustar = np_uniform(seed, gamma, step, int(streams[b]), oracle.TAG_ACCEPT)
        y[b], near = _cdf_flag(w, ustar)
        flags[b] |= 2 if near else 0
    return J, y, flags


def _logit2(p0):
    """fp32 logits (a, 0) of the two-token distribution (p0, 1 - p0)."""
    return np.array([np.log(p0 / (1.0 - p0)), 0.0], np.float32)


def _logit3(p0):
    """fp32 logits (a, b, 0) whose softmax puts p0 on token 0 to within a few 1e-12: a is set
    slightly high and the small third weight e^b (b near -11) takes up the difference, so
    rounding b to fp32 moves p0 by only ~1e-12 (rounding a alone would move it by ~1e-8)."""
    a = np.float32(np.log(p0 / (1.0 - p0)) + 2e-5)
    eb = np.exp(np.float64(a)) * (1.0 - p0) / p0 - 1.0
    return np.array([a, np.log(eb), 0.0], np.float32)


def crafted_ratio_inputs(seed, step, streams, deltas):
    """gamma = 1, V = 2, draft q = (1/2, 1/2) with token 0 drafted, target p(0) set so that
    p(0)/q(0) = u_0 + delta: the ratio test sits delta away from its threshold."""
    B = len(streams)
    tgt = np.zeros((B, 2, 2), np.float32)
    dr = np.zeros((B, 1, 2), np.float32)
    for b in range(B):
        u0 = np_uniform(seed, 0, step, int(streams[b]), oracle.TAG_ACCEPT)
        tgt[b, 0] = _logit2(0.5 * (u0 + deltas[b % len(deltas)]))
    return tgt, dr, np.zeros((B, 1), np.int32)


def crafted_draw_inputs(seed, step, streams, deltas):
    """gamma = 1, V = 3, target row 0 = draft row 0 (always accepted), bonus row p with
    p(0) = u* + delta: the extra draw sits delta away from the boundary C_0."""
    B = len(streams)
    tgt = np.zeros((B, 2, 3), np.float32)
    dr = np.zeros((B, 1, 3), np.float32)
    for b in range(B):
        us = np_uniform(seed, 1, step, int(streams[b]), oracle.TAG_ACCEPT)
        tgt[b, 1] = _logit3(us + deltas[b % len(deltas)])
    return tgt, dr, np.zeros((B, 1), np.int32)


def check_accept(handle, tgt, dr, toks, tau, seed, step, streams):
    res = oracle.spec_accept(SAMPLE, tgt, dr, toks, tau, seed=seed, step=step, stream_ids=streams, handle=handle)
    J, y, flags = accept_expected(tgt, dr, toks, tau, seed, step, streams)
    assert np.array_equal(res["flags"], flags), (res["flags"], flags)
    assert np.array_equal(res["accept_len"], J)
    assert np.array_equal(res["out_tokens"][np.arange(len(J)), J], y)
    return flags


def _streams(n, off=0):
    return (np.arange(n, dtype=np.uint64) * 7919 + 13 + off).astype(np.uint64)


def run_accept_pins(handle):
    """Every check of this file on one oracle build; returns the flag counts seen."""
    seen = {}
    st = _streams(48)
    f = check_accept(handle, *crafted_ratio_inputs(101, 3, st, DELTAS), 1.0, 101, 3, st)
    seen["ratio"] = int(((f & 1) != 0).sum())
    f = check_accept(handle, *crafted_draw_inputs(102, 5, st, DRAW_DELTAS), 1.0, 102, 5, st)
    seen["draw"] = int(((f & 2) != 0).sum())
    r = np.random.default_rng(3)
    B, gamma, V = 64, 4, 300
    tgt = (r.standard_normal((B, gamma + 1, V)) * 1.7).astype(np.float32)
    dr = (tgt[:, :gamma] + r.standard_normal((B, gamma, V))).astype(np.float32)
    toks = r.integers(0, V, (B, gamma)).astype(np.int32)
    for step in range(3):
        f = check_accept(handle, tgt, dr, toks, 0.8, 7, step, _streams(B, step))
        seen["random"] = seen.get("random", 0) + int((f != 0).sum())
    return seen


def test_accept_flags_recomputed():
    seen = run_accept_pins(None)
    # 6 of the 12 crafted distances lie inside their window: 4 sequences each of the 48
    assert seen["ratio"] == 24 and seen["draw"] == 24, seen
    assert seen["random"] == 0, seen


def test_forced_ratio_flag_fails_the_pins():
    """Negative control: a copy of the oracle whose ratio flag fires on every evaluated test."""
    bad = oracle.compile_variant({"if (qx > 0.0 && fabs(u - px / qx) < ORC_NEAR_RATIO) fl |= 1;": "fl |= 1;"},
                                 "ratio_flag_on")
    with pytest.raises(AssertionError):
        run_accept_pins(bad)


def test_dropped_draw_flag_fails_the_pins():
    """Negative control: a copy of the oracle whose draw flag never fires."""
    bad = oracle.compile_variant({"if (near) fl |= 2;\n        for (int32_t i = 0; i < J; ++i)":
                                  "(void)near;\n        for (int32_t i = 0; i < J; ++i)"}, "draw_flag_off")
    with pytest.raises(AssertionError):
        run_accept_pins(bad)


# --------------------------------------------------------------------------- #
def walk_expected(lg, toks, parents, tau, seed, step, streams, max_depth):
    """Sampled walk and its draw flags, recomputed in NumPy."""
    B, n, V = lg.shape
    p = _sm(lg, tau)
    out = []
    for b in range(B):
        v, d, fl, path = 0, 0, 0, [0]
        while True:
            u = np_uniform(seed, d, step, int(streams[b]), oracle.TAG_WALK)
            y, near = _cdf_flag(p[b, v], u)
            fl |= 2 if near else 0
            kids = [c for c in range(v + 1, n) if parents[c] == v and toks[b, c] == y]
            if not kids or d + 1 > max_depth:
                break
            v = kids[0]
            d += 1
            path.append(v)
        out.append((d, path, y, fl))
    return out


def check_walk(handle, lg, toks, parents, tau, seed, step, streams):
    max_depth = int(oracle.tree_mask(parents, 0)[1].max())
    res = oracle.tree_walk(SAMPLE, lg, toks, parents, tau, seed=seed, step=step, stream_ids=streams,
                           max_depth=max_depth, handle=handle)
    flags = []
    for b, (J, path, y, fl) in enumerate(walk_expected(lg, toks, parents, tau, seed, step, streams, max_depth)):
        assert res["accept_len"][b] == J
        assert list(res["path"][b, :J + 1]) == path
        assert res["out_tokens"][b, J] == y
        assert res["flags"][b] == fl, (b, res["flags"][b], fl)
        flags.append(fl)
    return np.array(flags)


def run_walk_pins(handle):
    st = _streams(36)
    # a root-only tree over three tokens: the root's draw sits delta from the boundary C_0
    B = len(st)
    lg = np.zeros((B, 1, 3), np.float32)
    for b in range(B):
        u = np_uniform(201, 0, 2, int(st[b]), oracle.TAG_WALK)
        lg[b, 0] = _logit3(u + DRAW_DELTAS[b % len(DRAW_DELTAS)])
    crafted = check_walk(handle, lg, np.zeros((B, 1), np.int32), np.array([-1]), 1.0, 201, 2, st)
    r = np.random.default_rng(4)
    parents = np.array([-1, 0, 0, 1, 1, 2, 3, 3, 6])
    lg = (r.standard_normal((40, 9, 50)) * 2).astype(np.float32)
    toks = r.integers(0, 50, (40, 9)).astype(np.int32)
    p = _sm(lg, 0.7)
    for c in range(1, 9):  # drafts that the target often picks, so that walks go deep
        toks[:, c] = np.argmax(p[:, parents[c]] + 0.3 * r.random((40, 50)), axis=-1)
    rnd = check_walk(handle, lg, toks, parents, 0.7, 5, 1, _streams(40))
    return int((crafted != 0).sum()), int((rnd != 0).sum())


def test_walk_flags_recomputed():
    crafted, rnd = run_walk_pins(None)
    assert crafted == 18 and rnd == 0, (crafted, rnd)


def test_dropped_walk_flag_fails_the_pins():
    bad = oracle.compile_variant({"if (near) fl |= 2;\n            }": "(void)near;\n            }"},
                                 "walk_flag_off")
    with pytest.raises(AssertionError):
        run_walk_pins(bad)
