"""Pins of the oracle's acceptance (greedy prefix match and speculative sampling).

Against what the pages fix: the three-token worked example; alpha = sum min(p,q)
= 1 - TV(p,q); the special cases (greedy target, deterministic draft, p = q);
the output law equals p (chi-square over seeded draws, with a planted
"resample from p" mistake in a copy of the oracle as the negative control);
E[J] = sum_i prod_{j<=i} alpha_j; the expected-token values the pages print;
the block-verification toy's token-wise 10/9; inverse-CDF sampling against
numpy.searchsorted; greedy against numpy.argmax.
"""
import math

import numpy as np
import pytest
from scipy import special, stats

import oracle
import synth
from conftest import read_golden

GREEDY, SAMPLE = oracle.GREEDY, oracle.SAMPLE


def _logits_of(p):
    with np.errstate(divide="ignore"):
        lg = np.log(np.asarray(p, dtype=np.float64))
    return np.where(np.isfinite(lg), lg, -1000.0).astype(np.float32)


def _draw_from(probs, u):
    """Inverse-CDF draws (test-side drafter): rows of probs, one uniform per row."""
    c = np.cumsum(probs, axis=-1)
    return np.minimum((c < u[..., None] * c[..., -1:]).sum(axis=-1), probs.shape[-1] - 1)


def _sm(lg, tau=1.0):
    """softmax(lg / tau) in fp64; tau crosses the boundary as fp32, so it is rounded the same way."""
    return special.softmax(np.asarray(lg, dtype=np.float64) / float(np.float32(tau)), axis=-1)


# --------------------------------------------------------------------------- #
def test_worked_example_alpha_tv_residual():
    g = read_golden("rule_example.txt")
    p = np.array(g["p"], dtype=float)
    q = np.array(g["q"], dtype=float)
    tgt = np.stack([_logits_of(p), _logits_of(p)])[None]        # gamma = 1: row 0, bonus row 1
    dr = _logits_of(q)[None, None]
    res = oracle.spec_accept(SAMPLE, tgt, dr, [[1]], 1.0, seed=1, want_alpha=True)
    pp, qq = _sm(tgt[0, 0]), _sm(dr[0, 0])
    assert abs(res["alpha"][0, 0] - float(g["alpha"][0])) < 1e-7
    assert abs(0.5 * np.abs(pp - qq).sum() - float(g["tv"][0])) < 1e-7
    assert abs((pp * qq).sum() - float(g["naive_agreement"][0])) < 1e-7
    keep = np.minimum(1.0, pp / qq)
    assert np.allclose(keep, np.array(g["keep_prob"], dtype=float), atol=1e-7)


def test_worked_example_output_law_and_residual():
    """Drafts x ~ q over many independent streams: rejected b's become a's, the
    keep rate of b is 1/2, and the first emitted token follows p = (.5,.3,.2)."""
    g = read_golden("rule_example.txt")
    p = np.array(g["p"], dtype=float)
    q = np.array(g["q"], dtype=float)
    N = 400_000
    tgt = np.broadcast_to(np.stack([_logits_of(p), _logits_of(p)]), (N, 2, 3))
    dr = np.broadcast_to(_logits_of(q)[None], (N, 1, 3))
    x = _draw_from(np.broadcast_to(q, (N, 3)), np.random.default_rng(3).random(N)).reshape(N, 1)
    res = oracle.spec_accept(SAMPLE, tgt, dr, x, 1.0, seed=77)
    J, out = res["accept_len"], res["out_tokens"]
    rejected = J == 0
    assert np.all(out[rejected, 0] == 0)                        # residual (1, 0, 0)
    assert np.all(J[x[:, 0] != 1] == 1)                         # a and c are always kept
    kb = J[x[:, 0] == 1].mean()
    nb = int((x[:, 0] == 1).sum())
    assert abs(kb - 0.5) < 4 * math.sqrt(0.25 / nb)
    counts = np.bincount(out[:, 0], minlength=3)
    law = np.array(g["output_law"], dtype=float)
    assert stats.chisquare(counts, law * N).pvalue > 1e-4


@pytest.mark.parametrize("tau", [0.5, 1.0, 1.7])
def test_alpha_equals_one_minus_tv(tau):
    r = np.random.default_rng(4)
    B, gamma, V = 16, 3, 50
    tgt = (r.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    dr = (tgt[:, :gamma] + r.standard_normal((B, gamma, V))).astype(np.float32)
    toks = r.integers(0, V, size=(B, gamma))
    res = oracle.spec_accept(SAMPLE, tgt, dr, toks, tau, seed=2, want_alpha=True)
    tv = 0.5 * np.abs(_sm(tgt[:, :gamma], tau) - _sm(dr, tau)).sum(-1)
    assert np.allclose(res["alpha"], 1.0 - tv, rtol=0, atol=1e-12)


def test_greedy_is_argmax_prefix_plus_one():
    r = np.random.default_rng(5)
    B, gamma, V = 500, 5, 40
    tgt = r.standard_normal((B, gamma + 1, V)).astype(np.float32)
    tgt[:7, :, :3] = 1.5                                   # ties: lowest id wins
    z = np.argmax(tgt, axis=-1)                            # numpy returns the first maximum
    toks = np.where(r.random((B, gamma)) < 0.7, z[:, :gamma], r.integers(0, V, (B, gamma)))
    res = oracle.spec_accept(GREEDY, tgt, None, toks, 1.0, seed=0)
    for b in range(B):
        J = 0
        while J < gamma and toks[b, J] == z[b, J]:
            J += 1
        assert res["accept_len"][b] == J
        assert list(res["out_tokens"][b, :J + 1]) == list(toks[b, :J]) + [z[b, J]]
        assert np.all(res["out_tokens"][b, J + 1:] == -1)
    # temperature 0 in sampling mode is greedy
    res0 = oracle.spec_accept(SAMPLE, tgt, tgt[:, :gamma], toks, 0.0, seed=9)
    assert np.array_equal(res0["out_tokens"], res["out_tokens"])


def test_greedy_target_reduces_sampling_to_greedy():
    """p one-hot (a huge logit gap makes exp underflow to exactly 0): sampling == greedy."""
    r = np.random.default_rng(6)
    B, gamma, V = 300, 3, 20
    tgt = r.standard_normal((B, gamma + 1, V)).astype(np.float32)
    z = r.integers(0, V, (B, gamma + 1))
    np.put_along_axis(tgt, z[..., None], 2000.0, axis=-1)
    dr = r.standard_normal((B, gamma, V)).astype(np.float32)
    toks = np.where(r.random((B, gamma)) < 0.6, z[:, :gamma], r.integers(0, V, (B, gamma)))
    s = oracle.spec_accept(SAMPLE, tgt, dr, toks, 1.0, seed=3)
    gr = oracle.spec_accept(GREEDY, tgt, None, toks, 1.0, seed=3)
    assert np.array_equal(s["out_tokens"], gr["out_tokens"])
    assert np.array_equal(s["accept_len"], gr["accept_len"])


def test_deterministic_draft_accepts_with_p_and_residual_drops_it():
    """q one-hot at xh: accepted with probability p(xh); on rejection the residual is
    p with xh removed and renormalized."""
    V, N, xh = 6, 300_000, 2
    p = np.array([0.1, 0.25, 0.3, 0.05, 0.2, 0.1])
    q = np.zeros(V)
    q[xh] = 1.0
    tgt = np.broadcast_to(np.stack([_logits_of(p), _logits_of(p)]), (N, 2, V))
    dr = np.broadcast_to(_logits_of(q)[None], (N, 1, V))
    res = oracle.spec_accept(SAMPLE, tgt, dr, np.full((N, 1), xh), 1.0, seed=12)
    acc = res["accept_len"].mean()
    assert abs(acc - p[xh]) < 4 * math.sqrt(p[xh] * (1 - p[xh]) / N)
    rej = res["out_tokens"][res["accept_len"] == 0, 0]
    want = p.copy()
    want[xh] = 0
    want /= want.sum()
    counts = np.bincount(rej, minlength=V)
    assert counts[xh] == 0
    keep = want > 0
    assert stats.chisquare(counts[keep], want[keep] * len(rej)).pvalue > 1e-4


def test_equal_distributions_always_accept():
    r = np.random.default_rng(7)
    B, gamma, V = 2000, 4, 30
    tgt = r.standard_normal((B, gamma + 1, V)).astype(np.float32)
    toks = r.integers(0, V, (B, gamma))
    res = oracle.spec_accept(SAMPLE, tgt, tgt[:, :gamma].copy(), toks, 0.9, seed=4)
    assert np.all(res["accept_len"] == gamma)


# --------------------------------------------------------------------------- #
def _bigram_models(seed, V=6):
    r = np.random.default_rng(seed)
    tl = r.standard_normal((V, V))
    dl = tl + 0.7 * r.standard_normal((V, V))
    return tl.astype(np.float32), dl.astype(np.float32)


def _bigram_two_tokens(handle, N, seed, s0=0, gamma=2):
    """The textbook's check ("A whole round of speculative sampling"): two bigram models over
    six tokens, each drafted position conditioned on the drafts before it; returns the first
    two emitted tokens of N sequences (running a second round when the first emits one)."""
    tl, dl = _bigram_models(seed)
    V = tl.shape[0]
    r = np.random.default_rng(seed + 100)
    qd = _sm(dl)
    x = np.zeros((N, gamma), dtype=np.int64)
    prev = np.full(N, s0)
    for i in range(gamma):
        x[:, i] = _draw_from(qd[prev], r.random(N))
        prev = x[:, i]
    ctx = np.concatenate([np.full((N, 1), s0), x], axis=1)          # token before each position
    tgt = tl[ctx]                                                    # [N][gamma+1][V]
    dr = dl[ctx[:, :gamma]]
    res = oracle.spec_accept(SAMPLE, tgt, dr, x, 1.0, seed=seed, step=0, handle=handle)
    J, out = res["accept_len"], res["out_tokens"]
    t1 = out[:, 0].copy()
    t2 = out[:, 1].copy()
    need = J == 0
    m = int(need.sum())
    if m:
        y = t1[need]
        x2 = _draw_from(qd[y], r.random(m)).reshape(m, 1)
        tgt2 = np.stack([tl[y], tl[x2[:, 0]]], axis=1)
        dr2 = dl[y][:, None, :]
        res2 = oracle.spec_accept(SAMPLE, tgt2, dr2, x2, 1.0, seed=seed, step=1, handle=handle)
        t2[need] = res2["out_tokens"][:, 0]
    exact = np.outer(_sm(tl[s0]), np.ones(V)) * _sm(tl)             # p(a|s0) p(b|a)
    counts = np.zeros((V, V))
    np.add.at(counts, (t1, t2), 1)
    return counts, exact * N


def test_bigram_two_token_law_chi_square():
    counts, expected = _bigram_two_tokens(None, 1_000_000, seed=21)
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert stats.chi2.sf(chi2, df=35) > 1e-4, chi2


def test_planted_resample_from_p_fails_chi_square():
    """Negative control: a copy of the oracle that resamples from p after a rejection
    (the textbook's most common bug) must fail the same test."""
    bad = oracle.compile_variant({"q[x] = fmax(0.0, p[x] - q[x]);": "q[x] = p[x];"}, "resample_p")
    counts, expected = _bigram_two_tokens(bad, 1_000_000, seed=21)
    chi2 = ((counts - expected) ** 2 / expected).sum()
    assert stats.chi2.sf(chi2, df=35) < 1e-12, chi2


def test_output_law_tiny_vocab_chi_square():
    """The first emitted token of a round follows p_1 whatever q is (10^6 seeded draws, V = 8)."""
    V, N, gamma = 8, 1_000_000, 2
    r = np.random.default_rng(8)
    tgt1 = (r.standard_normal((gamma + 1, V)) * 1.5).astype(np.float32)
    dr1 = (tgt1[:gamma] + r.standard_normal((gamma, V))).astype(np.float32)
    x = np.stack([_draw_from(np.broadcast_to(_sm(dr1[i]), (N, V)), r.random(N)) for i in range(gamma)], 1)
    res = oracle.spec_accept(SAMPLE, np.broadcast_to(tgt1, (N, gamma + 1, V)),
                             np.broadcast_to(dr1, (N, gamma, V)), x, 1.0, seed=31)
    counts = np.bincount(res["out_tokens"][:, 0], minlength=V)
    assert stats.chisquare(counts, _sm(tgt1[0]) * N).pvalue > 1e-4


def test_mean_accepted_length_is_survival_sum():
    """Rows that do not depend on the drafted prefix: P(J >= i) = prod_{j<=i} alpha_j, so
    E[J] = sum_i prod_{j<=i} alpha_j (textbook "Speculative verification in PyTorch")."""
    V, N, gamma = 8, 400_000, 4
    r = np.random.default_rng(9)
    tgt1 = (r.standard_normal((gamma + 1, V)) * 1.3).astype(np.float32)
    dr1 = (tgt1[:gamma] + 0.8 * r.standard_normal((gamma, V))).astype(np.float32)
    x = np.stack([_draw_from(np.broadcast_to(_sm(dr1[i]), (N, V)), r.random(N)) for i in range(gamma)], 1)
    res = oracle.spec_accept(SAMPLE, np.broadcast_to(tgt1, (N, gamma + 1, V)),
                             np.broadcast_to(dr1, (N, gamma, V)), x, 1.0, seed=41, want_alpha=False)
    alpha = np.minimum(_sm(tgt1[:gamma]), _sm(dr1)).sum(-1)
    want = np.cumprod(alpha).sum()
    J = res["accept_len"]
    assert abs(J.mean() - want) < 4 * J.std() / math.sqrt(N)


@pytest.mark.parametrize("row", range(3))
def test_expected_tokens_printed_values(row):
    """alpha = 0.8 from p = (0.8, 0.2) and a draft that always proposes token 0."""
    a, gamma, printed, dec = read_golden("expected_tokens.txt")["_rows"][row]
    a, gamma, printed, dec = float(a), int(gamma), float(printed), int(dec)
    closed = (1 - a ** (gamma + 1)) / (1 - a)
    assert round(closed, dec) == printed
    N = 400_000
    p = np.array([a, 1 - a])
    tgt = np.broadcast_to(_logits_of(p), (N, gamma + 1, 2))
    dr = np.broadcast_to(_logits_of([1.0, 0.0]), (N, gamma, 2))
    res = oracle.spec_accept(SAMPLE, tgt, dr, np.zeros((N, gamma), dtype=np.int32), 1.0, seed=51)
    n_tok = res["accept_len"] + 1
    assert abs(n_tok.mean() - closed) < 4 * n_tok.std() / math.sqrt(N)


def test_block_verification_toy_tokenwise():
    g = read_golden("block_toy.txt")
    p = np.array(g["p"], dtype=float)
    q = np.array(g["q"], dtype=float)
    gamma = int(g["gamma"][0])
    want = int(g["tokenwise_EJ_num"][0]) / int(g["tokenwise_EJ_den"][0])
    N = 400_000
    r = np.random.default_rng(10)
    x = np.stack([_draw_from(np.broadcast_to(q, (N, 2)), r.random(N)) for _ in range(gamma)], 1)
    res = oracle.spec_accept(SAMPLE, np.broadcast_to(_logits_of(p), (N, gamma + 1, 2)),
                             np.broadcast_to(_logits_of(q), (N, gamma, 2)), x, 1.0, seed=61)
    J = res["accept_len"]
    assert abs(J.mean() - want) < 4 * J.std() / math.sqrt(N)


def test_inverse_cdf_matches_searchsorted():
    """The extra token is searchsorted(cumsum(r), u* Z, 'right') with u* the dedicated uniform."""
    r = np.random.default_rng(11)
    B, gamma, V = 400, 3, 300
    tgt = (r.standard_normal((B, gamma + 1, V)) * 2).astype(np.float32)
    dr = (tgt[:, :gamma] + r.standard_normal((B, gamma, V))).astype(np.float32)
    toks = r.integers(0, V, (B, gamma))
    tau, seed = 0.8, 5
    res = oracle.spec_accept(SAMPLE, tgt, dr, toks, tau, seed=seed, stream_ids=np.arange(B) * 7 + 3)
    pt, pd = _sm(tgt, tau), _sm(dr, tau)
    checked = 0
    for b in range(B):
        J = res["accept_len"][b]
        w = np.maximum(pt[b, J] - pd[b, J], 0.0) if J < gamma else pt[b, gamma]
        u = oracle.uniform(seed, gamma, 0, b * 7 + 3, oracle.TAG_ACCEPT)
        y = int(np.searchsorted(np.cumsum(w), u * w.sum(), side="right"))
        if res["flags"][b] & 2:
            continue
        checked += 1
        assert res["out_tokens"][b, J] == y
        # the ratio tests use the position-indexed uniforms
        for i in range(J + 1 if J < gamma else gamma):
            ui = oracle.uniform(seed, i, 0, b * 7 + 3, oracle.TAG_ACCEPT)
            passed = ui * pd[b, i, toks[b, i]] < pt[b, i, toks[b, i]]
            assert passed == (i < J)
    assert checked > B * 0.9


def test_synthetic_workload_inputs_run():
    """The tiny chain workload end to end through the oracle (greedy and sampling)."""
    cfg = synth.WORKLOADS[1]
    a = synth.accept_inputs(1, B=1, gamma=cfg["gamma"], V=cfg["V"], target_var=cfg["target_var"],
                            noise_var=cfg["noise_var"], tau=cfg["tau"])
    s = oracle.spec_accept(SAMPLE, a["target"], a["draft"], a["draft_tokens"], cfg["tau"], seed=1001,
                           want_alpha=True)
    g = oracle.spec_accept(GREEDY, a["target"], None, a["draft_tokens"], cfg["tau"], seed=1001)
    for res in (s, g):
        J = res["accept_len"][0]
        assert 0 <= J <= cfg["gamma"] and 0 <= res["out_tokens"][0, J] < cfg["V"]
    assert np.all((s["alpha"] > 0) & (s["alpha"] < 1))
