"""Pins of the oracle's rounds with per-sequence draft lengths (oracle.accept_ragged).

The pages fix what a round with fewer verified drafts emits through the trimming
counterexample ("Speculative decoding", section "Choosing how much to verify at every step",
box "Trimming a draft can break exactness"): with p = (0.5, 0.3, 0.2), q = (0.2, 0.6, 0.2),
verifying always and verifying never both emit p, while verifying only drafts other than b
emits (0.5, 0.18, 0.32).  Those laws are checked here by chi-square over many sequences, each
with its own length, and the wrapper's layout against single-sequence calls.
"""
import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from conftest import read_golden

SAMPLE, GREEDY = oracle.SAMPLE, oracle.GREEDY


def _toy(N, seed):
    g = read_golden("trim_counterexample.txt")
    p = np.array([float(v) for v in g["p"]])
    q = np.array([float(v) for v in g["q"]])
    law = np.array([float(v) for v in g["trimmed_law"]])
    lp, lq = np.log(p).astype(np.float32), np.log(q).astype(np.float32)
    target = np.broadcast_to(lp, (N, 2, 3)).copy()   # position 0, then the row after the draft
    draft = np.broadcast_to(lq, (N, 1, 3)).copy()
    x = np.random.default_rng(seed).choice(3, size=N, p=q).astype(np.int32).reshape(N, 1)
    return p, q, law, target, draft, x


@pytest.mark.parametrize("rule", [oracle.RULE_TOKEN, oracle.RULE_BLOCK])
def test_trimming_counterexample(rule):
    N = 200_000
    p, q, law, target, draft, x = _toy(N, 7)
    policies = {
        "always": (np.ones(N, np.int64), p),
        "never": (np.zeros(N, np.int64), p),
        "only drafts other than b": ((x[:, 0] != 1).astype(np.int64), law),
    }
    for name, (L, want) in policies.items():
        r = oracle.accept_ragged(rule, SAMPLE, target, draft, x, L, 1.0, seed=123, step=0)
        y = r["out_tokens"][:, 0]
        assert np.all(r["accept_len"] <= L)
        counts = np.bincount(y, minlength=3)
        pv = stats.chisquare(counts, want * N).pvalue
        print(name, counts / N, pv)
        assert pv > 1e-4, (name, counts / N)
        if name.startswith("only"):
            # the test tells the trimmed law from p
            assert stats.chisquare(counts, p * N).pvalue < 1e-12


def test_full_lengths_equal_the_fixed_round():
    a = synth.accept_inputs(3, B=24, gamma=5, V=300, target_var=3.0, noise_var=1.0, tau=0.8)
    L = np.full(24, 5)
    r = oracle.accept_ragged(oracle.RULE_TOKEN, SAMPLE, a["target"], a["draft"], a["draft_tokens"], L, 0.8,
                             seed=5, step=2, want_alpha=True)
    f = oracle.spec_accept(SAMPLE, a["target"], a["draft"], a["draft_tokens"], 0.8, seed=5, step=2,
                           want_alpha=True)
    for k in ("accept_len", "out_tokens", "flags"):
        assert np.array_equal(r[k], f[k]), k
    assert np.array_equal(r["alpha"], f["alpha"])


@pytest.mark.parametrize("rule,mode", [(oracle.RULE_TOKEN, SAMPLE), (oracle.RULE_BLOCK, SAMPLE),
                                       (oracle.RULE_GUMBEL, SAMPLE), (oracle.RULE_TOKEN, GREEDY)])
def test_each_sequence_is_its_own_round(rule, mode):
    """Sequence b with length L_b equals a round of that sequence alone at gamma = L_b, with
    its own stream of uniforms; outputs past it are -1, alpha past L_b NaN."""
    B, g, V = 30, 6, 200
    a = synth.accept_inputs(11, B=B, gamma=g, V=V, target_var=2.0, noise_var=0.5, tau=0.7,
                            greedy_drafts=(mode == GREEDY))
    L = np.random.default_rng(2).integers(0, g + 1, B)
    L[:3] = [0, g, 1]
    sid = np.arange(100, 100 + B, dtype=np.uint64)
    r = oracle.accept_ragged(rule, mode, a["target"], a["draft"], a["draft_tokens"], L, 0.7, seed=9, step=1,
                             stream_ids=sid, want_alpha=(rule == oracle.RULE_TOKEN))
    for b in range(B):
        lb = int(L[b])
        t, d, x = a["target"][b:b + 1, :lb + 1], a["draft"][b:b + 1, :lb], a["draft_tokens"][b:b + 1, :lb]
        if mode == GREEDY:
            one = oracle.spec_accept(GREEDY, t, None, x, 0.7, seed=9, step=1, stream_ids=sid[b:b + 1])
        elif rule == oracle.RULE_GUMBEL:
            one = oracle.gumbel_accept(t, x, 0.7, seed=9, step=1, stream_ids=sid[b:b + 1])
        elif rule == oracle.RULE_BLOCK:
            one = oracle.block_accept(t, d, x, 0.7, seed=9, step=1, stream_ids=sid[b:b + 1])
        else:
            one = oracle.spec_accept(SAMPLE, t, d, x, 0.7, seed=9, step=1, stream_ids=sid[b:b + 1], want_alpha=True)
        assert r["accept_len"][b] == one["accept_len"][0] <= lb
        assert np.array_equal(r["out_tokens"][b, :lb + 1], one["out_tokens"][0])
        assert np.all(r["out_tokens"][b, lb + 1:] == -1)
        if rule == oracle.RULE_TOKEN and mode == SAMPLE:
            assert np.array_equal(r["alpha"][b, :lb], one["alpha"][0])
            assert np.all(np.isnan(r["alpha"][b, lb:]))


def test_zero_length_gumbel_is_the_targets_own_sample():
    B, V = 50, 97
    a = synth.accept_inputs(4, B=B, gamma=3, V=V, target_var=2.0, noise_var=0.5, tau=0.9)
    r = oracle.accept_ragged(oracle.RULE_GUMBEL, SAMPLE, a["target"], None, a["draft_tokens"], np.zeros(B), 0.9,
                             seed=3, step=4)
    y, _ = oracle.gumbel_argmax(a["target"][:, :1], 0.9, seed=3, step=4, stream_ids=np.arange(B, dtype=np.uint64))
    assert np.all(r["accept_len"] == 0)
    assert np.array_equal(r["out_tokens"][:, 0], y[:, 0])


def test_lengths_outside_the_range_are_refused():
    a = synth.accept_inputs(1, B=2, gamma=2, V=10, target_var=1.0, noise_var=1.0, tau=1.0)
    for L in ([0, 3], [-1, 1]):
        with pytest.raises(ValueError):
            oracle.accept_ragged(oracle.RULE_TOKEN, SAMPLE, a["target"], a["draft"], a["draft_tokens"], L, 1.0, 0)
