"""GPU parity of sv_spec_accept with per-sequence draft lengths (draft_len) against
oracle.accept_ragged: every rule, sampled and greedy, lengths 0..gamma mixed in one call.

Bar as for the fixed-length rounds: accepted lengths and emitted tokens bit-exact on every
sequence the oracle does not flag near-threshold, flagged ones bounded; alpha within 1e-5
where verified and NaN past each length; status 3 for a length outside [0, gamma].
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import draft_token_verification_attention_amd as sv  # noqa: E402
from svgpu import dev_array, to_host  # noqa: E402
from test_gpu_accept import _assert_parity  # noqa: E402

RULES = {"token": (oracle.RULE_TOKEN, sv.SV_RULE_TOKEN), "block": (oracle.RULE_BLOCK, sv.SV_RULE_BLOCK),
         "gumbel": (oracle.RULE_GUMBEL, sv.SV_RULE_GUMBEL)}


def _lengths(B, g, seed):
    L = np.random.default_rng(seed).integers(0, g + 1, B)
    L[:4] = [0, g, 1, 0]
    return L.astype(np.int32)


def _run(rule, mode, a, L, tau, seed, step=0, want_alpha=False):
    orule, grule = RULES[rule]
    ref = oracle.accept_ragged(orule, mode, a["target"], a["draft"], a["draft_tokens"], L, tau, seed, step,
                               want_alpha=want_alpha)
    got = to_host(sv.sv_spec_accept(mode, dev_array(a["target"]),
                                    None if a["draft"] is None else dev_array(a["draft"]),
                                    dev_array(a["draft_tokens"].astype(np.int32)), tau, seed, step,
                                    want_alpha=want_alpha, rule=grule, draft_len=dev_array(L)))
    return ref, got


@pytest.mark.parametrize("rule", ["token", "block", "gumbel"])
@pytest.mark.parametrize("V,g", [(5000, 6), (1023, 16), (128256, 4)])
def test_ragged_parity(rule, V, g):
    B = 16 if V > 100000 else 96
    a = synth.accept_inputs(V + g, B=B, gamma=g, V=V, target_var=3.0, noise_var=1.0, tau=0.9)
    L = _lengths(B, g, V)
    for step in range(2):
        ref, got = _run(rule, sv.SV_SAMPLE, a, L, 0.9, seed=21, step=step, want_alpha=(rule == "token"))
        _assert_parity(ref, got, "%s V=%d gamma=%d step=%d" % (rule, V, g, step))
        assert np.all(got["accept_len"] <= L)
        if rule == "token":
            verified = np.arange(g)[None, :] < L[:, None]
            assert np.all(np.isnan(got["alpha"][~verified]))
            assert np.abs(got["alpha"][verified] - ref["alpha"][verified]).max() < 1e-5


@pytest.mark.parametrize("V", [3, 5000, 128256])
def test_ragged_greedy(V):
    B, g = 64, 5
    a = synth.accept_inputs(V, B=B, gamma=g, V=V, target_var=3.0, noise_var=0.3, tau=1.0, greedy_drafts=True)
    L = _lengths(B, g, 1)
    ref, got = _run("token", sv.SV_GREEDY, dict(a, draft=None), L, 1.0, seed=0)
    assert np.array_equal(ref["accept_len"], got["accept_len"])
    assert np.array_equal(ref["out_tokens"], got["out_tokens"])
    assert np.all(got["status"] == 0)


@pytest.mark.parametrize("rule", ["token", "block", "gumbel"])
def test_full_lengths_equal_no_lengths(rule):
    """draft_len all gamma gives the same results as no draft_len (bit for bit)."""
    B, g, V = 32, 5, 4097
    a = synth.accept_inputs(8, B=B, gamma=g, V=V, target_var=3.0, noise_var=1.0, tau=0.8)
    args = (sv.SV_SAMPLE, dev_array(a["target"]), dev_array(a["draft"]), dev_array(a["draft_tokens"].astype(np.int32)),
            0.8, 4, 1)
    x = to_host(sv.sv_spec_accept(*args, rule=RULES[rule][1]))
    y = to_host(sv.sv_spec_accept(*args, rule=RULES[rule][1], draft_len=dev_array(np.full(B, g, np.int32))))
    for k in ("accept_len", "out_tokens", "status"):
        assert np.array_equal(x[k], y[k]), k


def test_all_zero_lengths_sample_the_target():
    """L = 0 everywhere: one draw from target row 0 per sequence, whatever the drafts."""
    B, g, V = 200, 3, 700
    a = synth.accept_inputs(2, B=B, gamma=g, V=V, target_var=3.0, noise_var=1.0, tau=1.0)
    L = np.zeros(B, np.int32)
    ref, got = _run("token", sv.SV_SAMPLE, a, L, 1.0, seed=8)
    _assert_parity(ref, got, "zero lengths")
    assert np.all(got["accept_len"] == 0) and np.all(got["out_tokens"][:, 1:] == -1)


def test_out_of_range_lengths_report_status_3():
    B, g, V = 8, 4, 500
    a = synth.accept_inputs(5, B=B, gamma=g, V=V, target_var=2.0, noise_var=1.0, tau=1.0)
    L = np.array([0, 4, -1, 5, 2, 9, 1, 3], np.int32)
    for rule in ("token", "block", "gumbel"):
        got = to_host(sv.sv_spec_accept(sv.SV_SAMPLE, dev_array(a["target"]), dev_array(a["draft"]),
                                        dev_array(a["draft_tokens"].astype(np.int32)), 1.0, 3, 0,
                                        rule=RULES[rule][1], draft_len=dev_array(L)))
        assert list(got["status"]) == [0, 0, 3, 3, 0, 3, 0, 0], (rule, got["status"])
        ok = np.array([0, 1, 4, 6, 7])
        assert np.all(got["accept_len"][ok] <= L[ok])


def test_static_entry_point_takes_lengths():
    """sv_spec_accept_static with draft_len: the same kernels, bit for bit."""
    B, g, V = 40, 5, 5000
    a = synth.accept_inputs(12, B=B, gamma=g, V=V, target_var=3.0, noise_var=1.0, tau=1.0)
    L = dev_array(_lengths(B, g, 4))
    args = (sv.SV_SAMPLE, dev_array(a["target"]), dev_array(a["draft"]), dev_array(a["draft_tokens"].astype(np.int32)),
            1.0, 6, 2)
    x = to_host(sv.sv_spec_accept(*args, want_alpha=True, draft_len=L))
    y = to_host(sv.sv_spec_accept_static(*args, want_alpha=True, draft_len=L))
    for k in ("accept_len", "out_tokens", "status"):
        assert np.array_equal(x[k], y[k]), k
    assert np.array_equal(x["alpha"], y["alpha"], equal_nan=True)
