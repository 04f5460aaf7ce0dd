"""GPU parity of sv_spec_accept against the fp64 oracle, plus distribution checks of the
GPU's own draws.

Bar: accepted lengths and emitted tokens bit-exact on the same Philox uniforms, except in
sequences the oracle flags as near-threshold (a ratio-test uniform within 1e-6 of p/q, or
the extra draw within 1e-10 of probability mass of a CDF boundary); those are counted,
reported, and bounded: at most 2 per call below 1000 sequences, else 1e-3 of them.
"""
import math

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

GREEDY, SAMPLE = sv.SV_GREEDY, sv.SV_SAMPLE


def _run_both(mode, target, draft, toks, tau, seed, step=0, stream_ids=None, want_alpha=False):
    ref = oracle.spec_accept(mode, target, draft, toks, tau, seed=seed, step=step, stream_ids=stream_ids,
                             want_alpha=want_alpha)
    got = to_host(sv.sv_spec_accept(mode, dev_array(target), None if draft is None else dev_array(draft),
                                    dev_array(toks.astype(np.int32)), tau, seed, step,
                                    None if stream_ids is None else dev_array(np.asarray(stream_ids, np.int64)),
                                    want_alpha=want_alpha))
    return ref, got


def near_threshold_limit(n):
    """Flagged sequences a parity check may excuse: at most 2 below 1000 compared, else
    1e-3 of them (a uniform within 1e-6 of its threshold has probability about 2e-6 per
    decision, so a flag that fires more often than this is broken, not unlucky)."""
    return 2 if n < 1000 else int(1e-3 * n)


def _assert_parity(ref, got, label="", excused_ok=None):
    flagged = ref["flags"] != 0
    same = (ref["accept_len"] == got["accept_len"]) & np.all(ref["out_tokens"] == got["out_tokens"], axis=1)
    bad = ~same & ~flagged
    print("%s sequences=%d near-threshold=%d mismatched(near)=%d mismatched(other)=%d"
          % (label, len(same), flagged.sum(), (~same & flagged).sum(), bad.sum()))
    assert not bad.any(), np.nonzero(bad)[0][:10]
    limit = near_threshold_limit(len(same)) if excused_ok is None else excused_ok
    assert flagged.sum() <= limit, (flagged.sum(), limit)
    assert np.all(got["status"] == 0)


@pytest.mark.parametrize("V", [1, 2, 7, 1000, 1023, 4096, 4097, 5000, 12289])
@pytest.mark.parametrize("gamma", [1, 5, 16])
def test_sample_parity_shapes(V, gamma):
    B = 64
    a = synth.accept_inputs(V + gamma, B=B, gamma=gamma, V=V, target_var=3.0, noise_var=1.0, tau=0.9)
    for step in range(3):
        ref, got = _run_both(SAMPLE, a["target"], a["draft"], a["draft_tokens"], 0.9, seed=11, step=step)
        _assert_parity(ref, got, "V=%d gamma=%d step=%d" % (V, gamma, step))


@pytest.mark.parametrize("B,gamma,V", [(100, 3, 128256), (600, 2, 50257), (3, 4, 128256)])
def test_residual_draw_grid_shapes(B, gamma, V):
    """Residual-draw grids whose blocks take several chunks of a sequence's rows, evenly or
    not: 100 sequences (3 or 4 chunks a block), 600 (every chunk of a sequence in one block),
    and 3 (a block per chunk)."""
    a = synth.accept_inputs(B + V, B=B, gamma=gamma, V=V, target_var=3.0, noise_var=1.0, tau=0.9)
    ref, got = _run_both(SAMPLE, a["target"], a["draft"], a["draft_tokens"], 0.9, seed=5, step=0)
    _assert_parity(ref, got, "B=%d gamma=%d V=%d" % (B, gamma, V))


@pytest.mark.parametrize("V", [1, 3, 1000, 1023, 4097, 128256])
@pytest.mark.parametrize("gamma", [1, 4, 64])
def test_greedy_parity_shapes(V, gamma):
    B = 16 if V > 10000 else 128
    a = synth.accept_inputs(V * 3 + gamma, B=B, gamma=gamma, V=V, target_var=3.0, noise_var=0.3, tau=1.0,
                            greedy_drafts=True)
    tgt = a["target"].copy()
    if V >= 4:
        tgt[: B // 4, :, 1:4] = tgt[: B // 4, :, 1:4].max() + 1.0   # exact ties: lowest id wins
    ref, got = _run_both(GREEDY, tgt, None, a["draft_tokens"], 1.0, seed=0)
    assert np.array_equal(ref["accept_len"], got["accept_len"])
    assert np.array_equal(ref["out_tokens"], got["out_tokens"])


@pytest.mark.parametrize("wl", [1, 2])
@pytest.mark.parametrize("mode", [GREEDY, SAMPLE])
def test_workload_parity(wl, mode):
    cfg = synth.WORKLOADS[wl]
    a = synth.accept_inputs(wl, B=cfg["B"], gamma=cfg["gamma"], V=cfg["V"], target_var=cfg["target_var"],
                            noise_var=cfg["noise_var"], tau=cfg["tau"], greedy_drafts=(mode == GREEDY))
    for step in range(20):
        ref, got = _run_both(mode, a["target"], a["draft"] if mode == SAMPLE else None, a["draft_tokens"],
                             cfg["tau"], seed=1000 + wl, step=step)
        _assert_parity(ref, got, "workload %d step %d" % (wl, step))


@pytest.mark.parametrize("mode", [GREEDY, SAMPLE])
def test_workload_batched_parity(mode):
    cfg = synth.WORKLOADS[4]
    a = synth.accept_inputs(4, B=cfg["B"], gamma=cfg["gamma"], V=cfg["V"], target_var=cfg["target_var"],
                            noise_var=cfg["noise_var"], tau=cfg["tau"], greedy_drafts=(mode == GREEDY))
    sid = np.arange(cfg["B"], dtype=np.int64) * 1000 + 17
    for step in range(3):
        ref, got = _run_both(mode, a["target"], a["draft"] if mode == SAMPLE else None, a["draft_tokens"],
                             cfg["tau"], seed=1004, step=step, stream_ids=sid)
        _assert_parity(ref, got, "batched step %d" % step)


def test_alpha_matches_oracle():
    a = synth.accept_inputs(3, B=8, gamma=5, V=128256, target_var=3.0, noise_var=1.5, tau=0.8)
    ref, got = _run_both(SAMPLE, a["target"], a["draft"], a["draft_tokens"], 0.8, seed=5, want_alpha=True)
    assert np.abs(got["alpha"] - ref["alpha"]).max() < 1e-5
    ref_g, got_g = _run_both(GREEDY, a["target"], None, a["draft_tokens"], 0.8, seed=5, want_alpha=True)
    assert np.isnan(got_g["alpha"]).all()


def test_temperature_zero_is_greedy():
    a = synth.accept_inputs(4, B=32, gamma=4, V=5000, target_var=3.0, noise_var=0.2, tau=1.0, greedy_drafts=True)
    _, g = _run_both(GREEDY, a["target"], None, a["draft_tokens"], 1.0, seed=1)
    _, s0 = _run_both(SAMPLE, a["target"], a["draft"], a["draft_tokens"], 0.0, seed=1)
    assert np.array_equal(g["out_tokens"], s0["out_tokens"])


def test_bad_draft_token_sets_status():
    a = synth.accept_inputs(5, B=4, gamma=3, V=100, target_var=1.0, noise_var=1.0, tau=1.0)
    toks = a["draft_tokens"].copy()
    toks[2, 1] = 100
    got = to_host(sv.sv_spec_accept(SAMPLE, dev_array(a["target"]), dev_array(a["draft"]), dev_array(toks), 1.0, 3))
    assert list(got["status"]) == [0, 0, 2, 0]


def test_output_law_chi_square_on_gpu():
    """10^6 seeded rounds on an 8-token vocabulary: the first emitted token follows p_1."""
    from scipy import special, stats
    V, N, gamma = 8, 1_000_000, 2
    r = np.random.default_rng(8)
    tgt1 = (r.standard_normal((gamma + 1, V)) * 1.5).astype(np.float32)
    dr1 = (tgt1[:gamma] + r.standard_normal((gamma, V))).astype(np.float32)
    q = special.softmax(dr1.astype(np.float64), axis=-1)
    x = np.stack([(np.cumsum(q[i])[None, :] < r.random(N)[:, None]).sum(1) for i in range(gamma)], 1)
    x = np.minimum(x, V - 1).astype(np.int32)
    per = 25_000                      # rounds per call; each call uses its own Philox step
    tgt = torch.from_numpy(tgt1).cuda().expand(per, gamma + 1, V).contiguous()
    dr = torch.from_numpy(dr1).cuda().expand(per, gamma, V).contiguous()
    parts = [to_host(sv.sv_spec_accept(SAMPLE, tgt, dr, dev_array(x[k:k + per]), 1.0, 31, k // per))
             for k in range(0, N, per)]
    got = {key: np.concatenate([p[key] for p in parts]) for key in ("out_tokens", "accept_len")}
    counts = np.bincount(got["out_tokens"][:, 0], minlength=V)
    p1 = special.softmax(tgt1[0].astype(np.float64))
    assert stats.chisquare(counts, p1 * N).pvalue > 1e-4
    alpha = np.minimum(special.softmax(tgt1[:gamma].astype(np.float64), -1), q).sum(-1)
    J = got["accept_len"]
    assert abs(J.mean() - np.cumprod(alpha).sum()) < 4 * J.std() / math.sqrt(N)


@pytest.mark.parametrize("B,gamma,V", [(1, 5, 128256), (4, 3, 5000), (16, 2, 1000), (1, 64, 4097), (64, 1, 7)])
def test_alpha_pass_changes_no_decision(B, gamma, V):
    """Asking for alpha adds its own pass over the rows between the statistics and the
    residual draw; the accepted lengths and tokens stay the same, bit for bit, over several
    rounds."""
    a = synth.accept_inputs(70 + B, B=B, gamma=gamma, V=V, target_var=3.0, noise_var=1.0, tau=0.8)
    for step in range(4):
        args = (SAMPLE, dev_array(a["target"]), dev_array(a["draft"]), dev_array(a["draft_tokens"]), 0.8, 9, step)
        one = to_host(sv.sv_spec_accept(*args))
        two = to_host(sv.sv_spec_accept(*args, want_alpha=True))
        assert np.array_equal(one["accept_len"], two["accept_len"])
        assert np.array_equal(one["out_tokens"], two["out_tokens"])
        assert np.all(one["status"] == 0) and np.all(two["status"] == 0)


def test_deterministic_repeats():
    a = synth.accept_inputs(2, B=1, gamma=5, V=128256, target_var=3.0, noise_var=1.5, tau=0.8)
    args = (SAMPLE, dev_array(a["target"]), dev_array(a["draft"]), dev_array(a["draft_tokens"]), 0.8, 7)
    first = to_host(sv.sv_spec_accept(*args))
    for _ in range(10):
        again = to_host(sv.sv_spec_accept(*args))
        assert np.array_equal(first["out_tokens"], again["out_tokens"])


def test_shared_workspace_across_entry_points_and_shapes():
    """One zero-filled workspace serves a sequence of calls of every entry point and shape
    (regression: a later call once found an earlier call's partial results where its own
    completion counters lived)."""
    cases = [(4, 5, 5000, SAMPLE), (128, 4, 1000, GREEDY), (64, 4, 3000, SAMPLE), (2, 16, 128256, SAMPLE),
             (200, 1, 77, GREEDY), (7, 3, 9000, SAMPLE)]
    parents = synth.random_tree(9, 30, branch_p=0.6)
    for k, (B, gamma, V, mode) in enumerate(cases):
        a = synth.accept_inputs(50 + k, B=B, gamma=gamma, V=V, target_var=3.0, noise_var=0.5, tau=0.9,
                                greedy_drafts=(mode == GREEDY))
        ref, got = _run_both(mode, a["target"], a["draft"] if mode == SAMPLE else None, a["draft_tokens"], 0.9,
                             seed=3, step=k)
        _assert_parity(ref, got, "shared workspace case %d" % k)
        # a tree walk and an attention call on the same workspace between acceptance calls
        lg = synth.tree_logits(k, 3, 30, 700 + 13 * k, 3.0)
        tk = synth.node_tokens(k, lg, parents)
        maxd = int(oracle.tree_mask(parents, 0)[1].max())
        w = to_host(sv.sv_tree_walk(SAMPLE, dev_array(lg), dev_array(tk), dev_array(parents.astype(np.int32)), maxd,
                                    0.7, 5, k))
        r = oracle.tree_walk(SAMPLE, lg, tk, parents, 0.7, seed=5, step=k, max_depth=maxd)
        ok = (r["flags"] != 0) | np.all(w["path"] == r["path"], axis=1)
        assert ok.all()
        inp = synth.attention_inputs(k, B=2, n_q=5, Hq=8, Hkv=2, D=128, prefix_len=[300 + 97 * k, 40],
                                     dtype="bf16")
        ref_o, _, rows = oracle.attention(inp, scale=0.09)
        from svgpu import attention_on_gpu, rows_of
        out, _ = attention_on_gpu(inp, 0.09, split_keys=128)
        assert np.abs(rows_of(out, rows) - ref_o).max() <= 2e-2


def test_crafted_near_threshold_decisions():
    """Ratio tests placed 1e-7 ... 1e-5 from p/q and extra draws placed 1e-11 ... 1e-9 from a
    CDF boundary (inputs built from NumPy's own Philox): every decision outside its window
    (1e-6 for a ratio test, 1e-10 of probability mass for a draw) must match the oracle bit
    for bit, which bounds the GPU's error in p/q and in the CDF; the sequences the oracle
    flags are exactly the crafted ones inside the window."""
    from test_oracle_flags import DELTAS, DRAW_DELTAS, STEPS, crafted_draw_inputs, crafted_ratio_inputs, _streams
    st = _streams(48)
    near = np.array([abs(STEPS[b % len(STEPS)]) < 1.0 for b in range(len(st))])
    for make, deltas, seed, step in ((crafted_ratio_inputs, DELTAS, 101, 3), (crafted_draw_inputs, DRAW_DELTAS, 102, 5)):
        tgt, dr, toks = make(seed, step, st, deltas)
        ref, got = _run_both(SAMPLE, tgt, dr, toks, 1.0, seed=seed, step=step, stream_ids=st.astype(np.int64))
        assert np.array_equal(ref["flags"] != 0, near)
        _assert_parity(ref, got, make.__name__, excused_ok=int(near.sum()))
