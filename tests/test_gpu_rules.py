"""GPU parity of sv_spec_accept's other verification rules against the fp64 oracle:
block verification (SV_RULE_BLOCK) and Gumbel-coupled verification (SV_RULE_GUMBEL).
Accepted lengths and emitted tokens bit-exact on the same uniforms (the same noise),
except in sequences the oracle flags near a threshold (bounded as for speculative
sampling); the GPU's own Gumbel-max draws follow the target's law."""
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
from test_gpu_accept import _assert_parity  # noqa: E402

SAMPLE, GREEDY = sv.SV_SAMPLE, sv.SV_GREEDY


def _gpu(rule, a, tau, seed, step=0, stream_ids=None, mode=SAMPLE, draft_tokens=None):
    toks = a["draft_tokens"] if draft_tokens is None else draft_tokens
    return to_host(sv.sv_spec_accept(mode, dev_array(a["target"]), dev_array(a["draft"]),
                                     dev_array(np.asarray(toks, np.int32)), tau, seed, step,
                                     None if stream_ids is None else dev_array(np.asarray(stream_ids, np.int64)),
                                     rule=rule))


@pytest.mark.parametrize("V", [7, 1000, 4097, 12289, 128256])
@pytest.mark.parametrize("gamma", [1, 4, 16])
def test_block_parity_shapes(V, gamma):
    B = 16 if V > 100000 else 64
    a = synth.accept_inputs(V + 3 * gamma, B=B, gamma=gamma, V=V, target_var=3.0, noise_var=1.0, tau=0.9)
    for step in range(2):
        ref = oracle.block_accept(a["target"], a["draft"], a["draft_tokens"], 0.9, seed=13, step=step)
        got = _gpu(sv.SV_RULE_BLOCK, a, 0.9, 13, step)
        _assert_parity(ref, got, "block V=%d gamma=%d step=%d" % (V, gamma, step))


def test_block_one_draft_is_speculative_sampling_on_gpu():
    a = synth.accept_inputs(77, B=256, gamma=1, V=5000, target_var=3.0, noise_var=1.0, tau=0.8)
    blk = _gpu(sv.SV_RULE_BLOCK, a, 0.8, 3, 1)
    tok = _gpu(sv.SV_RULE_TOKEN, a, 0.8, 3, 1)
    assert np.array_equal(blk["accept_len"], tok["accept_len"]) and np.array_equal(blk["out_tokens"], tok["out_tokens"])


@pytest.mark.parametrize("wl", [2, 4])
def test_block_workload_parity(wl):
    cfg = synth.WORKLOADS[wl]
    a = synth.accept_inputs(wl, B=cfg["B"], gamma=cfg["gamma"], V=cfg["V"], target_var=cfg["target_var"],
                            noise_var=cfg["noise_var"], tau=cfg["tau"])
    for step in range(3 if wl == 4 else 10):
        ref = oracle.block_accept(a["target"], a["draft"], a["draft_tokens"], cfg["tau"], seed=1000 + wl, step=step)
        got = _gpu(sv.SV_RULE_BLOCK, a, cfg["tau"], 1000 + wl, step)
        _assert_parity(ref, got, "block workload %d step %d" % (wl, step))


def test_block_greedy_mode_is_greedy():
    a = synth.accept_inputs(78, B=64, gamma=4, V=3000, target_var=3.0, noise_var=0.3, tau=1.0, greedy_drafts=True)
    g = _gpu(sv.SV_RULE_BLOCK, a, 1.0, 0, mode=GREEDY)
    t = _gpu(sv.SV_RULE_TOKEN, a, 1.0, 0, mode=GREEDY)
    assert np.array_equal(g["out_tokens"], t["out_tokens"])


def _coupled_drafts(a, tau, seed, step, stream_ids=None):
    drafts, _ = oracle.gumbel_argmax(a["draft"], tau, seed=seed, step=step, stream_ids=stream_ids)
    return drafts


@pytest.mark.parametrize("V", [7, 1000, 4097, 12289, 128256])
@pytest.mark.parametrize("gamma", [1, 4, 16])
def test_gumbel_parity_shapes(V, gamma):
    B = 16 if V > 100000 else 64
    a = synth.accept_inputs(V + 5 * gamma, B=B, gamma=gamma, V=V, target_var=3.0, noise_var=0.5, tau=0.9)
    for step in range(2):
        x = _coupled_drafts(a, 0.9, 17, step)
        ref = oracle.gumbel_accept(a["target"], x, 0.9, seed=17, step=step)
        got = _gpu(sv.SV_RULE_GUMBEL, a, 0.9, 17, step, draft_tokens=x)
        _assert_parity(ref, got, "gumbel V=%d gamma=%d step=%d mean J=%.2f" % (V, gamma, step,
                                                                                ref["accept_len"].mean()))


@pytest.mark.parametrize("wl", [2, 4])
def test_gumbel_workload_parity(wl):
    cfg = synth.WORKLOADS[wl]
    a = synth.accept_inputs(wl, B=cfg["B"], gamma=cfg["gamma"], V=cfg["V"], target_var=cfg["target_var"],
                            noise_var=cfg["noise_var"], tau=cfg["tau"])
    sid = np.arange(cfg["B"], dtype=np.int64) * 31 + 7
    for step in range(3):
        x = _coupled_drafts(a, cfg["tau"], 2000 + wl, step, sid.astype(np.uint64))
        ref = oracle.gumbel_accept(a["target"], x, cfg["tau"], seed=2000 + wl, step=step, stream_ids=sid)
        got = _gpu(sv.SV_RULE_GUMBEL, a, cfg["tau"], 2000 + wl, step, stream_ids=sid, draft_tokens=x)
        _assert_parity(ref, got, "gumbel workload %d step %d" % (wl, step))


def test_gumbel_draws_follow_the_target_law_on_gpu():
    """The first emitted token of rounds whose first draft is always rejected is the GPU's
    own Gumbel-max sample of position 0: it follows softmax(l / T) (10^6 draws, V = 8)."""
    from scipy import special, stats
    V, N = 8, 1_000_000
    lg = (np.random.default_rng(35).standard_normal((2, V)) * 1.5).astype(np.float32)
    per = 25_000                      # rounds per call; each call uses its own Philox step
    tgt = torch.from_numpy(lg).cuda().expand(per, 2, V).contiguous()
    toks = torch.full((per, 1), -1, dtype=torch.int32, device="cuda")   # never a sample: J = 0
    parts = [to_host(sv.sv_spec_accept(SAMPLE, tgt, None, toks, 0.7, 5, k, rule=sv.SV_RULE_GUMBEL))
             for k in range(N // per)]
    got = {key: np.concatenate([q[key] for q in parts]) for key in ("out_tokens", "accept_len", "status")}
    counts = np.bincount(got["out_tokens"][:, 0], minlength=V)
    p = special.softmax(lg[0].astype(np.float64) / float(np.float32(0.7)))
    assert stats.chisquare(counts, p * N).pvalue > 1e-4
    assert np.all(got["accept_len"] == 0) and np.all(got["status"] == 2)


@pytest.mark.parametrize("same_chunk", [True, False])
def test_gumbel_near_ties_below_fp32_resolution(same_chunk):
    """Two contenders per row whose fp64 Gumbel scores l/T + g differ by less than an fp32
    ulp of the score (the second logit is the fp32 value nearest to a tie), far above the
    oracle's 1e-12 tie window: the GPU's winner is the fp64 one, at both positions, with
    the contenders in one 4096-token chunk or in two."""
    from np_philox import block as np_block, word_to_uniform
    B, V, seed, step = 128, 5000, 23, 4
    tau = float(np.float32(0.9))
    sid = np.arange(B, dtype=np.uint64) * 11 + 5
    r = np.random.default_rng(9 + same_chunk)

    def g(tok, b, pos):
        w = np_block([tok >> 2, step, int(sid[b]), oracle.TAG_GUMBEL + (pos << 32)], [seed, 0])[tok & 3]
        return -math.log(-math.log(word_to_uniform(w)))

    tgt = np.full((B, 2, V), -40.0, np.float32)
    toks = np.zeros((B, 1), np.int32)
    win = np.zeros((B, 2), np.int64)
    gaps = []
    for b in range(B):
        for pos in range(2):
            ta = int(r.integers(0, 2000))
            tb = int(r.integers(2100, 4000)) if same_chunk else int(r.integers(4096, V))
            la = np.float32(r.uniform(5.0, 12.0))
            lb = np.float32(float(la) + tau * (g(ta, b, pos) - g(tb, b, pos)))
            tgt[b, pos, ta], tgt[b, pos, tb] = la, lb
            gap = (float(la) / tau + g(ta, b, pos)) - (float(lb) / tau + g(tb, b, pos))
            gaps.append(abs(gap))
            win[b, pos] = ta if gap > 0 else tb
            if pos == 0:
                toks[b, 0] = ta if r.random() < 0.5 else tb
    gaps = np.array(gaps)
    assert gaps.max() < 2e-6 and gaps.min() > 1e-11, (gaps.min(), gaps.max())
    got = to_host(sv.sv_spec_accept(SAMPLE, dev_array(tgt), None, dev_array(toks), tau, seed, step,
                                    dev_array(sid.astype(np.int64)), rule=sv.SV_RULE_GUMBEL))
    ref = oracle.gumbel_accept(tgt, toks, tau, seed=seed, step=step, stream_ids=sid)
    _assert_parity(ref, got, "gumbel near ties same_chunk=%s" % same_chunk, excused_ok=0)
    J = (toks[:, 0] == win[:, 0]).astype(np.int64)
    assert np.array_equal(got["accept_len"], J)
    assert np.array_equal(got["out_tokens"][np.arange(B), J], win[np.arange(B), J])
    first = win[:, 0] == np.array([int(np.nonzero(tgt[b, 0] > -40)[0][0]) for b in range(B)])
    assert 0.2 < first.mean() < 0.8, first.mean()     # both contenders win often
