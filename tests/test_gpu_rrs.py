"""GPU parity of sv_tree_walk's recursive-rejection rules (SV_WALK_RRS, SV_WALK_RRS_WOR)
against the oracle: accepted lengths, paths and emitted tokens bit-exact on the same
uniforms except in walks the oracle flags near a threshold (bounded as for the other
rules).  Children tokens are drawn by the test's own sampler from the drafter's
distribution at their parent (i.i.d., or without replacement); the GPU's own output at a
node follows p (chi-square over 10^6 rounds)."""
import numpy as np
import pytest
from scipy import special

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import draft_token_verification_attention_amd as sv  # noqa: E402
from svgpu import dev_array, to_host  # noqa: E402

SAMPLE, GREEDY = sv.SV_SAMPLE, sv.SV_GREEDY


def _draft_children(seed, draft, parents, tau, wor):
    """Node tokens: each node's children drawn from softmax(draft[parent] / tau), i.i.d. or
    without replacement, in node order (the root's token is arbitrary)."""
    B, n, V = draft.shape
    r = np.random.default_rng(seed)
    toks = np.zeros((B, n), np.int32)
    kids = {}
    for c in range(1, n):
        kids.setdefault(int(parents[c]), []).append(c)
    for b in range(B):
        for v, cs in kids.items():
            q = special.softmax(draft[b, v].astype(np.float64) / float(np.float32(tau)))
            if wor and len(cs) <= V:
                pick = r.choice(V, size=len(cs), replace=False, p=q)
            else:
                pick = r.choice(V, size=len(cs), replace=True, p=q)
            toks[b, cs] = pick
    return toks


def _both(target, draft, toks, parents, tau, seed, step, wor, max_children, stream_ids=None, mode=SAMPLE):
    maxd = int(oracle.tree_mask(parents, 0)[1].max())
    ref = oracle.tree_rrs(target, draft, toks, parents, tau, seed=seed, step=step, stream_ids=stream_ids,
                          max_depth=maxd, without_replacement=wor)
    got = to_host(sv.sv_tree_walk(mode, dev_array(target), dev_array(toks), dev_array(np.asarray(parents, np.int32)),
                                  maxd, tau, seed, step,
                                  None if stream_ids is None else dev_array(np.asarray(stream_ids, np.int64)),
                                  rule=sv.SV_WALK_RRS_WOR if wor else sv.SV_WALK_RRS, draft_logits=dev_array(draft),
                                  max_children=max_children))
    return ref, got


def _assert_rrs(ref, got, label):
    flagged = ref["flags"] != 0
    same = ((ref["accept_len"] == got["accept_len"]) & np.all(ref["path"] == got["path"], 1)
            & np.all(ref["out_tokens"] == got["out_tokens"], 1))
    bad = ~same & ~flagged
    print("%s walks=%d near-threshold=%d mismatched(near)=%d mismatched(other)=%d mean J=%.3f"
          % (label, len(same), flagged.sum(), (~same & flagged).sum(), bad.sum(), got["accept_len"].mean()))
    assert not bad.any(), np.nonzero(bad)[0][:10]
    assert flagged.sum() <= (2 if len(same) < 1000 else int(1e-3 * len(same)))
    assert np.all(got["status"] == 0)


def _max_kids(parents):
    return int(np.bincount(np.asarray(parents)[1:], minlength=len(parents)).max())


@pytest.mark.parametrize("wor", [False, True])
@pytest.mark.parametrize("seed,n,V,br", [(0, 12, 16, 0.6), (1, 65, 1000, 0.8), (2, 150, 4097, 0.9), (3, 40, 7, 0.5)])
def test_rrs_parity_random_trees(wor, seed, n, V, br):
    parents = synth.random_tree(seed, n, branch_p=br)
    B = 32
    tgt = synth.tree_logits(seed, B, n, V, 3.0)
    dr = (tgt + np.random.default_rng(seed + 50).standard_normal(tgt.shape).astype(np.float32)).astype(np.float32)
    toks = _draft_children(seed, dr, parents, 0.8, wor)
    for step in range(2):
        ref, got = _both(tgt, dr, toks, parents, 0.8, 31, step, wor, _max_kids(parents))
        _assert_rrs(ref, got, "rrs wor=%d seed %d step %d" % (wor, seed, step))


@pytest.mark.parametrize("wor", [False, True])
def test_rrs_workload_medusa(wor):
    cfg = synth.WORKLOADS[3]
    parents, _ = synth.build_tree(cfg)
    n = len(parents)
    B = 2
    tgt = synth.tree_logits(3, B, n, cfg["V"], cfg["target_var"])
    dr = (tgt + np.random.default_rng(77).standard_normal(tgt.shape).astype(np.float32)).astype(np.float32)
    toks = _draft_children(3, dr, parents, cfg["tau"], wor)
    for step in range(4):
        ref, got = _both(tgt, dr, toks, parents, cfg["tau"], 1003, step, wor, _max_kids(parents))
        _assert_rrs(ref, got, "medusa rrs wor=%d step %d" % (wor, step))


def test_rrs_small_cartesian_full_vocab():
    paths = synth.cartesian_paths(3, 4)
    parents, _ = synth.tree_from_rank_paths(paths)
    n = len(parents)
    tgt = synth.tree_logits(5, 1, n, 128256, 3.0)
    dr = (tgt + np.random.default_rng(78).standard_normal(tgt.shape).astype(np.float32)).astype(np.float32)
    toks = _draft_children(5, dr, parents, 0.7, False)
    for step in range(3):
        ref, got = _both(tgt, dr, toks, parents, 0.7, 1005, step, False, 4)
        _assert_rrs(ref, got, "cartesian rrs step %d" % step)


def test_rrs_output_law_on_gpu():
    """One node, four i.i.d. children drawn from q: the first emitted token follows p."""
    from scipy import stats
    V, k, per, calls = 8, 4, 25_000, 40
    r = np.random.default_rng(79)
    tl = (r.standard_normal(V) * 1.4).astype(np.float32)
    dl = (tl + r.standard_normal(V)).astype(np.float32)
    p, q = special.softmax(tl.astype(np.float64)), special.softmax(dl.astype(np.float64))
    parents = np.array([-1] + [0] * k, np.int32)
    tgt = torch.from_numpy(tl).cuda().expand(per, k + 1, V).contiguous()
    dr = torch.from_numpy(dl).cuda().expand(per, k + 1, V).contiguous()
    firsts = []
    for call in range(calls):
        kids = r.choice(V, size=(per, k), p=q)
        toks = np.concatenate([np.zeros((per, 1), np.int64), kids], 1).astype(np.int32)
        got = to_host(sv.sv_tree_walk(SAMPLE, tgt, dev_array(toks), dev_array(parents), 1, 1.0, 9, call,
                                      rule=sv.SV_WALK_RRS, draft_logits=dr, max_children=k))
        firsts.append(got["out_tokens"][:, 0])
    counts = np.bincount(np.concatenate(firsts), minlength=V)
    assert stats.chisquare(counts, p * per * calls).pvalue > 1e-4


def test_rrs_too_many_children_sets_status():
    parents = np.array([-1, 0, 0, 0, 1], np.int32)
    tgt = synth.tree_logits(6, 2, 5, 64, 2.0)
    toks = np.ones((2, 5), np.int32)
    got = to_host(sv.sv_tree_walk(SAMPLE, dev_array(tgt), dev_array(toks), dev_array(parents), 2, 1.0, 0,
                                  rule=sv.SV_WALK_RRS, draft_logits=dev_array(tgt), max_children=2))
    assert list(got["status"]) == [5, 5] and list(got["accept_len"]) == [0, 0]


def test_rrs_rule_under_greedy_is_the_greedy_walk():
    parents = synth.random_tree(8, 30, branch_p=0.7)
    tgt = synth.tree_logits(8, 8, 30, 500, 3.0)
    toks = synth.node_tokens(8, tgt, parents)
    a = to_host(sv.sv_tree_walk(GREEDY, dev_array(tgt), dev_array(toks), dev_array(parents.astype(np.int32)),
                                int(oracle.tree_mask(parents, 0)[1].max()), 1.0, 0, rule=sv.SV_WALK_RRS,
                                draft_logits=dev_array(tgt), max_children=_max_kids(parents)))
    ref = oracle.tree_walk(oracle.GREEDY, tgt, toks, parents, 1.0, seed=0)
    assert np.array_equal(a["path"], ref["path"]) and np.array_equal(a["out_tokens"], ref["out_tokens"])
