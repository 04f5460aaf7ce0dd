"""GPU parity of sv_build_tree_mask and sv_tree_walk against the fp64 oracle.

Masks, depths and position ids are bit-exact; walk paths and tokens are bit-exact except
in sequences the oracle flags as near-threshold draws (within 1e-10 of probability mass of
a CDF boundary: counted, reported, and at most 2 per call below 1000 walks, else 1e-3).
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

GREEDY, SAMPLE = sv.SV_GREEDY, sv.SV_SAMPLE


def _mask_on_gpu(parents, P):
    bits, depth, pos, st = sv.sv_build_tree_mask(dev_array(np.asarray(parents, np.int32)), P)
    torch.cuda.synchronize()
    return bits.cpu().numpy().view(np.uint32), depth.cpu().numpy(), pos.cpu().numpy(), int(st.cpu()[0])


@pytest.mark.parametrize("case", ["page", "chain1", "chain70", "random513", "forest", "medusa", "cartesian",
                                  "chain2500", "random9000"])
def test_tree_mask_parity(case):
    """Chains, random trees and forests up to 9000 nodes, the page's example and both workload trees."""
    P = 17
    if case == "chain2500":
        parents = np.arange(2500) - 1
    elif case == "random9000":
        parents = synth.random_tree(5, 9000, branch_p=0.9)
    elif case == "page":
        parents = np.array([-1, -1, 0, 0, 1, 2])
    elif case == "chain1":
        parents = np.array([-1])
    elif case == "chain70":
        parents = np.arange(70) - 1
    elif case == "random513":
        parents = synth.random_tree(3, 513, branch_p=0.8)
    elif case == "forest":
        parents = synth.random_tree(4, 300, branch_p=0.5)
        parents[[10, 77, 200]] = -1
    elif case == "medusa":
        parents, _ = synth.build_tree(synth.WORKLOADS[3])
    else:
        parents, _ = synth.build_tree(synth.WORKLOADS[5])
    bits, depth, pos = oracle.tree_mask(parents, P)
    gb, gd, gp, st = _mask_on_gpu(parents, P)
    assert st == 0
    assert np.array_equal(gb, bits) and np.array_equal(gd, depth) and np.array_equal(gp, pos)


@pytest.mark.parametrize("bad,first", [([-1, 0, 5, 1], 3), ([-1, 0, 1, -2, 7], 4), ([0], 1), ([-1, 1], 2)])
def test_tree_mask_bad_parents(bad, first):
    _, _, _, st = _mask_on_gpu(bad, 3)
    assert st == first


def _walk_both(mode, lg, toks, parents, tau, seed, step=0, stream_ids=None, max_depth=None):
    if max_depth is None:
        max_depth = int(oracle.tree_mask(parents, 0)[1].max())
    ref = oracle.tree_walk(mode, lg, toks, parents, tau, seed=seed, step=step, stream_ids=stream_ids,
                           max_depth=max_depth)
    got = to_host(sv.sv_tree_walk(mode, dev_array(lg), dev_array(toks.astype(np.int32)),
                                  dev_array(np.asarray(parents, np.int32)), max_depth, tau, seed, step,
                                  None if stream_ids is None else dev_array(np.asarray(stream_ids, np.int64))))
    return ref, got


def _assert_walk_parity(ref, got, label=""):
    flagged = ref["flags"] != 0
    same = ((ref["accept_len"] == got["accept_len"]) & np.all(ref["path"] == got["path"], 1)
            & np.all(ref["out_tokens"] == got["out_tokens"], 1))
    bad = ~same & ~flagged
    print("%s walks=%d near-threshold=%d mismatched(near)=%d mismatched(other)=%d mean J=%.3f"
          % (label, len(same), flagged.sum(), (~same & flagged).sum(), bad.sum(), got["accept_len"].mean()))
    assert not bad.any(), np.nonzero(bad)[0][:10]
    limit = 2 if len(same) < 1000 else int(1e-3 * len(same))
    assert flagged.sum() <= limit, (flagged.sum(), limit)
    assert np.all(got["status"] == 0)


@pytest.mark.parametrize("mode", [GREEDY, SAMPLE])
@pytest.mark.parametrize("seed,n,V,br", [(0, 12, 16, 0.5), (1, 65, 1000, 0.8), (2, 200, 4097, 0.9), (3, 40, 7, 0.3)])
def test_walk_parity_random_trees(mode, seed, n, V, br):
    parents = synth.random_tree(seed, n, branch_p=br)
    B = 32
    lg = synth.tree_logits(seed, B, n, V, 3.0)
    toks = synth.node_tokens(seed, lg, parents)
    for step in range(3):
        ref, got = _walk_both(mode, lg, toks, parents, 0.7, seed=21, step=step)
        _assert_walk_parity(ref, got, "seed %d step %d" % (seed, step))


@pytest.mark.parametrize("mode", [GREEDY, SAMPLE])
@pytest.mark.parametrize("fan", [100, 300])
def test_walk_wide_fanout(mode, fan):
    """A root with more children than the walk gathers in LDS (300) and with fewer (100),
    each child with one grandchild: the child lookup takes both of its forms."""
    parents = np.array([-1] + [0] * fan + list(range(1, fan + 1)), dtype=np.int64)
    B = 16
    lg = synth.tree_logits(fan, B, len(parents), 700, 3.0)
    toks = synth.node_tokens(fan, lg, parents)
    for step in range(2):
        ref, got = _walk_both(mode, lg, toks, parents, 0.8, seed=9, step=step)
        _assert_walk_parity(ref, got, "fan %d step %d" % (fan, step))


@pytest.mark.parametrize("mode", [GREEDY, SAMPLE])
def test_walk_workload_medusa(mode):
    cfg = synth.WORKLOADS[3]
    parents, paths = synth.build_tree(cfg)
    n = len(parents)
    lg = synth.tree_logits(3, 1, n, cfg["V"], cfg["target_var"])
    toks = synth.node_tokens(3, lg, parents, synth.path_ranks(paths))
    for step in range(10):
        ref, got = _walk_both(mode, lg, toks, parents, cfg["tau"], seed=1003, step=step)
        _assert_walk_parity(ref, got, "medusa step %d" % step)


@pytest.mark.parametrize("mode", [GREEDY, SAMPLE])
def test_walk_workload_cartesian_full(mode):
    cfg = synth.WORKLOADS[5]
    parents, paths = synth.build_tree(cfg)
    n = len(parents)
    lg = synth.tree_logits(5, 1, n, cfg["V"], cfg["target_var"])
    toks = synth.node_tokens(5, lg, parents, synth.path_ranks(paths))
    for step in range(4):
        ref, got = _walk_both(mode, lg, toks, parents, cfg["tau"], seed=1005, step=step)
        _assert_walk_parity(ref, got, "cartesian step %d" % step)


@pytest.mark.parametrize("mode", [GREEDY, SAMPLE])
def test_walk_too_deep_sets_status(mode):
    """max_depth below the tree's depth: the walk stops at the node at max_depth and emits
    the choice there (status 3); path and tokens equal the oracle's under the same cap."""
    parents = np.arange(4) - 1
    lg = np.zeros((2, 4, 3), dtype=np.float32)
    lg[:, :, 1] = 30.0                       # token 1 wins (and is sampled) at every node
    toks = np.ones((2, 4), dtype=np.int32)
    toks[1, 2] = 2                           # sequence 1 stops at depth 1 by itself
    got = to_host(sv.sv_tree_walk(mode, dev_array(lg), dev_array(toks), dev_array(parents.astype(np.int32)),
                                  2, 1.0, 0))
    ref = oracle.tree_walk(mode, lg, toks, parents, 1.0, seed=0, max_depth=2, allow_too_deep=True)
    assert ref["status"] == 3
    assert list(got["status"]) == [3, 0] and list(got["accept_len"]) == [2, 1]
    assert np.array_equal(got["path"], ref["path"]) and np.array_equal(got["out_tokens"], ref["out_tokens"])
    assert np.array_equal(got["accept_len"], ref["accept_len"])
    assert list(got["out_tokens"][0]) == [1, 1, 1]


def test_crafted_near_threshold_walk_draws():
    """Root draws placed 1e-11 ... 1e-9 from a CDF boundary: those outside the 1e-10 window
    match the oracle bit for bit; the flagged ones are exactly the crafted ones inside it."""
    from np_philox import uniform as np_uniform
    from test_oracle_flags import DRAW_DELTAS, STEPS, _logit3, _streams
    st = _streams(36)
    B = len(st)
    lg = np.zeros((B, 1, 3), np.float32)
    for b in range(B):
        lg[b, 0] = _logit3(np_uniform(201, 0, 2, int(st[b]), oracle.TAG_WALK) + DRAW_DELTAS[b % len(DRAW_DELTAS)])
    toks = np.zeros((B, 1), np.int32)
    ref, got = _walk_both(SAMPLE, lg, toks, np.array([-1]), 1.0, seed=201, step=2, stream_ids=st.astype(np.int64))
    near = np.array([abs(STEPS[b % len(STEPS)]) < 1.0 for b in range(B)])
    assert np.array_equal(ref["flags"] != 0, near)
    same = np.all(ref["out_tokens"] == got["out_tokens"], 1)
    assert same[~near].all()


def test_chain_tree_walk_equals_greedy_accept_on_gpu():
    B, gamma, V = 64, 5, 3000
    a = synth.accept_inputs(6, B=B, gamma=gamma, V=V, target_var=3.0, noise_var=0.2, tau=1.0, greedy_drafts=True)
    toks = np.concatenate([np.zeros((B, 1), np.int32), a["draft_tokens"]], 1)
    w = to_host(sv.sv_tree_walk(GREEDY, dev_array(a["target"]), dev_array(toks),
                                dev_array((np.arange(gamma + 1) - 1).astype(np.int32)), gamma, 1.0, 0))
    g = to_host(sv.sv_spec_accept(GREEDY, dev_array(a["target"]), None, dev_array(a["draft_tokens"]), 1.0, 0))
    assert np.array_equal(w["accept_len"], g["accept_len"])
    assert np.array_equal(w["out_tokens"], g["out_tokens"])
