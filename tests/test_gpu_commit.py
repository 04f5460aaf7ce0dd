"""GPU parity of sv_kv_commit against the oracle: the caches after the commit (every byte of
K and V), the new lengths and the status words are bit-exact.  Paths come from random
branches of the workload trees and of a deep random tree (several rounds of moves per
sequence), and from the GPU's own tree walk; chains move only the length; bad lengths and
paths leave their sequence untouched."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import draft_token_verification_attention_amd as sv  # noqa: E402
from svgpu import dense_cache, dev_array, to_host  # noqa: E402


def _random_paths(seed, parents, B, max_depth):
    r = np.random.default_rng(seed)
    n = len(parents)
    paths = np.full((B, max_depth + 1), -1, np.int32)
    J = np.zeros(B, np.int32)
    for b in range(B):
        leaf = int(r.integers(0, n))
        br = []
        while leaf >= 0:
            br.append(leaf)
            leaf = int(parents[leaf])
        br = br[::-1]
        J[b] = int(r.integers(0, len(br)))
        paths[b, :J[b] + 1] = br[:J[b] + 1]
    return paths, J


def _run(inp, J, paths, dense=False, in_place=True):
    bf = inp["dtype"] == "bf16"
    B, n_q, Hkv, D = inp["B"], inp["n_q"], inp["Hkv"], inp["D"]
    if dense:
        kd, vd, kv_sb = dense_cache(inp, int(inp["prefix_len"].max()) + n_q)
        k, v, kv_off = dev_array(kd, bf), dev_array(vd, bf), None
        hk, hv = kd, vd
        off = np.arange(B, dtype=np.int64) * kv_sb
    else:
        k, v, kv_sb = dev_array(inp["k"], bf), dev_array(inp["v"], bf), 0
        kv_off = dev_array(inp["kv_off"].astype(np.int64))
        hk, hv, off = inp["k"], inp["v"], inp["kv_off"]
    pl = dev_array(inp["prefix_len"].astype(np.int32))
    new_len, status = sv.sv_kv_commit(k, v, kv_off, pl, dev_array(np.asarray(J, np.int32)), n_q=n_q, Hkv=Hkv, D=D,
                                      kv_sh=inp["kv_sh"], kv_st=inp["kv_st"], kv_sb=kv_sb,
                                      path=None if paths is None else dev_array(paths), in_place=in_place)
    torch.cuda.synchronize()
    to_np = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if bf else (lambda t: t.cpu().numpy())
    ref_k, ref_v, ref_len, st = oracle.kv_commit(hk, hv, off, inp["prefix_len"], J, n_q=n_q, Hkv=Hkv, D=D,
                                                 kv_sh=inp["kv_sh"], kv_st=inp["kv_st"], path=paths)
    return dict(k=to_np(k), v=to_np(v), new_len=new_len.cpu().numpy(), status=status.cpu().numpy(),
                prefix=pl.cpu().numpy()), dict(k=ref_k, v=ref_v, new_len=ref_len, status=st)


def _assert_same(got, ref):
    assert np.array_equal(got["k"].view(np.uint8), ref["k"].view(np.uint8))
    assert np.array_equal(got["v"].view(np.uint8), ref["v"].view(np.uint8))
    assert np.array_equal(got["new_len"], ref["new_len"])


@pytest.mark.parametrize("tree", ["medusa", "cartesian", "deep"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tree_commit_parity(tree, dtype):
    if tree == "medusa":
        parents, _ = synth.build_tree(synth.WORKLOADS[3])
        B, P, Hkv, D = 6, [2048, 0, 1, 777, 64, 5000], 8, 128
    elif tree == "cartesian":
        parents, _ = synth.build_tree(synth.WORKLOADS[5])
        B, P, Hkv, D = 3, [300, 16384, 0], 8, 128
    else:
        parents = synth.random_tree(21, 300, branch_p=0.15)   # deep: paths of ~60 nodes, 8 rounds of moves
        B, P, Hkv, D = 5, [10, 0, 100, 3, 4096], 8, 128
    n = len(parents)
    depth = oracle.tree_mask(parents, 0)[1]
    paths, J = _random_paths(n, parents, B, int(depth.max()))
    inp = synth.attention_inputs(n + B, B=B, n_q=n, Hq=Hkv, Hkv=Hkv, D=D, prefix_len=P, dtype=dtype)
    got, ref = _run(inp, J, paths)
    assert ref["status"] == 0 and np.all(got["status"] == 0)
    _assert_same(got, ref)
    assert np.array_equal(got["prefix"], np.array(P) + 1 + J)          # updated in place


def test_commit_of_gpu_walk_paths():
    cfg = synth.WORKLOADS[3]
    parents, paths_r = synth.build_tree(cfg)
    n = len(parents)
    B = 4
    lg = synth.tree_logits(3, B, n, 4096, cfg["target_var"])
    toks = synth.node_tokens(3, lg, parents, synth.path_ranks(paths_r))
    maxd = int(oracle.tree_mask(parents, 0)[1].max())
    w = sv.sv_tree_walk(sv.SV_GREEDY, dev_array(lg), dev_array(toks), dev_array(parents.astype(np.int32)), maxd, 1.0, 0)
    inp = synth.attention_inputs(9, B=B, n_q=n, Hq=8, Hkv=8, D=128, prefix_len=[100, 200, 0, 31], dtype="bf16")
    got, ref = _run(inp, to_host(w)["accept_len"], to_host(w)["path"])
    _assert_same(got, ref)


@pytest.mark.parametrize("dense", [False, True])
def test_chain_commit_moves_only_the_length(dense):
    inp = synth.attention_inputs(4, B=5, n_q=6, Hq=8, Hkv=2, D=64, prefix_len=[10, 0, 300, 5, 7], dtype="bf16")
    got, ref = _run(inp, [0, 5, 3, 1, 2], None, dense=dense, in_place=False)
    assert list(got["new_len"]) == [11, 6, 304, 7, 10] and list(got["prefix"]) == [10, 0, 300, 5, 7]
    if not dense:
        _assert_same(got, ref)
        assert np.array_equal(got["k"], inp["k"])


def test_dense_tree_commit():
    parents = synth.random_tree(22, 50, branch_p=0.6)
    paths, J = _random_paths(5, parents, 4, int(oracle.tree_mask(parents, 0)[1].max()))
    inp = synth.attention_inputs(5, B=4, n_q=50, Hq=4, Hkv=4, D=64, prefix_len=[40, 0, 12, 40], dtype="f32")
    got, ref = _run(inp, J, paths, dense=True)
    # the oracle works on the same dense copy (kv_off = b * kv_sb; unused slots hold NaN,
    # hence the byte comparison)
    _assert_same(got, ref)


def test_bad_inputs_set_status_and_leave_the_sequence():
    parents = np.array([-1, 0, 0, 1, 3])
    inp = synth.attention_inputs(6, B=3, n_q=5, Hq=2, Hkv=2, D=64, prefix_len=[4, 4, 4], dtype="bf16")
    paths = np.array([[0, 1, 3, 4]] * 3, np.int32)
    paths[2, 2] = 1
    got, ref = _run(inp, [3, 5, 3], paths)
    assert list(got["status"]) == [0, 4, 4] and ref["status"] == 2
    _assert_same(got, ref)
    assert list(got["prefix"]) == [8, 4, 4]
