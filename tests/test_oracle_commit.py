"""Pins of the oracle's KV-cache commit.

"Speculative decoding" (textbook), section "Keeping the caches consistent after a
rejection": after a round the cache must hold exactly what a plain pass over the accepted
tokens would have written.  Two independent checks of that:

* simulation: a stand-in model whose key/value at a position depend on the tokens of the
  path leading to it (and the position); a tree pass writes every node's entry, a chain
  pass over the accepted tokens writes theirs, and after the commit the cache equals the
  chain pass's cache up to the new length;
* attention: a query attending to the committed cache under a causal mask equals the same
  query attending to the uncommitted cache under the tree mask of the accepted branch
  (torch's float64 scaled_dot_product_attention on both sides).

Chains only move the length pointer; bad lengths or paths leave a sequence untouched.
"""
import hashlib

import numpy as np
import pytest

import oracle
import synth


def _model_kv(tokens_on_path, position, Hkv, D):
    """Deterministic stand-in for a model: K and V of the last token of `tokens_on_path`
    at `position`, a function of the whole path (and nothing else)."""
    h = hashlib.sha256(repr((tuple(int(t) for t in tokens_on_path), int(position))).encode()).digest()
    r = np.random.default_rng(np.frombuffer(h[:16], dtype=np.uint64))
    return r.standard_normal((2, Hkv, D)).astype(np.float32)


def _path_tokens(parents, tokens, j):
    out = []
    while j >= 0:
        out.append(int(tokens[j]))
        j = parents[j]
    return out[::-1]


def _tree_round(seed, B, P_list, parents, Hkv, D, dtype):
    """Caches after a tree pass (prefix entries random, node j at P + j from the model),
    plus each sequence's node tokens and a random accepted path."""
    n = len(parents)
    r = np.random.default_rng(seed)
    depth = np.zeros(n, np.int64)
    for j in range(1, n):
        depth[j] = depth[parents[j]] + 1
    toks = r.integers(0, 1000, (B, n))
    tot = sum(P + n for P in P_list)
    k = np.zeros((tot, Hkv, D), np.float32)
    v = np.zeros((tot, Hkv, D), np.float32)
    kv_off = np.zeros(B, np.int64)
    paths = np.full((B, int(depth.max()) + 1), -1, np.int32)
    J = np.zeros(B, np.int32)
    o = 0
    for b, P in enumerate(P_list):
        kv_off[b] = o * Hkv * D
        k[o:o + P] = r.standard_normal((P, Hkv, D))
        v[o:o + P] = r.standard_normal((P, Hkv, D))
        for j in range(n):
            kv = _model_kv(_path_tokens(parents, toks[b], j), P + depth[j], Hkv, D)
            k[o + P + j], v[o + P + j] = kv[0], kv[1]
        leaf = int(r.integers(0, n))
        branch = []
        while leaf >= 0:
            branch.append(leaf)
            leaf = parents[leaf]
        branch = branch[::-1]
        J[b] = int(r.integers(0, len(branch)))
        paths[b, :J[b] + 1] = branch[:J[b] + 1]
        o += P + n
    k, v = k.reshape(-1), v.reshape(-1)
    if dtype == "bf16":
        k, v = synth.to_bf16_bits(k), synth.to_bf16_bits(v)
    return k, v, kv_off, toks, paths, J


def _widen(a):
    return synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tree", ["medusa", "random"])
def test_commit_equals_chain_pass_over_accepted_tokens(dtype, tree):
    Hkv, D = 2, 16
    if tree == "medusa":
        parents, _ = synth.build_tree(synth.WORKLOADS[3])
    else:
        parents = synth.random_tree(11, 40, branch_p=0.7)
    P_list = [0, 5, 33, 64]
    B, n = len(P_list), len(parents)
    k, v, kv_off, toks, paths, J = _tree_round(1, B, P_list, parents, Hkv, D, dtype)
    k2, v2, new_len, st = oracle.kv_commit(k, v, kv_off, P_list, J, n_q=n, Hkv=Hkv, D=D, kv_sh=D, kv_st=Hkv * D,
                                           path=paths)
    assert st == 0
    assert np.array_equal(new_len, np.array(P_list) + 1 + J)
    for b, P in enumerate(P_list):
        base = int(kv_off[b]) // (Hkv * D)
        got_k = _widen(k2).reshape(-1, Hkv, D)[base:base + P + 1 + J[b]]
        got_v = _widen(v2).reshape(-1, Hkv, D)[base:base + P + 1 + J[b]]
        old_k = _widen(k).reshape(-1, Hkv, D)[base:base + P]
        old_v = _widen(v).reshape(-1, Hkv, D)[base:base + P]
        assert np.array_equal(got_k[:P], old_k) and np.array_equal(got_v[:P], old_v)    # prefix untouched
        accepted = [int(toks[b, paths[b, i]]) for i in range(J[b] + 1)]
        for i in range(J[b] + 1):                 # a chain pass over the accepted tokens
            kv = _model_kv(accepted[:i + 1], P + i, Hkv, D)
            if dtype == "bf16":
                kv = synth.bf16_bits_to_f32(synth.to_bf16_bits(kv))
            assert np.array_equal(got_k[P + i], kv[0]) and np.array_equal(got_v[P + i], kv[1]), (b, i)


def test_commit_keeps_attention_of_the_accepted_branch():
    """softmax(q K^T) V over the committed cache (causal, P + 1 + J keys) equals the same
    query over the uncommitted cache under the accepted node's tree mask row."""
    torch = pytest.importorskip("torch")
    Hkv, D = 2, 32
    parents = synth.random_tree(12, 30, branch_p=0.8)
    P_list = [7, 40]
    B, n = len(P_list), len(parents)
    k, v, kv_off, toks, paths, J = _tree_round(2, B, P_list, parents, Hkv, D, "f32")
    k2, v2, new_len, st = oracle.kv_commit(k, v, kv_off, P_list, J, n_q=n, Hkv=Hkv, D=D, kv_sh=D, kv_st=Hkv * D,
                                           path=paths)
    bits, _, _ = oracle.tree_mask(parents, 0)
    q = np.random.default_rng(3).standard_normal((Hkv, 1, D))
    for b, P in enumerate(P_list):
        base = int(kv_off[b]) // (Hkv * D)
        node = int(paths[b, J[b]])
        mask = oracle.dense_mask(bits, n, P)[node]                        # prefix + ancestors-or-self
        K0 = torch.from_numpy(k.reshape(-1, Hkv, D)[base:base + P + n].transpose(1, 0, 2).astype(np.float64))
        V0 = torch.from_numpy(v.reshape(-1, Hkv, D)[base:base + P + n].transpose(1, 0, 2).astype(np.float64))
        L = int(new_len[b])
        K1 = torch.from_numpy(k2.reshape(-1, Hkv, D)[base:base + L].transpose(1, 0, 2).astype(np.float64))
        V1 = torch.from_numpy(v2.reshape(-1, Hkv, D)[base:base + L].transpose(1, 0, 2).astype(np.float64))
        qq = torch.from_numpy(q)
        tree_att = torch.nn.functional.scaled_dot_product_attention(
            qq, K0.contiguous(), V0.contiguous(), attn_mask=torch.from_numpy(mask[None, None, :]))
        chain_att = torch.nn.functional.scaled_dot_product_attention(qq, K1.contiguous(), V1.contiguous())
        assert L == int(mask.sum())
        assert torch.allclose(tree_att, chain_att, rtol=0, atol=1e-12)


def test_chain_commit_moves_only_the_length():
    inp = synth.attention_inputs(5, B=3, n_q=6, Hq=4, Hkv=2, D=64, prefix_len=[10, 0, 300], dtype="bf16")
    J = [0, 5, 3]
    k2, v2, new_len, st = oracle.kv_commit(inp["k"], inp["v"], inp["kv_off"], inp["prefix_len"], J, n_q=6, Hkv=2,
                                           D=64, kv_sh=inp["kv_sh"], kv_st=inp["kv_st"])
    assert st == 0 and list(new_len) == [11, 6, 304]
    assert np.array_equal(k2, inp["k"]) and np.array_equal(v2, inp["v"])


def test_bad_lengths_and_paths_leave_the_sequence_untouched():
    parents = np.array([-1, 0, 0, 1, 3])
    k, v, kv_off, toks, paths, J = _tree_round(3, 3, [4, 4, 4], parents, 1, 8, "f32")
    paths[:, :] = [0, 1, 3, 4]
    J[:] = [3, 5, 3]                        # sequence 1: J beyond the pass
    paths[2, 2] = 1                         # sequence 2: path node below its depth
    k2, v2, new_len, st = oracle.kv_commit(k, v, kv_off, [4, 4, 4], J, n_q=5, Hkv=1, D=8, kv_sh=8, kv_st=8,
                                           path=paths)
    assert st == 2 and list(new_len) == [8, 4, 4]
    seq = lambda a, b: a.reshape(3, 9, 8)[b]  # noqa: E731
    assert np.array_equal(seq(k2, 1), seq(k, 1)) and np.array_equal(seq(k2, 2), seq(k, 2))
    assert np.array_equal(seq(k2, 0)[5:8], seq(k, 0)[[5, 7, 8]])
