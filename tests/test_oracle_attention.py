"""Pins of the oracle's verify attention.

Against: torch's float64 scaled_dot_product_attention on CPU with an explicit
boolean mask (a library routine); per-path brute force (a tree row equals the
row obtained by running its root-to-node path alone as a causal chain over the
same prefix); closed-form special cases.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _to_f64(a, dtype):
    return torch.from_numpy(synth.bf16_bits_to_f32(a) if dtype == "bf16" else a).double()


def _sdpa_reference(inp, scale, dense_masks):
    """torch SDPA in float64, one sequence at a time, K/V heads repeated for GQA."""
    B, n_q, Hq, Hkv, D = inp["B"], inp["n_q"], inp["Hq"], inp["Hkv"], inp["D"]
    G = Hq // Hkv
    q = _to_f64(inp["q"], inp["dtype"]).reshape(B, n_q, Hq, D)
    k = _to_f64(inp["k"], inp["dtype"])
    v = _to_f64(inp["v"], inp["dtype"])
    outs, lses = [], []
    for b in range(B):
        P = int(inp["prefix_len"][b])
        T = P + n_q
        off = int(inp["kv_off"][b])
        kb = k[off:off + T * Hkv * D].reshape(T, Hkv, D).permute(1, 0, 2).repeat_interleave(G, dim=0)
        vb = v[off:off + T * Hkv * D].reshape(T, Hkv, D).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qb = q[b].permute(1, 0, 2)                                      # [Hq][n_q][D]
        m = torch.from_numpy(dense_masks[b])                            # [n_q][T] bool
        o = torch.nn.functional.scaled_dot_product_attention(qb, kb, vb, attn_mask=m, scale=scale)
        s = (qb @ kb.transpose(1, 2)) * scale
        s = s.masked_fill(~m, -math.inf)
        lses.append(torch.logsumexp(s, dim=-1).permute(1, 0).numpy())  # [n_q][Hq]
        outs.append(o.permute(1, 0, 2).numpy())                         # [n_q][Hq][D]
    return np.stack(outs), np.stack(lses)


def _chain_masks(inp):
    n = inp["n_q"]
    return [np.tril(np.ones((n, int(P) + n), dtype=bool), k=int(P)) for P in inp["prefix_len"]]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("B,n_q,Hq,Hkv,D,P", [
    (1, 1, 2, 2, 64, 0), (1, 5, 2, 2, 64, 128), (2, 6, 8, 2, 128, 63), (1, 17, 4, 1, 64, 65),
    (3, 2, 4, 4, 128, [1, 64, 9]),
])
def test_chain_matches_torch_sdpa(dtype, B, n_q, Hq, Hkv, D, P):
    pl = np.broadcast_to(np.array(P, dtype=np.int32), (B,)).copy()
    inp = synth.attention_inputs(11, B=B, n_q=n_q, Hq=Hq, Hkv=Hkv, D=D, prefix_len=pl, dtype=dtype)
    scale = 1.0 / math.sqrt(D)
    out, lse, _ = oracle.attention(inp, scale=scale)
    ref, ref_lse = _sdpa_reference(inp, scale, _chain_masks(inp))
    assert np.allclose(out.reshape(ref.shape), ref, rtol=0, atol=1e-12)
    assert np.allclose(lse.reshape(ref_lse.shape), ref_lse, rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed,n,P,Hq,Hkv", [(0, 6, 5, 2, 1), (1, 40, 33, 4, 2), (2, 65, 64, 8, 2)])
def test_tree_matches_torch_sdpa(seed, n, P, Hq, Hkv):
    parents = synth.random_tree(seed, n, branch_p=0.7)
    bits, _, _ = oracle.tree_mask(parents, P)
    dense = oracle.dense_mask(bits, n, P)
    B = 2
    inp = synth.attention_inputs(seed, B=B, n_q=n, Hq=Hq, Hkv=Hkv, D=64, prefix_len=[P, P], dtype="bf16")
    scale = 0.125
    out, lse, _ = oracle.attention(inp, scale=scale, tree_bits=bits, tree_sb=0)
    ref, ref_lse = _sdpa_reference(inp, scale, [dense, dense])
    assert np.allclose(out.reshape(ref.shape), ref, rtol=0, atol=1e-12)
    assert np.allclose(lse.reshape(ref_lse.shape), ref_lse, rtol=0, atol=1e-12)


def test_tree_row_equals_its_path_as_a_chain():
    """Brute force: each node's row equals the last row of a causal chain pass over
    (prefix, root-to-node path) with the same keys and values."""
    n, P, Hq, Hkv, D = 30, 20, 4, 2, 64
    parents = synth.random_tree(5, n, branch_p=0.6)
    bits, depth, _ = oracle.tree_mask(parents, P)
    inp = synth.attention_inputs(5, B=1, n_q=n, Hq=Hq, Hkv=Hkv, D=D, prefix_len=[P], dtype="bf16",
                                 qkv_scale=1.0)
    out, _, rows = oracle.attention(inp, scale=0.2, tree_bits=bits)
    out = out.reshape(1, n, Hq, D)
    k = inp["k"].reshape(P + n, Hkv, D)
    v = inp["v"].reshape(P + n, Hkv, D)
    q = inp["q"].reshape(1, n, Hq, D)
    for i in range(n):
        path = []
        j = i
        while j >= 0:
            path.append(j)
            j = parents[j]
        path = path[::-1]
        L = len(path)
        sel = list(range(P)) + [P + j for j in path]
        sub = dict(inp)
        sub.update(q=np.ascontiguousarray(q[:, path]), k=np.ascontiguousarray(k[sel]).ravel(),
                   v=np.ascontiguousarray(v[sel]).ravel(), n_q=L, kv_off=np.zeros(1, np.int64),
                   q_sb=L * Hq * D)
        sub_out, _, _ = oracle.attention(sub, scale=0.2)
        sub_out = sub_out.reshape(1, L, Hq, D)
        assert np.allclose(out[0, i], sub_out[0, L - 1], rtol=0, atol=1e-12)


def test_causal_equals_tree_of_a_chain():
    n, P = 9, 40
    inp = synth.attention_inputs(3, B=2, n_q=n, Hq=4, Hkv=2, D=128, prefix_len=[P, P], dtype="bf16")
    bits, _, _ = oracle.tree_mask(np.arange(n) - 1, P)
    a, la, _ = oracle.attention(inp, scale=0.09)
    b, lb, _ = oracle.attention(inp, scale=0.09, tree_bits=bits)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_single_visible_key_returns_its_value():
    """P = 0, one query row: the row sees only itself, so O is its own V row exactly."""
    inp = synth.attention_inputs(4, B=1, n_q=1, Hq=3, Hkv=1, D=64, prefix_len=[0], dtype="f32")
    out, lse, _ = oracle.attention(inp, scale=0.3)
    vrow = inp["v"].reshape(1, 1, 64).astype(np.float64)[0, 0]
    for h in range(3):
        assert np.array_equal(out[h], vrow)
        qk = float(np.dot(inp["q"].reshape(1, 1, 3, 64)[0, 0, h].astype(np.float64),
                          inp["k"].astype(np.float64)))
        assert abs(lse[h] - 0.3 * qk) < 1e-12


def test_identical_keys_give_mean_of_visible_values():
    n, P, D = 4, 10, 64
    inp = synth.attention_inputs(6, B=1, n_q=n, Hq=2, Hkv=1, D=D, prefix_len=[P], dtype="f32")
    k = inp["k"].reshape(P + n, 1, D)
    k[:] = k[0]
    inp["k"] = k.ravel()
    out, lse, _ = oracle.attention(inp, scale=0.5)
    out = out.reshape(n, 2, D)
    vv = inp["v"].reshape(P + n, D).astype(np.float64)
    for i in range(n):
        want = vv[: P + i + 1].mean(axis=0)
        assert np.allclose(out[i, 0], want, rtol=0, atol=1e-12)
        assert np.allclose(out[i, 1], want, rtol=0, atol=1e-12)
