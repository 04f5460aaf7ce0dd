"""GPU parity of sv_verify_attention against the fp64 oracle.

Tolerances (max-abs against fp64): 2e-2 for bf16 inputs, 1e-4 for fp32; the log-sum-exp
within 1e-3 (bf16) / 1e-5 (fp32).  Besides the workloads' own input scale, every shape
also runs with unscaled N(0,1) Q/K/V and with a 3x query scale, so the softmax is far
from uniform and the running-max rescaling is exercised.
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

from svgpu import attention_on_gpu, rows_of  # noqa: E402

BF16_TOL, F32_TOL = 2e-2, 1e-4


def _compare(inp, scale, tree_bits=None, tree_sb=0, rows=None, split_keys=0, max_prefix=None, dense=False):
    tol = BF16_TOL if inp["dtype"] == "bf16" else F32_TOL
    ltol = 1e-3 if inp["dtype"] == "bf16" else 1e-5
    ref, ref_lse, rows = oracle.attention(inp, scale=scale, tree_bits=tree_bits, tree_sb=tree_sb, rows=rows)
    out, lse = attention_on_gpu(inp, scale, tree_bits=tree_bits, tree_sb=tree_sb, split_keys=split_keys,
                                max_prefix=max_prefix, dense=dense)
    got = rows_of(out, rows)
    got_lse = rows_of(lse, rows)
    err = np.abs(got - ref).max()
    lerr = np.abs(got_lse - ref_lse).max()
    scale_o = np.abs(ref).max()
    print("rows=%d max_abs=%.3g (max|O|=%.3g) lse_err=%.3g" % (len(rows), err, scale_o, lerr))
    assert np.isfinite(got).all()
    assert err <= tol, err
    assert lerr <= ltol, lerr
    # relative to the output's own scale (bf16 outputs round to 2^-9 of each element): this
    # keeps the check meaningful where |O| is far below the absolute bound
    if inp["dtype"] == "bf16" and scale_o > 0:
        assert err / scale_o <= 1e-2, err / scale_o
    return err


CHAIN_SHAPES = [
    # B, n_q, Hq, Hkv, D, prefix lengths
    (1, 5, 2, 2, 64, [128]),
    (1, 1, 8, 8, 128, [0]),
    (1, 6, 32, 8, 128, [4096]),
    (2, 2, 4, 1, 64, [1, 63]),
    (3, 5, 32, 8, 128, [64, 65, 1000]),
    (1, 17, 8, 2, 128, [333]),
    (2, 8, 8, 1, 64, [31, 2047]),
    (1, 5, 4, 4, 128, [5000]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", CHAIN_SHAPES, ids=lambda s: "B%d_nq%d_H%d-%d_D%d_P%s" % (s[0], s[1], s[2], s[3], s[4], s[5]))
@pytest.mark.parametrize("qkv", ["unit", "workload", "sharp"])
def test_chain_parity(dtype, shape, qkv):
    B, n_q, Hq, Hkv, D, P = shape
    qkv_scale = {"unit": 1.0, "workload": 1 / math.sqrt(128), "sharp": 1.0}[qkv]
    q_scale = 3.0 if qkv == "sharp" else 1.0
    inp = synth.attention_inputs(7 + B + n_q, B=B, n_q=n_q, Hq=Hq, Hkv=Hkv, D=D, prefix_len=P, dtype=dtype,
                                 qkv_scale=qkv_scale, q_scale=q_scale)
    _compare(inp, 1.0 / math.sqrt(D))


@pytest.mark.parametrize("split_keys", [32, 128, 1000, 8192])
def test_chain_split_variants(split_keys):
    inp = synth.attention_inputs(21, B=2, n_q=6, Hq=32, Hkv=8, D=128, prefix_len=[4096, 777], dtype="bf16")
    _compare(inp, 1 / math.sqrt(128), split_keys=split_keys)


def test_workload_8b_chain_full():
    cfg = synth.WORKLOADS[2]
    n_q = cfg["gamma"] + 1
    inp = synth.attention_inputs(2, B=1, n_q=n_q, Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"],
                                 prefix_len=synth.prefix_lengths(2, cfg), dtype="bf16", qkv_scale=cfg["qkv_scale"])
    _compare(inp, 1 / math.sqrt(cfg["D"]))


def test_workload_tiny_fp32_full():
    cfg = synth.WORKLOADS[1]
    inp = synth.attention_inputs(1, B=1, n_q=cfg["gamma"] + 1, Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"],
                                 prefix_len=synth.prefix_lengths(1, cfg), dtype="f32")
    _compare(inp, 1 / math.sqrt(cfg["D"]))


@pytest.mark.parametrize("qkv", ["unit", "workload"])
def test_workload_batched_chain_all_rows(qkv):
    """Every one of the 64 x 5 x 32 = 10,240 rows of the batched workload, in the launch
    configuration the benchmark times (ragged cache, max_prefix 8192, default plan)."""
    cfg = synth.WORKLOADS[4]
    n_q = cfg["gamma"] + 1
    P = synth.prefix_lengths(4, cfg)
    inp = synth.attention_inputs(4, B=cfg["B"], n_q=n_q, Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"], prefix_len=P,
                                 dtype="bf16", qkv_scale=1.0 if qkv == "unit" else cfg["qkv_scale"])
    _compare(inp, 1 / math.sqrt(cfg["D"]), max_prefix=cfg["P_hi"])


TREE_CASES = [
    # seed, n, P, Hq, Hkv, D, branch
    (0, 6, 7, 2, 1, 64, 0.7),
    (1, 33, 100, 8, 2, 128, 0.6),
    (2, 65, 2048, 32, 8, 128, 0.8),
    (3, 200, 64, 4, 4, 64, 0.9),
    (4, 1, 50, 8, 8, 128, 0.5),
]


@pytest.mark.parametrize("case", TREE_CASES, ids=lambda c: "n%d_P%d_H%d-%d_D%d" % c[1:6])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tree_parity(case, dtype):
    seed, n, P, Hq, Hkv, D, br = case
    parents = synth.random_tree(seed, n, branch_p=br)
    if n > 10:
        parents[7] = -1                           # a forest
    bits, _, _ = oracle.tree_mask(parents, P)
    inp = synth.attention_inputs(seed, B=2, n_q=n, Hq=Hq, Hkv=Hkv, D=D, prefix_len=[P, P // 2 + 1], dtype=dtype)
    _compare(inp, 1 / math.sqrt(D), tree_bits=bits, tree_sb=0)


def test_tree_per_sequence_masks():
    n, P = 40, 300
    bits = [oracle.tree_mask(synth.random_tree(s, n, branch_p=0.5 + 0.1 * s), P)[0] for s in range(3)]
    tb = np.stack(bits)
    inp = synth.attention_inputs(9, B=3, n_q=n, Hq=16, Hkv=4, D=128, prefix_len=[P, P, P], dtype="bf16")
    _compare(inp, 1 / math.sqrt(128), tree_bits=tb, tree_sb=tb.shape[1] * tb.shape[2])


def test_chain_equals_tree_of_chain_on_gpu():
    n, P = 9, 500
    inp = synth.attention_inputs(5, B=2, n_q=n, Hq=8, Hkv=2, D=128, prefix_len=[P, P], dtype="bf16", qkv_scale=1.0)
    bits, _, _ = oracle.tree_mask(np.arange(n) - 1, P)
    a, la = attention_on_gpu(inp, 0.1)
    b, lb = attention_on_gpu(inp, 0.1, tree_bits=bits)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_workload_medusa_tree_full():
    cfg = synth.WORKLOADS[3]
    parents, _ = synth.build_tree(cfg)
    n = len(parents)
    bits, _, _ = oracle.tree_mask(parents, cfg["P"])
    inp = synth.attention_inputs(3, B=1, n_q=n, Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"],
                                 prefix_len=[cfg["P"]], dtype="bf16", qkv_scale=1.0)
    _compare(inp, 1 / math.sqrt(cfg["D"]), tree_bits=bits)


def test_workload_cartesian_tree_sampled_rows():
    cfg = synth.WORKLOADS[5]
    parents, _ = synth.build_tree(cfg)
    n = len(parents)
    bits, _, _ = oracle.tree_mask(parents, cfg["P"])
    inp = synth.attention_inputs(5, B=1, n_q=n, Hq=cfg["Hq"], Hkv=cfg["Hkv"], D=cfg["D"],
                                 prefix_len=[cfg["P"]], dtype="bf16", qkv_scale=1.0)
    r = np.random.default_rng(1)
    G = cfg["Hq"] // cfg["Hkv"]
    nodes = np.concatenate([np.arange(10), r.integers(0, n, 2000), np.arange(n - 10, n)])
    rows = np.stack([np.zeros_like(nodes), nodes, r.integers(0, cfg["Hq"], len(nodes))], 1)
    # one whole 128-row tile of KV head 3: nodes 1600..1615 x its 8 query heads
    ii, gg = np.meshgrid(np.arange(1600, 1600 + 128 // G), np.arange(G), indexing="ij")
    tile = np.stack([np.zeros(ii.size, np.int64), ii.ravel(), 3 * G + gg.ravel()], 1)
    _compare(inp, 1 / math.sqrt(cfg["D"]), tree_bits=bits, rows=np.concatenate([rows, tile]))


@pytest.mark.parametrize("n,P", [(129, 2048), (129, 9000), (33, 9000)], ids=["short-64row", "long-128row", "long-pad64"])
def test_tree_default_plans(n, P):
    """Default plans of the many-row forms: 64-row blocks on a short cache, 128-row blocks
    split to several blocks per CU on a long one, 64-row blocks padding fewer rows there."""
    parents = synth.random_tree(n + P, n, branch_p=0.6)
    bits, _, _ = oracle.tree_mask(parents, P)
    inp = synth.attention_inputs(n + 1, B=1, n_q=n, Hq=32, Hkv=8, D=128, prefix_len=[P], dtype="bf16", qkv_scale=1.0)
    r = np.random.default_rng(2)
    nodes = np.concatenate([np.arange(4), r.integers(0, n, 60), np.arange(n - 4, n)])
    rows = np.stack([np.zeros_like(nodes), nodes, r.integers(0, 32, len(nodes))], 1)
    _compare(inp, 1 / math.sqrt(128), tree_bits=bits, rows=rows)


MANY_ROW_CASES = [
    # name, seed, B, n_q, prefix lengths, Hq, Hkv, D, tree, split_keys, dense (max_prefix), q_scale
    ("tree-P7001-splits", 31, 1, 300, [7001], 32, 8, 128, True, 0, None, 1.0),
    ("tree-P7001-nosplit-sharp", 32, 1, 300, [7001], 32, 8, 128, True, 32768, None, 3.0),
    ("chain-nq48-B2", 33, 2, 48, [6500, 7003], 64, 8, 128, False, 0, None, 1.0),
    ("tree-D64", 34, 1, 150, [6300], 16, 2, 64, True, 0, None, 1.0),
    ("tree-dense-B2-sharp", 35, 2, 100, [6200, 6900], 64, 8, 128, True, 2048, 6950, 3.0),
]


def _tile_rows(inp, b, kvh, rt):
    """The (sequence, token, query head) triples of one 128-row tile of KV head kvh (rows are
    packed as token * G + g over the query heads of that KV head)."""
    G = inp["Hq"] // inp["Hkv"]
    r = np.arange(128 * rt, min(128 * (rt + 1), inp["n_q"] * G))
    return np.stack([np.full(r.size, b), r // G, kvh * G + r % G], 1)


@pytest.mark.parametrize("case", MANY_ROW_CASES, ids=lambda c: c[0])
def test_many_row_blocks(case):
    """128-row blocks on long caches (the software-pipelined kernel): tile masks from tree
    bits or the causal rule, a prefix that ends inside a tile, key splits and none, D = 64,
    the dense layout, and a sharp softmax that moves the running max."""
    name, seed, B, n, P, Hq, Hkv, D, tree, sk, mp, qs = case
    bits = None
    if tree:
        parents = synth.random_tree(seed, n, branch_p=0.6)
        parents[n // 3] = -1                      # a forest
        bits, _, _ = oracle.tree_mask(parents, P[0])
    inp = synth.attention_inputs(seed, B=B, n_q=n, Hq=Hq, Hkv=Hkv, D=D, prefix_len=P, dtype="bf16",
                                 qkv_scale=1.0, q_scale=qs)
    rows = np.concatenate([rows_of_sample(inp, 300), _tile_rows(inp, B - 1, Hkv - 1, 1),
                           _tile_rows(inp, 0, 0, (n * Hq // Hkv - 1) // 128)])
    _compare(inp, 1 / math.sqrt(D), tree_bits=bits, rows=rows, split_keys=sk, max_prefix=mp, dense=mp is not None)


@pytest.mark.parametrize("B,P", [(16, 1000), (8, 3000), (4, 5000)], ids=["no-split", "1024-split-B8", "1024-split-B4"])
def test_chain_batch_default_plans(B, P):
    """Default plans of the one-row-wave form for batches: one split per sequence on a short
    cache, at least 1024-key splits on longer ones."""
    inp = synth.attention_inputs(B * 7 + P, B=B, n_q=6, Hq=32, Hkv=8, D=128, prefix_len=[P - 3 * b for b in range(B)],
                                 dtype="bf16", qkv_scale=1.0)
    _compare(inp, 1 / math.sqrt(128), rows=rows_of_sample(inp, 120))


DENSE_SHAPES = [
    # B, n_q, Hq, Hkv, D, prefix lengths, max_prefix (token slots per sequence = max_prefix + n_q)
    (1, 6, 32, 8, 128, [4096], 4096),     # the 8B chain: first tiles loaded before the length
    (1, 6, 32, 8, 128, [4000], 4100),     # slots past the sequence hold NaN and are read
    (3, 5, 32, 8, 128, [64, 65, 1000], 1100),
    (2, 8, 8, 1, 64, [31, 2047], 2047),
    (40, 4, 32, 8, 128, [int(x) for x in np.linspace(3, 700, 40)], 720),  # grid beyond one block per CU
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", DENSE_SHAPES, ids=lambda s: "B%d_nq%d_D%d_mp%d" % (s[0], s[1], s[4], s[6]))
def test_dense_layout_parity(dtype, shape):
    """kv_off NULL: sequence b at b*kv_sb; every unused token slot of the cache is NaN."""
    B, n_q, Hq, Hkv, D, P, mp = shape
    inp = synth.attention_inputs(21, B=B, n_q=n_q, Hq=Hq, Hkv=Hkv, D=D, prefix_len=P, dtype=dtype, qkv_scale=1.0)
    rows = None if B * n_q * Hq <= 2048 else rows_of_sample(inp, 400)
    _compare(inp, 1 / math.sqrt(D), rows=rows, max_prefix=mp, dense=True)


@pytest.mark.parametrize("split_keys", [128, 256])
def test_dense_even_split_count(split_keys):
    """8 or 4 key splits: the grid gets one more, empty, split index (an odd width spreads
    the splits over the XCDs); its blocks issue their clamped first-tile loads and return."""
    inp = synth.attention_inputs(24, B=2, n_q=5, Hq=32, Hkv=8, D=128, prefix_len=[100, 1000], dtype="bf16",
                                 qkv_scale=1.0)
    _compare(inp, 1 / math.sqrt(128), max_prefix=1000, split_keys=split_keys, dense=True)


@pytest.mark.parametrize("split_keys", [0, 64])
def test_dense_layout_tree(split_keys):
    n = 7
    parents = np.array([-1, 0, 0, 1, 1, 2, 5], dtype=np.int32)
    bits, _, _ = oracle.tree_mask(parents, 700)
    inp = synth.attention_inputs(22, B=1, n_q=n, Hq=8, Hkv=2, D=128, prefix_len=[700], dtype="bf16", qkv_scale=1.0)
    _compare(inp, 1 / math.sqrt(128), tree_bits=bits, max_prefix=760, split_keys=split_keys, dense=True)


def rows_of_sample(inp, n):
    r = np.random.default_rng(5)
    return np.stack([r.integers(0, inp["B"], n), r.integers(0, inp["n_q"], n), r.integers(0, inp["Hq"], n)], 1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dense", [False, True])
def test_prefix_just_beyond_bound_gives_nan(dtype, dense):
    """P = max_prefix + 1 still fits the launch's one 128-key split, yet its rows are NaN
    (and with a dense cache nothing past the sequence's max_prefix + n_q slots is read)."""
    inp = synth.attention_inputs(7, B=2, n_q=4, Hq=8, Hkv=2, D=128, prefix_len=[100, 101], dtype=dtype)
    out, lse = attention_on_gpu(inp, 0.1, max_prefix=100, split_keys=128, dense=dense)
    assert np.isfinite(out[0]).all() and np.isfinite(lse[0]).all()
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()


def test_prefix_beyond_bound_gives_nan():
    inp = synth.attention_inputs(6, B=2, n_q=4, Hq=8, Hkv=2, D=128, prefix_len=[100, 900], dtype="bf16")
    out, lse = attention_on_gpu(inp, 0.1, max_prefix=100, split_keys=128)
    assert np.isfinite(out[0]).all()
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("split_keys", [0, 64])
def test_negative_prefix_gives_nan(dtype, split_keys):
    """A negative prefix length reads nothing and gives NaN rows, like one beyond max_prefix
    (with 64-key splits the call also runs the split combine); the other sequences match
    the oracle."""
    inp = synth.attention_inputs(8, B=3, n_q=4, Hq=8, Hkv=2, D=128, prefix_len=[100, 100, 37], dtype=dtype)
    ref, ref_lse, rows = oracle.attention(inp, scale=0.1)
    bad = dict(inp)
    bad["prefix_len"] = np.array([100, -3, 37], np.int32)
    out, lse = attention_on_gpu(bad, 0.1, max_prefix=100, split_keys=split_keys)
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    keep = rows[:, 0] != 1
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert np.abs(rows_of(out, rows[keep]) - ref[keep]).max() <= tol
    assert np.isfinite(out[[0, 2]]).all()


def test_batch_split_edges():
    """A batch of many 256-key splits: sequences that end exactly on a split boundary, empty
    prefixes, sequences beyond max_prefix (NaN rows), and repeated calls on one workspace."""
    n_q, Hq, Hkv, D, sk = 5, 32, 8, 128, 256
    r = np.random.default_rng(3)
    P = list(r.integers(0, 2000, 40)) + [0, 251, 507, 1019, 2000, 2001, 2600, 1, 763]
    inp = synth.attention_inputs(23, B=len(P), n_q=n_q, Hq=Hq, Hkv=Hkv, D=D, prefix_len=P, dtype="bf16",
                                 qkv_scale=1.0)
    ok = [b for b in range(len(P)) if P[b] <= 2000]
    rows = rows_of_sample(dict(inp, B=len(ok)), 500)
    rows[:, 0] = np.array(ok)[rows[:, 0]]
    rows = np.concatenate([rows, np.array([[b, n_q - 1, Hq - 1] for b in ok])])
    _compare(inp, 1 / math.sqrt(D), rows=rows, max_prefix=2000, split_keys=sk)
    first, fl = attention_on_gpu(inp, 0.09, max_prefix=2000, split_keys=sk)
    for b in range(len(P)):
        assert np.isnan(first[b]).all() == (P[b] > 2000), b
    again, al = attention_on_gpu(inp, 0.09, max_prefix=2000, split_keys=sk)
    assert np.array_equal(np.nan_to_num(again, nan=7.0), np.nan_to_num(first, nan=7.0))
    assert np.array_equal(np.nan_to_num(al, nan=7.0), np.nan_to_num(fl, nan=7.0))


@pytest.mark.parametrize("split_keys", [64, 128, 256])
def test_batch_many_splits_combine(split_keys):
    """A batch whose combine grid is large: four split lanes per row, each merging 2, 4 or 8
    splits (32, 16 and 8 splits of up to 2000 + 5 keys)."""
    n_q, Hq, Hkv, D = 5, 32, 8, 128
    P = list(np.random.default_rng(5).integers(0, 2001, 40))
    inp = synth.attention_inputs(25, B=len(P), n_q=n_q, Hq=Hq, Hkv=Hkv, D=D, prefix_len=P, dtype="bf16",
                                 qkv_scale=1.0)
    rows = rows_of_sample(inp, 600)
    _compare(inp, 1 / math.sqrt(D), rows=rows, max_prefix=2000, split_keys=split_keys)


def test_deterministic_repeats():
    inp = synth.attention_inputs(8, B=1, n_q=6, Hq=32, Hkv=8, D=128, prefix_len=[4096], dtype="bf16")
    first, fl = attention_on_gpu(inp, 0.088)
    for _ in range(5):
        o, l = attention_on_gpu(inp, 0.088)
        assert np.array_equal(o, first) and np.array_equal(l, fl)


# --------------------------------------------------------------------------------------
# Score profiles that move the online softmax's reference: each query's first dimension is 1
# and key t's first dimension is profile(t), the rest small noise, so that (scale 1) the
# scores follow the profile.  Rising scores pass the reference by more than 16 in log2
# units on every tile (a new reference each tile); a sink or falling scores leave every
# later weight far below it (underflow to 0); a slow ramp and a sawtooth mix tiles that keep
# the reference with tiles that move it.
PROFILES = {
    "rising": lambda t: 0.38 * t,  # 17.5 in log2 units per 32-key tile
    "sink": lambda t: np.where(t == 0, 40.0, 0.0),
    "falling": lambda t: -0.38 * t,
    "ramp": lambda t: 0.05 * t,
    "sawtooth": lambda t: 30.0 * ((t // 300) % 2),
    # rising for 3000 keys, then flat (long caches: scores stay near 1e3, where the fp32
    # score's own rounding stays well inside the log-sum-exp bound)
    "rising_flat": lambda t: 0.38 * np.minimum(t, 3000),
}


def _profile_inputs(seed, profile, P, n_q, Hq, Hkv, D=128):
    inp = synth.attention_inputs(seed, B=1, n_q=n_q, Hq=Hq, Hkv=Hkv, D=D, prefix_len=[P], dtype="f32",
                                 qkv_scale=0.1)
    T = P + n_q
    q = inp["q"].reshape(1, n_q, Hq, D).copy()
    k = inp["k"].reshape(T, Hkv, D).copy()
    v = synth.normal(seed, "misc", (T, Hkv, D))
    q[..., 0] = 1.0
    k[:, :, 0] = PROFILES[profile](np.arange(T, dtype=np.float64))[:, None]
    return dict(inp, q=synth.to_bf16_bits(q), k=synth.to_bf16_bits(k).reshape(-1),
                v=synth.to_bf16_bits(v).reshape(-1), dtype="bf16")


@pytest.mark.parametrize("profile", ["rising", "sink", "falling", "ramp", "sawtooth"])
@pytest.mark.parametrize("split_keys", [0, 512])
def test_softmax_reference_moves_chain(profile, split_keys):
    inp = _profile_inputs(31, profile, 3000, 5, 8, 2)
    _compare(inp, 1.0, split_keys=split_keys)


@pytest.mark.parametrize("profile", ["rising", "sink", "sawtooth"])
def test_softmax_reference_moves_tree(profile):
    n, P = 40, 1200
    bits = oracle.tree_mask(synth.random_tree(41, n, branch_p=0.6), P)[0]
    inp = _profile_inputs(32, profile, P, n, 16, 4)
    _compare(inp, 1.0, tree_bits=bits, split_keys=256)


@pytest.mark.parametrize("profile", ["rising_flat", "ramp", "sawtooth"])
def test_softmax_reference_moves_many_rows(profile):
    """A long cache and several hundred rows: the 128-row-block kernel."""
    n, P = 100, 7000
    bits = oracle.tree_mask(synth.random_tree(42, n, branch_p=0.5), P)[0]
    inp = _profile_inputs(33, profile, P, n, 32, 8)
    _compare(inp, 1.0, tree_bits=bits, rows=rows_of_sample(inp, 300))
