"""Seeded synthetic inputs for the speculative-decoding verify step.

Both the HIP library's tests/bench and the CPU oracle draw their inputs from
here.  This module holds none of the verify method's arithmetic: no softmax,
no acceptance test, no residual, no attention.  It only draws random arrays,
lays them out, and builds token-tree topologies (the drafter's side of the
method, which the verifier receives as input).

Every array comes from its own named NumPy stream, ``default_rng([seed, id])``,
so that drawing one array never shifts another and any subset can be generated
alone.  Normal laws are written N(mean, variance), as the pages write them.

Layouts (shared conventions of the verify boundary):
  Q     [B][n_q][Hq][D]                       row-major
  K, V  one flat buffer; sequence b starts at element kv_off[b] and holds
        [P_b + n_q][Hkv][D] (token-major cache, heads interleaved)
  target logits [B][gamma+1][V] fp32, draft logits [B][gamma][V] fp32
  tree logits   [B][n][V] fp32 (row v = the target after node v)
"""
from __future__ import annotations

import itertools
import math

import numpy as np

# stable stream ids for the named arrays
_STREAM = {
    "prefix": 1, "q": 2, "k": 3, "v": 4, "target": 5, "draft_noise": 6,
    "draft_gumbel": 7, "node_noise": 8, "tree_logits": 9, "root_token": 10,
    "misc": 11, "logit_rows": 12,
}


def rng(seed: int, name: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), _STREAM[name]])


def normal(seed: int, name: str, shape, variance: float = 1.0, scale: float = 1.0) -> np.ndarray:
    """float32 draws of N(0, variance), times ``scale``."""
    a = rng(seed, name).standard_normal(size=shape, dtype=np.float32)
    f = np.float32(math.sqrt(variance) * scale)
    if f != 1.0:
        a *= f
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (round to nearest even) and return the raw 16-bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- #
# the five workloads                                                            #
# --------------------------------------------------------------------------- #
WORKLOADS = {
    1: dict(name="tiny-chain-fp32", kind="chain", B=1, gamma=4, P=128, Hq=2, Hkv=2, D=64,
            dtype="f32", qkv_scale=1.0, V=1000, target_var=2.0, noise_var=1.0, tau=1.0),
    2: dict(name="8b-chain-bf16", kind="chain", B=1, gamma=5, P=4096, Hq=32, Hkv=8, D=128,
            dtype="bf16", qkv_scale=1.0 / math.sqrt(128.0), V=128256, target_var=3.0,
            noise_var=1.5, tau=0.8),
    3: dict(name="medusa64-tree-bf16", kind="tree", B=1, tree="medusa", n_nodes=64, K=4, top=10,
            P=2048, Hq=32, Hkv=8, D=128, dtype="bf16", qkv_scale=1.0 / math.sqrt(128.0),
            V=128256, target_var=3.0, tau=0.7),
    4: dict(name="batched-chain-bf16", kind="chain", B=64, gamma=4, P_lo=512, P_hi=8192,
            Hq=32, Hkv=8, D=128, dtype="bf16", qkv_scale=1.0 / math.sqrt(128.0), V=128256,
            target_var=3.0, noise_var=1.0, tau=1.0),
    5: dict(name="cartesian4x8-tree-bf16", kind="tree", B=1, tree="cartesian", K=4, top=8,
            P=16384, Hq=64, Hkv=8, D=128, dtype="bf16", qkv_scale=1.0 / math.sqrt(128.0),
            V=128256, target_var=3.0, tau=0.7),
}


def prefix_lengths(seed: int, cfg: dict) -> np.ndarray:
    B = cfg["B"]
    if "P_lo" in cfg:
        return rng(seed, "prefix").integers(cfg["P_lo"], cfg["P_hi"], size=B, endpoint=True).astype(np.int32)
    return np.full(B, cfg["P"], dtype=np.int32)


# --------------------------------------------------------------------------- #
# attention inputs                                                              #
# --------------------------------------------------------------------------- #
def attention_inputs(seed: int, *, B: int, n_q: int, Hq: int, Hkv: int, D: int,
                     prefix_len, dtype: str = "bf16", qkv_scale: float = 1.0,
                     q_scale: float = 1.0) -> dict:
    """Q, K, V ~ N(0,1) * qkv_scale (Q also times q_scale), token-major caches.

    Returns numpy arrays: float32 for dtype 'f32', raw bf16 bit patterns
    (uint16) for 'bf16'.  The cache of sequence b holds P_b + n_q tokens: the
    P_b cached ones and the n_q new ones (the verify pass has written their
    keys and values before attention runs).
    """
    P = np.asarray(prefix_len, dtype=np.int32).reshape(B)
    toks = (P.astype(np.int64) + n_q)
    kv_off = np.zeros(B, dtype=np.int64)
    kv_off[1:] = np.cumsum(toks[:-1] * Hkv * D)
    total = int(toks.sum()) * Hkv * D
    q = normal(seed, "q", (B, n_q, Hq, D), scale=qkv_scale * q_scale)
    k = normal(seed, "k", (total,), scale=qkv_scale)
    v = normal(seed, "v", (total,), scale=qkv_scale)
    if dtype == "bf16":
        q, k, v = to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return dict(q=q, k=k, v=v, kv_off=kv_off, prefix_len=P, B=B, n_q=n_q, Hq=Hq, Hkv=Hkv, D=D,
                dtype=dtype, kv_st=Hkv * D, kv_sh=D, q_sb=n_q * Hq * D, q_st=Hq * D, q_sh=D)


# --------------------------------------------------------------------------- #
# acceptance inputs                                                             #
# --------------------------------------------------------------------------- #
def gumbel_draw(logits: np.ndarray, tau: float, g_uniform: np.ndarray) -> np.ndarray:
    """The drafter's own sampler: x = argmax(logits/tau + Gumbel noise), i.e. a draw
    from softmax(logits/tau) by the Gumbel-max trick; tau == 0 is the argmax."""
    if tau == 0.0:
        return np.argmax(logits, axis=-1)
    g = -np.log(-np.log(g_uniform))
    return np.argmax(logits.astype(np.float64) / tau + g, axis=-1)


def accept_inputs(seed: int, *, B: int, gamma: int, V: int, target_var: float, noise_var: float,
                  tau: float, greedy_drafts: bool = False) -> dict:
    """target ~ N(0, target_var); draft = target[:gamma] + N(0, noise_var);
    drafts x_i sampled from the draft at temperature tau (argmax when greedy)."""
    target = normal(seed, "target", (B, gamma + 1, V), variance=target_var)
    noise = normal(seed, "draft_noise", (B, gamma, V), variance=noise_var)
    draft = target[:, :gamma, :] + noise
    if greedy_drafts or tau == 0.0:
        toks = np.argmax(draft, axis=-1)
    else:
        u = rng(seed, "draft_gumbel").random(size=(B, gamma, V))
        u = np.clip(u, 1e-300, 1.0 - 1e-16)
        toks = gumbel_draw(draft, tau, u)
    return dict(target=np.ascontiguousarray(target), draft=np.ascontiguousarray(draft),
                draft_tokens=np.ascontiguousarray(toks.astype(np.int32)))


# --------------------------------------------------------------------------- #
# token trees (the drafter's side: topologies the verifier receives)            #
# --------------------------------------------------------------------------- #
def _bfs_order(paths):
    return sorted(paths, key=lambda p: (len(p), p))


def tree_from_rank_paths(paths) -> tuple[np.ndarray, list]:
    """Root (empty path) at node 0, then the given rank paths in BFS order
    (depth, then lexicographic).  Returns parents (root = -1) and the ordered paths."""
    ordered = [()] + _bfs_order([tuple(p) for p in paths if len(p) > 0])
    index = {p: i for i, p in enumerate(ordered)}
    parents = np.empty(len(ordered), dtype=np.int32)
    parents[0] = -1
    for i, p in enumerate(ordered[1:], start=1):
        parents[i] = index[p[:-1]]
    return parents, ordered


def cartesian_paths(K: int, s: int) -> list:
    """Fixed product tree: every rank path of length 1..K with ranks 1..s
    ("Speculative-Decoding" (Medusa notes), section "Attention Tree")."""
    out = []
    for m in range(1, K + 1):
        out.extend(itertools.product(range(1, s + 1), repeat=m))
    return out


def medusa_accuracy(k: int, i: int) -> float:
    """Synthetic head accuracy of head k, rank i: 0.7^k * 0.6^(i-1)."""
    return 0.7 ** k * 0.6 ** (i - 1)


def medusa_greedy_paths(n_nodes: int, K: int, top: int) -> list:
    """Greedy sparse tree ("Speculative-Decoding", section on optimized tree
    construction): starting from the root, repeatedly add the node whose path
    score prod_j a_j^(i_j) -- its contribution to the expected accepted length --
    is largest among the children of nodes already in the tree, until n_nodes
    drafted nodes.  Ties (equal scores) go to the lexicographically smaller
    rank path.  Scores are 0.7^A * 0.6^B with integer A, B, so equal scores
    are exactly equal (A, B) and the fp64 log comparison is exact in order."""
    def key(p):
        m = len(p)
        return (-(m * (m + 1) // 2) * math.log(0.7) - sum(i - 1 for i in p) * math.log(0.6), p)

    chosen = []
    frontier = {(i,) for i in range(1, top + 1)}
    while len(chosen) < n_nodes and frontier:
        best = min(frontier, key=key)
        frontier.remove(best)
        chosen.append(best)
        if len(best) < K:
            frontier.update(best + (i,) for i in range(1, top + 1))
    return chosen


def build_tree(cfg: dict) -> tuple[np.ndarray, list]:
    if cfg["tree"] == "cartesian":
        return tree_from_rank_paths(cartesian_paths(cfg["K"], cfg["top"]))
    if cfg["tree"] == "medusa":
        return tree_from_rank_paths(medusa_greedy_paths(cfg["n_nodes"], cfg["K"], cfg["top"]))
    raise ValueError(cfg["tree"])


def random_tree(seed: int, n: int, branch_p: float = 0.5) -> np.ndarray:
    """A random forest-free tree with root 0: node i > 0 picks a parent among
    0..i-1 (recent nodes more likely when branch_p is small)."""
    r = rng(seed, "misc")
    parents = np.empty(n, dtype=np.int32)
    parents[0] = -1
    for i in range(1, n):
        if r.random() < branch_p:
            parents[i] = r.integers(0, i)
        else:
            parents[i] = i - 1
    return parents


def tree_logits(seed: int, B: int, n: int, V: int, variance: float) -> np.ndarray:
    return normal(seed, "tree_logits", (B, n, V), variance=variance)


def sibling_ranks(parents: np.ndarray) -> np.ndarray:
    """rank(i) = 1 + number of earlier nodes with the same parent (0 for the root)."""
    n = len(parents)
    ranks = np.zeros(n, dtype=np.int32)
    seen = {}
    for i in range(1, n):
        p = int(parents[i])
        seen[p] = seen.get(p, 0) + 1
        ranks[i] = seen[p]
    return ranks


def node_tokens(seed: int, logits: np.ndarray, parents: np.ndarray, ranks=None) -> np.ndarray:
    """Draft tokens of the tree nodes: the children of node v at ranks 1..s get the
    rank-ordered top tokens of logits[v] + N(0,1) noise, a stand-in for a drafter
    that is correlated with the target.  The root gets a random token.
    ``ranks`` defaults to the sibling order (for trees built from rank paths in
    BFS order the sibling order is the rank order when every rank is present)."""
    B, n, V = logits.shape
    parents = np.asarray(parents)
    if ranks is None:
        ranks = sibling_ranks(parents)
    ranks = np.asarray(ranks)
    toks = np.empty((B, n), dtype=np.int32)
    maxrank = int(ranks.max()) if n > 1 else 1
    has_child = np.zeros(n, dtype=bool)
    has_child[parents[parents >= 0]] = True
    parent_rows = np.nonzero(has_child)[0]
    r = rng(seed, "node_noise")
    toks[:, 0] = rng(seed, "root_token").integers(0, V, size=B)
    for b in range(B):
        top = {}
        for v in parent_rows:
            noisy = logits[b, v].astype(np.float32) + r.standard_normal(V, dtype=np.float32)
            kk = min(maxrank, V)
            part = np.argpartition(-noisy, kk - 1)[:kk]
            top[v] = part[np.argsort(-noisy[part], kind="stable")]
        for i in range(1, n):
            rk = min(int(ranks[i]), V)
            toks[b, i] = top[int(parents[i])][rk - 1]
    return toks


def path_ranks(paths: list) -> np.ndarray:
    """Last rank of each node's rank path (0 for the root)."""
    return np.array([p[-1] if p else 0 for p in paths], dtype=np.int32)


def logit_rows(seed: int, R: int, V: int, variance: float, grid: float = 0.0) -> np.ndarray:
    """fp32 logit rows [R][V] ~ N(0, variance); with grid > 0 every logit is rounded to a
    multiple of grid, so that rows hold many exactly equal logits (ties)."""
    a = normal(seed, "logit_rows", (R, V), variance)
    if grid > 0:
        a = (np.round(a / np.float32(grid)) * np.float32(grid)).astype(np.float32)
    return a
