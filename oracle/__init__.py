"""fp64 CPU oracle of the speculative-decoding verify step (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py are the only callers.  It shares no code with the HIP library
and never imports it.  See oracle.c for the definitions and their sources.

Pins (tests/test_oracle_*.py): Philox against NumPy's independent Philox and the
published known answer; the tree mask against the worked example of the
textbook page ("Token tree and tree attention" box) and the Cartesian counts of
the Medusa page; attention against torch's float64 scaled_dot_product_attention
on CPU and against per-path brute force; acceptance against the three-token
worked example, alpha = 1 - TV, the special cases, chi-square of the output law
and E[J] = sum_i prod_{j<=i} alpha_j; the tree walk against brute force and the
closed-form node-acceptance probabilities; the near-threshold flags against an
independent NumPy recomputation on crafted inputs; the KV commit against a
simulated chain pass and attention through torch's SDPA; block verification
against the printed 11/9 and the two-token law; Gumbel coupling against NumPy's
Philox, the Gumbel-max law and the printed match-probability formula; recursive
rejection against the output law p and the printed acceptance formula.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

TAG_ACCEPT = 0x53560001
TAG_WALK = 0x53560002
TAG_GUMBEL = 0x53560003
TAG_RRS = 0x53560004
GREEDY, SAMPLE = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = _typed(ctypes.CDLL(_SO))
    return _lib


def _typed(L):
    P = ctypes.c_void_p
    i32, i64, u64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float, ctypes.c_double
    L.orc_philox4x64_10.argtypes = [P, P, P]
    L.orc_philox4x64_10.restype = None
    L.orc_uniform.argtypes = [u64, u64, u64, u64, u64]
    L.orc_uniform.restype = f64
    L.orc_tree_mask.argtypes = [P, i32, i32, P, i32, P, P]
    L.orc_tree_mask.restype = i32
    L.orc_attention.argtypes = [i32, i32, i32, i32, i32, i32, f64, i32, P, i64, i64, i64, P, P, P,
                                i64, i64, P, P, i64, i32, P, i64, P, P]
    L.orc_attention.restype = i32
    L.orc_spec_accept.argtypes = [i32, i32, i32, i32, f32, P, P, P, u64, u64, P, P, P, P, P]
    L.orc_spec_accept.restype = i32
    L.orc_tree_walk.argtypes = [i32, i32, i32, i32, i32, f32, P, P, P, u64, u64, P, P, P, P, P]
    L.orc_tree_walk.restype = i32
    L.orc_kv_commit.argtypes = [i32, i32, i32, i32, i32, P, P, P, i64, i64, P, P, P, i32, P]
    L.orc_kv_commit.restype = i32
    L.orc_block_accept.argtypes = [i32, i32, i32, f32, P, P, P, u64, u64, P, P, P, P, P]
    L.orc_block_accept.restype = i32
    L.orc_gumbel_argmax.argtypes = [i32, i32, i32, f32, P, u64, u64, P, P, P]
    L.orc_gumbel_argmax.restype = i32
    L.orc_gumbel_accept.argtypes = [i32, i32, i32, f32, P, P, u64, u64, P, P, P, P]
    L.orc_gumbel_accept.restype = i32
    L.orc_tree_rrs.argtypes = [i32, i32, i32, i32, f32, i32, P, P, P, P, u64, u64, P, P, P, P, P]
    L.orc_tree_rrs.restype = i32
    L.orc_truncate.argtypes = [i32, i32, f32, i32, f32, P, P, P, P, P, P]
    L.orc_truncate.restype = i32
    L.orc_penalize.argtypes = [i32, i32, i32, P, P, P, P, i32, P, i32, f32, f32, f32]
    L.orc_penalize.restype = i32
    return L


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def set_threads(n: int) -> None:
    """Threads for the OpenMP loops over independent outputs (OMP_NUM_THREADS)."""
    try:
        import ctypes.util
        gomp = ctypes.CDLL(ctypes.util.find_library("gomp") or "libgomp.so.1")
        gomp.omp_set_num_threads(int(n))
    except OSError:
        os.environ["OMP_NUM_THREADS"] = str(int(n))


# --------------------------------------------------------------------------- #
def philox4x64_10(counter, key) -> np.ndarray:
    c = _c(counter, np.uint64)
    k = _c(key, np.uint64)
    out = np.zeros(4, dtype=np.uint64)
    lib().orc_philox4x64_10(_p(c), _p(k), _p(out))
    return out


def uniform(seed: int, c0: int, step: int, stream: int, tag: int) -> float:
    return lib().orc_uniform(seed, c0, step, stream, tag)


def tree_mask(parents, prefix_len: int):
    """-> (bits uint32 [n][ceil(n/32)], depth int32 [n], pos int64 [n]); raises on a bad parent."""
    par = _c(parents, np.int32)
    n = len(par)
    words = (n + 31) // 32
    bits = np.zeros((n, words), dtype=np.uint32)
    depth = np.zeros(n, dtype=np.int32)
    pos = np.zeros(n, dtype=np.int64)
    st = lib().orc_tree_mask(_p(par), n, int(prefix_len), _p(bits), words, _p(depth), _p(pos))
    if st != 0:
        raise ValueError("bad parent at node %d" % (st - 1))
    return bits, depth, pos


def dense_mask(bits: np.ndarray, n: int, prefix_len: int) -> np.ndarray:
    """Expand bit rows to the boolean (n, P + n) mask (prefix block all ones)."""
    j = np.arange(n)
    node = ((bits[:, j >> 5] >> (j & 31).astype(np.uint32)) & 1).astype(bool)
    return np.concatenate([np.ones((n, prefix_len), dtype=bool), node], axis=1)


def attention(inp: dict, *, scale: float, tree_bits=None, tree_sb: int = 0, rows=None):
    """fp64 attention for the listed (b, i, h) rows (all rows when None).

    ``inp`` is a synth.attention_inputs dict (float32 or bf16-bit arrays).
    Returns (out [n_rows][D] float64, lse [n_rows] float64, rows int32 [n_rows][3]).
    """
    B, n_q, Hq, Hkv, D = inp["B"], inp["n_q"], inp["Hq"], inp["Hkv"], inp["D"]
    dt = 0 if inp["dtype"] == "f32" else 1
    edt = np.float32 if dt == 0 else np.uint16
    q, k, v = _c(inp["q"], edt), _c(inp["k"], edt), _c(inp["v"], edt)
    if rows is None:
        bb, ii, hh = np.meshgrid(np.arange(B), np.arange(n_q), np.arange(Hq), indexing="ij")
        rows = np.stack([bb.ravel(), ii.ravel(), hh.ravel()], axis=1)
    rows = _c(rows, np.int32).reshape(-1, 3)
    nr = rows.shape[0]
    out = np.zeros((nr, D), dtype=np.float64)
    lse = np.zeros(nr, dtype=np.float64)
    kv_off = _c(inp["kv_off"], np.int64)
    pl = _c(inp["prefix_len"], np.int32)
    tb = None if tree_bits is None else _c(tree_bits, np.uint32)
    words = 0 if tb is None else tb.shape[-1]
    st = lib().orc_attention(dt, B, n_q, Hq, Hkv, D, float(scale), 0 if tb is None else 1,
                             _p(q), inp["q_sb"], inp["q_st"], inp["q_sh"], _p(k), _p(v), _p(kv_off),
                             inp["kv_sh"], inp["kv_st"], _p(pl), _p(tb), int(tree_sb), words,
                             _p(rows), nr, _p(out), _p(lse))
    if st != 0:
        raise ValueError("orc_attention status %d" % st)
    return out, lse, rows


def compile_variant(replacements: dict, tag: str):
    """Build a copy of oracle.c with literal source replacements into a temporary
    library (used by tests that plant a known mistake in the oracle, on the CPU).
    Every replacement must match exactly once.  Returns a loaded ctypes handle."""
    import tempfile
    src = open(_SRC).read()
    for old, new in replacements.items():
        if src.count(old) != 1:
            raise ValueError("replacement must match exactly once: %r" % old)
        src = src.replace(old, new)
    d = tempfile.mkdtemp(prefix="oracle_%s_" % tag)
    c, so = os.path.join(d, "variant.c"), os.path.join(d, "libvariant.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-o", so, c, "-lm"])
    return _typed(ctypes.CDLL(so))


def spec_accept(mode: int, target, draft, draft_tokens, temperature: float, seed: int, step: int = 0,
                stream_ids=None, want_alpha: bool = False, handle=None):
    """-> dict(accept_len [B], out_tokens [B][gamma+1], alpha [B][gamma] or None, flags [B])."""
    tgt = _c(target, np.float32)
    B, g1, V = tgt.shape
    gamma = g1 - 1
    dr = None if draft is None else _c(draft, np.float32)
    if dr is None and not (mode == GREEDY or temperature == 0.0):
        raise ValueError("sampling needs draft logits")
    toks = _c(draft_tokens, np.int32).reshape(B, gamma)
    sid = None if stream_ids is None else _c(stream_ids, np.uint64)
    acc = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, gamma + 1), dtype=np.int32)
    alpha = np.zeros((B, gamma), dtype=np.float64) if want_alpha else None
    flags = np.zeros(B, dtype=np.int32)
    st = (handle or lib()).orc_spec_accept(int(mode), B, gamma, V, float(temperature), _p(tgt), _p(dr), _p(toks),
                               int(seed), int(step), _p(sid), _p(acc), _p(out), _p(alpha), _p(flags))
    if st != 0:
        raise ValueError("orc_spec_accept status %d" % st)
    return dict(accept_len=acc, out_tokens=out, alpha=alpha, flags=flags)


def tree_walk(mode: int, logits, tokens, parents, temperature: float, seed: int, step: int = 0,
              stream_ids=None, max_depth=None, handle=None, allow_too_deep: bool = False):
    """-> dict(accept_len [B], path [B][max_depth+1], out_tokens [B][max_depth+1], flags [B])."""
    lg = _c(logits, np.float32)
    B, n, V = lg.shape
    tk = _c(tokens, np.int32).reshape(B, n)
    par = _c(parents, np.int32)
    if max_depth is None:
        _, depth, _ = tree_mask(par, 0)
        max_depth = int(depth.max())
    sid = None if stream_ids is None else _c(stream_ids, np.uint64)
    acc = np.zeros(B, dtype=np.int32)
    path = np.zeros((B, max_depth + 1), dtype=np.int32)
    out = np.zeros((B, max_depth + 1), dtype=np.int32)
    flags = np.zeros(B, dtype=np.int32)
    st = (handle or lib()).orc_tree_walk(int(mode), B, n, V, int(max_depth), float(temperature), _p(lg), _p(tk),
                                         _p(par), int(seed), int(step), _p(sid), _p(acc), _p(path), _p(out),
                                         _p(flags))
    if st != 0 and not (st == 3 and allow_too_deep):
        raise ValueError("orc_tree_walk status %d" % st)
    return dict(accept_len=acc, path=path, out_tokens=out, flags=flags, status=st)


# --------------------------------------------------------------------------- #
def kv_commit(k, v, kv_off, prefix_len, accept_len, *, n_q: int, Hkv: int, D: int, kv_sh: int, kv_st: int,
              path=None):
    """Commit in place on copies of the flat caches k, v (numpy; float32 or bf16 bit patterns).
    Returns (k, v, new_len, status) -- status 0, or 1 + the first bad sequence."""
    k = np.array(k, copy=True, order="C")
    v = np.array(v, copy=True, order="C")
    B = len(prefix_len)
    pl = _c(prefix_len, np.int32)
    acc = _c(accept_len, np.int32)
    pth = None if path is None else _c(path, np.int32).reshape(B, -1)
    new_len = np.zeros(B, dtype=np.int32)
    st = lib().orc_kv_commit(B, int(n_q), int(Hkv), int(D), k.itemsize, _p(k), _p(v), _p(_c(kv_off, np.int64)),
                             int(kv_sh), int(kv_st), _p(pl), _p(acc), _p(pth), 0 if pth is None else pth.shape[1],
                             _p(new_len))
    return k, v, new_len, st


def block_accept(target, draft, draft_tokens, temperature: float, seed: int, step: int = 0, stream_ids=None,
                 handle=None):
    """Block verification -> dict(accept_len, out_tokens, weights [B][gamma+1], flags)."""
    tgt = _c(target, np.float32)
    B, g1, V = tgt.shape
    gamma = g1 - 1
    dr = _c(draft, np.float32)
    toks = _c(draft_tokens, np.int32).reshape(B, gamma)
    sid = None if stream_ids is None else _c(stream_ids, np.uint64)
    acc = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, g1), dtype=np.int32)
    w = np.zeros((B, g1), dtype=np.float64)
    flags = np.zeros(B, dtype=np.int32)
    st = (handle or lib()).orc_block_accept(B, gamma, V, float(temperature), _p(tgt), _p(dr), _p(toks), int(seed),
                                            int(step), _p(sid), _p(acc), _p(out), _p(w), _p(flags))
    if st != 0:
        raise ValueError("orc_block_accept status %d" % st)
    return dict(accept_len=acc, out_tokens=out, weights=w, flags=flags)


def gumbel_argmax(logits, temperature: float, seed: int, step: int = 0, stream_ids=None):
    """argmax(logits/T + shared Gumbel noise) of every row [B][rows][V] (row i = position i)
    -> (tokens [B][rows], gap [B][rows])."""
    lg = _c(logits, np.float32)
    B, rows, V = lg.shape
    sid = None if stream_ids is None else _c(stream_ids, np.uint64)
    out = np.zeros((B, rows), dtype=np.int32)
    gap = np.zeros((B, rows), dtype=np.float64)
    st = lib().orc_gumbel_argmax(B, rows, V, float(temperature), _p(lg), int(seed), int(step), _p(sid), _p(out),
                                 _p(gap))
    if st != 0:
        raise ValueError("orc_gumbel_argmax status %d" % st)
    return out, gap


def gumbel_accept(target, draft_tokens, temperature: float, seed: int, step: int = 0, stream_ids=None):
    """Gumbel-coupled verification -> dict(accept_len, out_tokens, flags)."""
    tgt = _c(target, np.float32)
    B, g1, V = tgt.shape
    toks = _c(draft_tokens, np.int32).reshape(B, g1 - 1)
    sid = None if stream_ids is None else _c(stream_ids, np.uint64)
    acc = np.zeros(B, dtype=np.int32)
    out = np.zeros((B, g1), dtype=np.int32)
    flags = np.zeros(B, dtype=np.int32)
    st = lib().orc_gumbel_accept(B, g1 - 1, V, float(temperature), _p(tgt), _p(toks), int(seed), int(step), _p(sid),
                                 _p(acc), _p(out), _p(flags))
    if st != 0:
        raise ValueError("orc_gumbel_accept status %d" % st)
    return dict(accept_len=acc, out_tokens=out, flags=flags)


def truncate(logits, temperature: float, top_k: int = 0, top_p: float = 1.0, top_k_rows=None, top_p_rows=None,
             handle=None):
    """Top-k, then top-p truncation of every row of logits [..., V] (oracle.c orc_truncate)
    -> dict(out (same shape, -inf off the kept set), kept [rows], flags [rows])."""
    lg = _c(logits, np.float32)
    shape = lg.shape
    V = shape[-1]
    rows = lg.reshape(-1, V)
    R = rows.shape[0]
    out = np.empty_like(rows)
    kept = np.zeros(R, dtype=np.int32)
    flags = np.zeros(R, dtype=np.int32)
    kr = None if top_k_rows is None else _c(top_k_rows, np.int32).reshape(R)
    pr = None if top_p_rows is None else _c(top_p_rows, np.float32).reshape(R)
    st = (handle or lib()).orc_truncate(R, V, float(temperature), int(top_k), float(top_p), _p(kr), _p(pr),
                                        _p(rows), _p(out), _p(kept), _p(flags))
    if st != 0:
        raise ValueError("orc_truncate status %d" % st)
    return dict(out=out.reshape(shape), kept=kept, flags=flags)


def penalize(logits, history=None, hist_len=None, drafts=None, repetition: float = 1.0, frequency: float = 0.0,
             presence: float = 0.0, handle=None):
    """Repetition / frequency / presence penalties on logits [B][n_rows][V], row i's context
    being the history then drafts[:, :i] (oracle.c orc_penalize) -> penalized copy."""
    lg = _c(logits, np.float32)
    B, n_rows, V = lg.shape
    out = np.empty_like(lg)
    hs = None if history is None else _c(history, np.int32).reshape(B, -1)
    hl = None if hist_len is None else _c(hist_len, np.int32).reshape(B)
    if hs is not None and hl is None:
        hl = np.full(B, hs.shape[1], np.int32)
    dr = None if drafts is None else _c(drafts, np.int32).reshape(B, -1)
    st = (handle or lib()).orc_penalize(B, n_rows, V, _p(lg), _p(out), _p(hs), _p(hl),
                                        0 if hs is None else hs.shape[1], _p(dr), 0 if dr is None else dr.shape[1],
                                        float(repetition), float(frequency), float(presence))
    if st != 0:
        raise ValueError("orc_penalize status %d" % st)
    return out


RULE_TOKEN, RULE_BLOCK, RULE_GUMBEL = 0, 1, 2


def accept_ragged(rule: int, mode: int, target, draft, draft_tokens, draft_len, temperature: float, seed: int,
                  step: int = 0, stream_ids=None, want_alpha: bool = False):
    """One round where sequence b verifies only its first L_b = draft_len[b] drafts.

    "Speculative decoding" (Zero to Frontier), section "Choosing how much to verify at every
    step": a step that verifies l_r drafts of request r runs the target over 1 + l_r tokens of
    it, so the round of sequence b is the ordinary round with gamma = L_b on its first L_b + 1
    target rows, L_b draft rows and tokens, with its own stream of uniforms.  This calls the
    fixed-gamma functions above once per distinct length (rule 0: spec_accept, 1: block_accept,
    2: gumbel_accept) and lays the results out at the full gamma: out_tokens [B][gamma+1]
    padded with -1, alpha [B][gamma] NaN past L_b.  L_b = 0 is one draw from target row 0.
    """
    tgt = _c(target, np.float32)
    B, g1, V = tgt.shape
    gamma = g1 - 1
    dr = None if draft is None else _c(draft, np.float32)
    toks = _c(draft_tokens, np.int32).reshape(B, gamma)
    L = np.asarray(draft_len, dtype=np.int64).reshape(B)
    if (L < 0).any() or (L > gamma).any():
        raise ValueError("draft lengths must lie in [0, gamma]")
    sid = np.arange(B, dtype=np.uint64) if stream_ids is None else _c(stream_ids, np.uint64).reshape(B)
    acc = np.zeros(B, dtype=np.int32)
    out = np.full((B, g1), -1, dtype=np.int32)
    alpha = np.full((B, gamma), np.nan) if want_alpha else None
    flags = np.zeros(B, dtype=np.int32)
    for lb in np.unique(L):
        lb = int(lb)
        idx = np.nonzero(L == lb)[0]
        t = np.ascontiguousarray(tgt[idx, :lb + 1])
        x = np.ascontiguousarray(toks[idx, :lb])
        d = None if dr is None else np.ascontiguousarray(dr[idx, :lb])
        s = np.ascontiguousarray(sid[idx])
        sampled = not (mode == GREEDY or temperature == 0.0)  # else every rule is the greedy one
        if sampled and rule == RULE_GUMBEL:
            r = gumbel_accept(t, x, temperature, seed, step, stream_ids=s)
        elif sampled and rule == RULE_BLOCK:
            r = block_accept(t, d, x, temperature, seed, step, stream_ids=s)
        else:
            r = spec_accept(mode, t, d, x, temperature, seed, step, stream_ids=s, want_alpha=want_alpha)
            if want_alpha and lb > 0:
                alpha[idx, :lb] = r["alpha"]
        acc[idx] = r["accept_len"]
        out[idx, :lb + 1] = r["out_tokens"]
        flags[idx] = r["flags"]
    return dict(accept_len=acc, out_tokens=out, alpha=alpha, flags=flags)


def tree_rrs(target, draft, tokens, parents, temperature: float, seed: int, step: int = 0, stream_ids=None,
             max_depth=None, without_replacement: bool = False, handle=None, allow_too_deep: bool = False):
    """Recursive rejection over a token tree -> dict(accept_len, path, out_tokens, flags, status)."""
    tgt = _c(target, np.float32)
    B, n, V = tgt.shape
    dr = _c(draft, np.float32)
    tk = _c(tokens, np.int32).reshape(B, n)
    par = _c(parents, np.int32)
    if max_depth is None:
        _, depth, _ = tree_mask(par, 0)
        max_depth = int(depth.max())
    sid = None if stream_ids is None else _c(stream_ids, np.uint64)
    acc = np.zeros(B, dtype=np.int32)
    path = np.zeros((B, max_depth + 1), dtype=np.int32)
    out = np.zeros((B, max_depth + 1), dtype=np.int32)
    flags = np.zeros(B, dtype=np.int32)
    st = (handle or lib()).orc_tree_rrs(B, n, V, int(max_depth), float(temperature), int(bool(without_replacement)),
                                        _p(tgt), _p(dr), _p(tk), _p(par), int(seed), int(step), _p(sid), _p(acc),
                                        _p(path), _p(out), _p(flags))
    if st != 0 and not (st == 3 and allow_too_deep):
        raise ValueError("orc_tree_rrs status %d" % st)
    return dict(accept_len=acc, path=path, out_tokens=out, flags=flags, status=st)
