"""Python binding of libspecverify (the verify step of speculative decoding, HIP on gfx950).

Argument marshalling only: every step of the path runs in the library's kernels.
PyTorch supplies device memory and the current HIP stream.  The names mirror the
C entry points declared in include/specverify.h.

The library must be built in-tree (``python draft_token_verification_attention_amd/_build.py``);
importing this package without it raises ImportError -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_ERR_INVALID_ARG, SV_ERR_UNSUPPORTED, SV_ERR_WORKSPACE, SV_ERR_HIP = range(5)
SV_STATIC_SCRATCH_BYTES = 16 << 20
SV_F32, SV_BF16 = 0, 1
SV_GREEDY, SV_SAMPLE = 0, 1
SV_RULE_TOKEN, SV_RULE_BLOCK, SV_RULE_GUMBEL = 0, 1, 2
SV_WALK_MATCH, SV_WALK_RRS, SV_WALK_RRS_WOR = 0, 1, 2
SV_MASK_CAUSAL, SV_MASK_TREE = 0, 1

_P = ctypes.c_void_p
_i32, _i64, _u64, _f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float


class sv_philox(ctypes.Structure):
    _fields_ = [("seed", _u64), ("step", _u64), ("stream_ids", _P)]


class sv_attn_desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("mask", ctypes.c_int),
                ("B", _i32), ("n_q", _i32), ("Hq", _i32), ("Hkv", _i32), ("D", _i32),
                ("max_prefix", _i32), ("split_keys", _i32), ("scale", _f32),
                ("q", _P), ("q_sb", _i64), ("q_st", _i64), ("q_sh", _i64),
                ("k", _P), ("v", _P), ("kv_off", _P), ("kv_sh", _i64), ("kv_st", _i64),
                ("kv_sb", _i64), ("prefix_len", _P), ("tree_bits", _P), ("tree_sb", _i64),
                ("out", _P), ("o_sb", _i64), ("o_st", _i64), ("o_sh", _i64), ("lse", _P),
                ("ev_kernel_start", _P), ("ev_kernel_stop", _P), ("ev_call_stop", _P)]


class sv_accept_desc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("B", _i32), ("gamma", _i32), ("V", _i32), ("temperature", _f32),
                ("target_logits", _P), ("draft_logits", _P), ("draft_tokens", _P), ("rng", sv_philox),
                ("accept_len", _P), ("out_tokens", _P), ("alpha", _P), ("dev_status", _P),
                ("rule", ctypes.c_int), ("draft_len", _P)]


class sv_walk_desc(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("B", _i32), ("n", _i32), ("V", _i32), ("max_depth", _i32),
                ("temperature", _f32), ("logits", _P), ("tokens", _P), ("parents", _P), ("rng", sv_philox),
                ("accept_len", _P), ("path", _P), ("out_tokens", _P), ("dev_status", _P),
                ("rule", ctypes.c_int), ("draft_logits", _P), ("max_children", _i32)]


class sv_commit_desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("B", _i32), ("n_q", _i32), ("Hkv", _i32), ("D", _i32),
                ("k", _P), ("v", _P), ("kv_off", _P), ("kv_sb", _i64), ("kv_sh", _i64), ("kv_st", _i64),
                ("prefix_len", _P), ("accept_len", _P), ("path", _P), ("path_stride", _i32),
                ("new_len", _P), ("dev_status", _P)]


class sv_trunc_desc(ctypes.Structure):
    _fields_ = [("R", _i32), ("V", _i32), ("temperature", _f32), ("top_k", _i32), ("top_p", _f32),
                ("top_k_rows", _P), ("top_p_rows", _P), ("logits", _P), ("out", _P), ("kept", _P)]


class sv_penalty_desc(ctypes.Structure):
    _fields_ = [("B", _i32), ("n_rows", _i32), ("V", _i32), ("logits", _P), ("history", _P), ("hist_len", _P),
                ("hist_stride", _i32), ("draft_tokens", _P), ("n_drafts", _i32), ("repetition", _f32),
                ("frequency", _f32), ("presence", _f32)]


EXPORTS = ("sv_build_tree_mask", "sv_verify_attention_workspace", "sv_verify_attention",
           "sv_spec_accept_workspace", "sv_spec_accept", "sv_spec_accept_static", "sv_tree_walk_workspace",
           "sv_tree_walk", "sv_kv_commit", "sv_truncate_workspace", "sv_truncate", "sv_penalize_workspace", "sv_penalize",
           "sv_status_string")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libspecverify.so is not built: run "
                          "`python draft_token_verification_attention_amd/_build.py` (%s)" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    L.sv_build_tree_mask.argtypes = [_P, _i32, _i32, _P, _P, _P, _P, _P]
    L.sv_build_tree_mask.restype = ctypes.c_int
    L.sv_verify_attention_workspace.argtypes = [ctypes.POINTER(sv_attn_desc)]
    L.sv_verify_attention_workspace.restype = ctypes.c_size_t
    L.sv_verify_attention.argtypes = [ctypes.POINTER(sv_attn_desc), _P, ctypes.c_size_t, _P]
    L.sv_verify_attention.restype = ctypes.c_int
    L.sv_spec_accept_workspace.argtypes = [ctypes.POINTER(sv_accept_desc)]
    L.sv_spec_accept_workspace.restype = ctypes.c_size_t
    L.sv_spec_accept.argtypes = [ctypes.POINTER(sv_accept_desc), _P, ctypes.c_size_t, _P]
    L.sv_spec_accept.restype = ctypes.c_int
    L.sv_spec_accept_static.argtypes = [ctypes.POINTER(sv_accept_desc), _P]
    L.sv_spec_accept_static.restype = ctypes.c_int
    L.sv_tree_walk_workspace.argtypes = [ctypes.POINTER(sv_walk_desc)]
    L.sv_tree_walk_workspace.restype = ctypes.c_size_t
    L.sv_tree_walk.argtypes = [ctypes.POINTER(sv_walk_desc), _P, ctypes.c_size_t, _P]
    L.sv_tree_walk.restype = ctypes.c_int
    L.sv_kv_commit.argtypes = [ctypes.POINTER(sv_commit_desc), _P]
    L.sv_kv_commit.restype = ctypes.c_int
    L.sv_truncate_workspace.argtypes = [ctypes.POINTER(sv_trunc_desc)]
    L.sv_truncate_workspace.restype = ctypes.c_size_t
    L.sv_truncate.argtypes = [ctypes.POINTER(sv_trunc_desc), _P, ctypes.c_size_t, _P]
    L.sv_truncate.restype = ctypes.c_int
    L.sv_penalize_workspace.argtypes = [ctypes.POINTER(sv_penalty_desc)]
    L.sv_penalize_workspace.restype = ctypes.c_size_t
    L.sv_penalize.argtypes = [ctypes.POINTER(sv_penalty_desc), _P, ctypes.c_size_t, _P]
    L.sv_penalize.restype = ctypes.c_int
    L.sv_status_string.argtypes = [ctypes.c_int]
    L.sv_status_string.restype = ctypes.c_char_p
    return L


lib = _load()


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s: %s" % (where, lib.sv_status_string(status).decode()))
        self.status = status


def _check(status: int, where: str) -> None:
    if status != SV_OK:
        raise SpecVerifyError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libspecverify takes device tensors")


# workspaces: zeroed once when created; every call leaves them zeroed again
_workspaces: dict = {}


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled, 256-byte aligned device buffer of at least nbytes, reused per
    (device, stream).  Calls that share it must not overlap."""
    key = (torch.device(device).index, torch.cuda.current_stream(device).cuda_stream)
    buf = _workspaces.get(key)
    if buf is None or buf.numel() < nbytes + 256:
        buf = torch.zeros(max(nbytes, 1) + 256, dtype=torch.uint8, device=device)
        _workspaces[key] = buf
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(nbytes, 1)]


# --------------------------------------------------------------------------- #
def sv_build_tree_mask(parents: torch.Tensor, prefix_len: int):
    """-> (bits uint32-as-int32 [n][ceil(n/32)], depth int32 [n], pos int64 [n], status int32 [1])."""
    _need_cuda(parents)
    parents = parents.contiguous().to(torch.int32)
    n = parents.numel()
    dev = parents.device
    bits = torch.empty((n, (n + 31) // 32), dtype=torch.int32, device=dev)
    depth = torch.empty(n, dtype=torch.int32, device=dev)
    pos = torch.empty(n, dtype=torch.int64, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.sv_build_tree_mask(_ptr(parents), n, int(prefix_len), _ptr(bits), _ptr(depth), _ptr(pos),
                                  _ptr(status), _stream(dev)), "sv_build_tree_mask")
    return bits, depth, pos, status


def attn_desc(q, k, v, kv_off, prefix_len, *, Hkv: int, max_prefix: int, scale: float,
              kv_sh: int, kv_st: int, out, lse=None, tree_bits=None, tree_sb: int = 0,
              split_keys: int = 0, kv_sb: int = 0) -> sv_attn_desc:
    B, n_q, Hq, D = q.shape
    d = sv_attn_desc()
    d.dtype = SV_BF16 if q.dtype == torch.bfloat16 else SV_F32
    d.mask = SV_MASK_TREE if tree_bits is not None else SV_MASK_CAUSAL
    d.B, d.n_q, d.Hq, d.Hkv, d.D = B, n_q, Hq, Hkv, D
    d.max_prefix, d.split_keys, d.scale = int(max_prefix), int(split_keys), float(scale)
    d.q = q.data_ptr()
    d.q_sb, d.q_st, d.q_sh = q.stride(0), q.stride(1), q.stride(2)
    d.k, d.v = k.data_ptr(), v.data_ptr()
    d.kv_off = None if kv_off is None else kv_off.data_ptr()
    d.kv_sh, d.kv_st, d.kv_sb = int(kv_sh), int(kv_st), int(kv_sb)
    d.prefix_len = prefix_len.data_ptr()
    d.tree_bits = None if tree_bits is None else tree_bits.data_ptr()
    d.tree_sb = int(tree_sb)
    d.out = out.data_ptr()
    d.o_sb, d.o_st, d.o_sh = out.stride(0), out.stride(1), out.stride(2)
    d.lse = None if lse is None else lse.data_ptr()
    return d


def sv_verify_attention(q, k, v, kv_off, prefix_len, *, Hkv: int, max_prefix: int, scale: float,
                        kv_sh: int, kv_st: int, tree_bits=None, tree_sb: int = 0, out=None,
                        want_lse: bool = False, split_keys: int = 0, kv_sb: int = 0):
    """q [B][n_q][Hq][D] (bf16 or fp32, D contiguous); k, v flat caches of the same dtype;
    kv_off int64 [B], or None for a dense cache whose sequence b starts at element b*kv_sb
    (each sequence then owns max_prefix + n_q token slots); prefix_len int32 [B]; tree_bits
    int32 rows from sv_build_tree_mask (TREE) or None (CAUSAL).
    Returns (out [B][n_q][Hq][D], lse fp32 [B][n_q][Hq] or None)."""
    _need_cuda(q, k, v, kv_off, prefix_len, tree_bits)
    if q.stride(-1) != 1:
        raise ValueError("q must have a contiguous head dimension")
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    d = attn_desc(q, k, v, kv_off, prefix_len, Hkv=Hkv, max_prefix=max_prefix, scale=scale, kv_sh=kv_sh,
                  kv_st=kv_st, out=out, lse=lse, tree_bits=tree_bits, tree_sb=tree_sb, split_keys=split_keys,
                  kv_sb=kv_sb)
    nb = lib.sv_verify_attention_workspace(ctypes.byref(d))
    ws = workspace(nb, q.device)
    _check(lib.sv_verify_attention(ctypes.byref(d), _ptr(ws), nb, _stream(q.device)), "sv_verify_attention")
    return out, lse


def accept_desc(mode, target, draft, draft_tokens, temperature, seed, step, stream_ids,
                accept_len, out_tokens, alpha, dev_status, rule: int = SV_RULE_TOKEN,
                draft_len=None) -> sv_accept_desc:
    B, g1, V = target.shape
    d = sv_accept_desc()
    d.mode, d.B, d.gamma, d.V, d.temperature = int(mode), B, g1 - 1, V, float(temperature)
    d.target_logits = target.data_ptr()
    d.draft_logits = None if draft is None else draft.data_ptr()
    d.draft_tokens = draft_tokens.data_ptr()
    d.rng = sv_philox(int(seed), int(step), None if stream_ids is None else stream_ids.data_ptr())
    d.accept_len, d.out_tokens = accept_len.data_ptr(), out_tokens.data_ptr()
    d.alpha = None if alpha is None else alpha.data_ptr()
    d.dev_status = None if dev_status is None else dev_status.data_ptr()
    d.rule = int(rule)
    d.draft_len = None if draft_len is None else draft_len.data_ptr()
    return d


def sv_spec_accept(mode: int, target, draft, draft_tokens, temperature: float, seed: int, step: int = 0,
                   stream_ids=None, want_alpha: bool = False, rule: int = SV_RULE_TOKEN, draft_len=None):
    """target fp32 [B][gamma+1][V]; draft fp32 [B][gamma][V] (SAMPLE); draft_tokens int32 [B][gamma];
    draft_len optional int32 [B] (drafts each sequence verifies, 0..gamma).
    Returns dict(accept_len, out_tokens, alpha or None, status) as device tensors."""
    _need_cuda(target, draft, draft_tokens, stream_ids, draft_len)
    target = target.contiguous()
    draft = None if draft is None else draft.contiguous()
    draft_tokens = draft_tokens.to(torch.int32).contiguous()
    B, g1, V = target.shape
    dev = target.device
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    out = torch.empty((B, g1), dtype=torch.int32, device=dev)
    alpha = torch.empty((B, g1 - 1), dtype=torch.float32, device=dev) if want_alpha else None
    status = torch.empty(B, dtype=torch.int32, device=dev)
    sid = None if stream_ids is None else stream_ids.to(torch.int64).contiguous()
    dl = None if draft_len is None else draft_len.to(torch.int32).contiguous()
    d = accept_desc(mode, target, draft, draft_tokens, temperature, seed, step, sid, acc, out, alpha, status, rule,
                    dl)
    nb = lib.sv_spec_accept_workspace(ctypes.byref(d))
    ws = workspace(nb, dev)
    _check(lib.sv_spec_accept(ctypes.byref(d), _ptr(ws), nb, _stream(dev)), "sv_spec_accept")
    return dict(accept_len=acc, out_tokens=out, alpha=alpha, status=status)


def sv_spec_accept_static(mode: int, target, draft, draft_tokens, temperature: float, seed: int, step: int = 0,
                          stream_ids=None, want_alpha: bool = False, out=None, draft_len=None):
    """sv_spec_accept on the library's fixed device scratch (no workspace argument).  The
    output tensors can be passed in (``out`` = a dict like the one returned) so that the
    call itself allocates nothing.  Returns that dict."""
    _need_cuda(target, draft, draft_tokens, stream_ids)
    B, g1, V = target.shape
    dev = target.device
    if out is None:
        out = dict(accept_len=torch.empty(B, dtype=torch.int32, device=dev),
                   out_tokens=torch.empty((B, g1), dtype=torch.int32, device=dev),
                   alpha=torch.empty((B, g1 - 1), dtype=torch.float32, device=dev) if want_alpha else None,
                   status=torch.empty(B, dtype=torch.int32, device=dev))
    d = accept_desc(mode, target, draft, draft_tokens, temperature, seed, step, stream_ids, out["accept_len"],
                    out["out_tokens"], out.get("alpha"), out["status"], draft_len=draft_len)
    _check(lib.sv_spec_accept_static(ctypes.byref(d), _stream(dev)), "sv_spec_accept_static")
    return out


def walk_desc(mode, logits, tokens, parents, max_depth, temperature, seed, step, stream_ids,
              accept_len, path, out_tokens, dev_status, rule: int = SV_WALK_MATCH, draft_logits=None,
              max_children: int = 0) -> sv_walk_desc:
    B, n, V = logits.shape
    d = sv_walk_desc()
    d.mode, d.B, d.n, d.V, d.max_depth, d.temperature = int(mode), B, n, V, int(max_depth), float(temperature)
    d.logits, d.tokens, d.parents = logits.data_ptr(), tokens.data_ptr(), parents.data_ptr()
    d.rng = sv_philox(int(seed), int(step), None if stream_ids is None else stream_ids.data_ptr())
    d.accept_len, d.path, d.out_tokens = accept_len.data_ptr(), path.data_ptr(), out_tokens.data_ptr()
    d.dev_status = None if dev_status is None else dev_status.data_ptr()
    d.rule = int(rule)
    d.draft_logits = None if draft_logits is None else draft_logits.data_ptr()
    d.max_children = int(max_children)
    return d


def sv_tree_walk(mode: int, logits, tokens, parents, max_depth: int, temperature: float, seed: int,
                 step: int = 0, stream_ids=None, rule: int = SV_WALK_MATCH, draft_logits=None,
                 max_children: int = 0):
    """logits fp32 [B][n][V]; tokens int32 [B][n]; parents int32 [n].
    Returns dict(accept_len, path, out_tokens, status) as device tensors."""
    _need_cuda(logits, tokens, parents, stream_ids)
    logits = logits.contiguous()
    tokens = tokens.to(torch.int32).contiguous()
    parents = parents.to(torch.int32).contiguous()
    B, n, V = logits.shape
    dev = logits.device
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    out = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    sid = None if stream_ids is None else stream_ids.to(torch.int64).contiguous()
    _need_cuda(draft_logits)
    draft_logits = None if draft_logits is None else draft_logits.contiguous()
    d = walk_desc(mode, logits, tokens, parents, max_depth, temperature, seed, step, sid, acc, path, out, status,
                  rule, draft_logits, max_children)
    nb = lib.sv_tree_walk_workspace(ctypes.byref(d))
    ws = workspace(nb, dev)
    _check(lib.sv_tree_walk(ctypes.byref(d), _ptr(ws), nb, _stream(dev)), "sv_tree_walk")
    return dict(accept_len=acc, path=path, out_tokens=out, status=status)


def commit_desc(k, v, kv_off, prefix_len, accept_len, *, n_q: int, Hkv: int, D: int, kv_sh: int, kv_st: int,
                kv_sb: int = 0, path=None, new_len=None, dev_status=None) -> sv_commit_desc:
    d = sv_commit_desc()
    d.dtype = SV_BF16 if k.dtype == torch.bfloat16 else SV_F32
    d.B, d.n_q, d.Hkv, d.D = prefix_len.numel(), int(n_q), int(Hkv), int(D)
    d.k, d.v = k.data_ptr(), v.data_ptr()
    d.kv_off = None if kv_off is None else kv_off.data_ptr()
    d.kv_sb, d.kv_sh, d.kv_st = int(kv_sb), int(kv_sh), int(kv_st)
    d.prefix_len, d.accept_len = prefix_len.data_ptr(), accept_len.data_ptr()
    d.path = None if path is None else path.data_ptr()
    d.path_stride = 0 if path is None else path.shape[-1]
    d.new_len = (prefix_len if new_len is None else new_len).data_ptr()
    d.dev_status = None if dev_status is None else dev_status.data_ptr()
    return d


def sv_kv_commit(k, v, kv_off, prefix_len, accept_len, *, n_q: int, Hkv: int, D: int, kv_sh: int, kv_st: int,
                 kv_sb: int = 0, path=None, in_place: bool = False):
    """Commit a round in the caches k, v (moved in place).  Returns (new_len int32 [B], status
    int32 [B]); with in_place the new lengths are written into prefix_len as well (and it is
    returned)."""
    _need_cuda(k, v, kv_off, prefix_len, accept_len, path)
    B = prefix_len.numel()
    new_len = prefix_len if in_place else torch.empty(B, dtype=torch.int32, device=k.device)
    status = torch.empty(B, dtype=torch.int32, device=k.device)
    d = commit_desc(k, v, kv_off, prefix_len, accept_len, n_q=n_q, Hkv=Hkv, D=D, kv_sh=kv_sh, kv_st=kv_st,
                    kv_sb=kv_sb, path=None if path is None else path.contiguous(), new_len=new_len,
                    dev_status=status)
    _check(lib.sv_kv_commit(ctypes.byref(d), _stream(k.device)), "sv_kv_commit")
    return new_len, status


# --------------------------------------------------------------------------- #
def trunc_desc(logits, out, *, temperature: float, top_k: int = 0, top_p: float = 1.0, top_k_rows=None,
               top_p_rows=None, kept=None) -> sv_trunc_desc:
    d = sv_trunc_desc()
    d.R, d.V = logits.shape[0], logits.shape[1]
    d.temperature, d.top_k, d.top_p = float(temperature), int(top_k), float(top_p)
    d.top_k_rows = None if top_k_rows is None else top_k_rows.data_ptr()
    d.top_p_rows = None if top_p_rows is None else top_p_rows.data_ptr()
    d.logits, d.out = logits.data_ptr(), out.data_ptr()
    d.kept = None if kept is None else kept.data_ptr()
    return d


def sv_truncate(logits, *, temperature: float, top_k: int = 0, top_p: float = 1.0, top_k_rows=None,
                top_p_rows=None, in_place: bool = False, split: bool = True):
    """Top-k then top-p truncation of fp32 logit rows [R][V] (any leading shape is flattened
    into R); split=False runs without a workspace (the first level then stays in one
    workgroup per row).  Returns (out, kept int32 [R]): out holds the kept tokens' logits and -inf
    elsewhere; with in_place it is `logits` itself (which must then be contiguous fp32)."""
    _need_cuda(logits, top_k_rows, top_p_rows)
    if logits.dtype != torch.float32:
        raise ValueError("sv_truncate takes fp32 logits")
    V = logits.shape[-1]
    if in_place and not logits.is_contiguous():
        raise ValueError("sv_truncate in place needs contiguous logits")
    R = 1
    for n in logits.shape[:-1]:
        R *= n
    x = logits.reshape(R, V) if in_place else logits.contiguous().reshape(R, V)
    out = x if in_place else torch.empty_like(x)
    kept = torch.empty(R, dtype=torch.int32, device=x.device)
    kr = None if top_k_rows is None else top_k_rows.to(torch.int32).contiguous().reshape(R)
    pr = None if top_p_rows is None else top_p_rows.to(torch.float32).contiguous().reshape(R)
    d = trunc_desc(x, out, temperature=temperature, top_k=top_k, top_p=top_p, top_k_rows=kr, top_p_rows=pr,
                   kept=kept)
    nb = lib.sv_truncate_workspace(ctypes.byref(d)) if split else 0
    ws = workspace(nb, x.device) if nb else None
    _check(lib.sv_truncate(ctypes.byref(d), _ptr(ws), nb, _stream(x.device)), "sv_truncate")
    return out.reshape(logits.shape), kept


# --------------------------------------------------------------------------- #
def penalty_desc(logits, *, history=None, hist_len=None, draft_tokens=None, repetition: float = 1.0,
                 frequency: float = 0.0, presence: float = 0.0) -> sv_penalty_desc:
    d = sv_penalty_desc()
    d.B, d.n_rows, d.V = logits.shape
    d.logits = logits.data_ptr()
    d.history = None if history is None else history.data_ptr()
    d.hist_len = None if hist_len is None else hist_len.data_ptr()
    d.hist_stride = 0 if history is None else history.shape[-1]
    d.draft_tokens = None if draft_tokens is None else draft_tokens.data_ptr()
    d.n_drafts = 0 if draft_tokens is None else draft_tokens.shape[-1]
    d.repetition, d.frequency, d.presence = float(repetition), float(frequency), float(presence)
    return d


def sv_penalize(logits, *, history=None, hist_len=None, draft_tokens=None, repetition: float = 1.0,
                frequency: float = 0.0, presence: float = 0.0):
    """Penalties on fp32 logits [B][n_rows][V] in place (which must be contiguous): row i of
    sequence b counts history[b][:hist_len[b]] and draft_tokens[b][:i].  Returns logits."""
    _need_cuda(logits, history, hist_len, draft_tokens)
    if logits.dtype != torch.float32 or logits.dim() != 3 or not logits.is_contiguous():
        raise ValueError("sv_penalize takes contiguous fp32 logits [B][n_rows][V]")
    B = logits.shape[0]
    hs = None if history is None else history.to(torch.int32).contiguous().reshape(B, -1)
    hl = None if hist_len is None else hist_len.to(torch.int32).contiguous().reshape(B)
    dr = None if draft_tokens is None else draft_tokens.to(torch.int32).contiguous().reshape(B, -1)
    d = penalty_desc(logits, history=hs, hist_len=hl, draft_tokens=dr, repetition=repetition, frequency=frequency,
                     presence=presence)
    nb = lib.sv_penalize_workspace(ctypes.byref(d))
    ws = workspace(nb, logits.device)
    _check(lib.sv_penalize(ctypes.byref(d), _ptr(ws), nb, _stream(logits.device)), "sv_penalize")
    return logits
