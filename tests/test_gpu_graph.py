"""HIP-graph capture of the verify step: a captured attention + acceptance sequence is
replayed several times, with eager calls on other inputs and host synchronizations in
between, and every replay must equal the eager result on the same inputs."""
import ctypes
import math

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import draft_token_verification_attention_amd as sv  # noqa: E402
from svgpu import dev_array  # noqa: E402


def _inputs(seed, P):
    att = synth.attention_inputs(seed, B=2, n_q=6, Hq=32, Hkv=8, D=128, prefix_len=[P, P // 3 + 7], dtype="bf16",
                                 qkv_scale=1.0)
    acc = synth.accept_inputs(seed, B=2, gamma=5, V=20000, target_var=3.0, noise_var=1.0, tau=0.8)
    return att, acc


def test_graph_replays_match_eager():
    att, acc = _inputs(1, 3000)
    q, k, v = dev_array(att["q"], True), dev_array(att["k"], True), dev_array(att["v"], True)
    kv_off, pl = dev_array(att["kv_off"]), dev_array(att["prefix_len"])
    tgt, dr, tok = dev_array(acc["target"]), dev_array(acc["draft"]), dev_array(acc["draft_tokens"])
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    alen = torch.empty(2, dtype=torch.int32, device="cuda")
    otok = torch.empty((2, 6), dtype=torch.int32, device="cuda")
    ad = sv.attn_desc(q, k, v, kv_off, pl, Hkv=8, max_prefix=3000, scale=1 / math.sqrt(128), kv_sh=att["kv_sh"],
                      kv_st=att["kv_st"], out=out, lse=lse, split_keys=256)
    sd = sv.accept_desc(sv.SV_SAMPLE, tgt, dr, tok, 0.8, 99, 3, None, alen, otok, None, None)
    wa = torch.zeros(sv.lib.sv_verify_attention_workspace(ctypes.byref(ad)) + 256, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(sv.lib.sv_spec_accept_workspace(ctypes.byref(sd)) + 256, dtype=torch.uint8, device="cuda")
    pa = ctypes.c_void_p(wa.data_ptr() + (-wa.data_ptr()) % 256)
    ps = ctypes.c_void_p(ws.data_ptr() + (-ws.data_ptr()) % 256)

    def launch(stream):
        assert sv.lib.sv_verify_attention(ctypes.byref(ad), pa, wa.numel() - 256, stream) == 0
        assert sv.lib.sv_spec_accept(ctypes.byref(sd), ps, ws.numel() - 256, stream) == 0

    launch(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone(), alen.clone(), otok.clone())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    other_att, other_acc = _inputs(2, 1500)
    for rep in range(5):
        out.zero_(), lse.zero_(), alen.zero_(), otok.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1]), rep
        assert torch.equal(alen, ref[2]) and torch.equal(otok, ref[3]), rep
        # eager work on other inputs (and the shared binding workspace) between replays
        sv.sv_verify_attention(dev_array(other_att["q"], True), dev_array(other_att["k"], True),
                               dev_array(other_att["v"], True), dev_array(other_att["kv_off"]),
                               dev_array(other_att["prefix_len"]), Hkv=8, max_prefix=1500, scale=0.1,
                               kv_sh=other_att["kv_sh"], kv_st=other_att["kv_st"], split_keys=128)
        sv.sv_spec_accept(sv.SV_SAMPLE, dev_array(other_acc["target"]), dev_array(other_acc["draft"]),
                          dev_array(other_acc["draft_tokens"]), 0.8, 5, rep)
        torch.cuda.synchronize()


def test_tree_round_graph_replays_match_eager():
    """Mask build, tree attention and the sampled level-by-level walk (one launch per
    depth, completion counters in a shared workspace) captured once and replayed."""
    parents = synth.random_tree(3, 150, branch_p=0.8)
    n = len(parents)
    depth = np.zeros(n, np.int64)
    for i in range(1, n):
        depth[i] = depth[parents[i]] + 1 if parents[i] >= 0 else 0
    md = int(depth.max())
    P = 700
    att = synth.attention_inputs(4, B=1, n_q=n, Hq=16, Hkv=4, D=128, prefix_len=[P], dtype="bf16", qkv_scale=1.0)
    lg = synth.tree_logits(4, 1, n, 9000, 3.0)
    toks = synth.node_tokens(4, lg, parents)
    par = dev_array(np.asarray(parents, np.int32))
    q, k, v = dev_array(att["q"], True), dev_array(att["k"], True), dev_array(att["v"], True)
    kv_off, pl = dev_array(att["kv_off"]), dev_array(att["prefix_len"])
    lgd, tkd = dev_array(lg), dev_array(toks.astype(np.int32))
    words = (n + 31) // 32
    bits = torch.empty((n, words), dtype=torch.int32, device="cuda")
    dep = torch.empty(n, dtype=torch.int32, device="cuda")
    pos = torch.empty(n, dtype=torch.int64, device="cuda")
    mst = torch.empty(1, dtype=torch.int32, device="cuda")
    out = torch.empty(q.shape, dtype=q.dtype, device="cuda")
    alen = torch.empty(1, dtype=torch.int32, device="cuda")
    path = torch.empty((1, md + 1), dtype=torch.int32, device="cuda")
    otok = torch.empty((1, md + 1), dtype=torch.int32, device="cuda")
    wst = torch.empty(1, dtype=torch.int32, device="cuda")
    ad = sv.attn_desc(q, k, v, kv_off, pl, Hkv=4, max_prefix=P, scale=1 / math.sqrt(128), kv_sh=att["kv_sh"],
                      kv_st=att["kv_st"], out=out, tree_bits=bits)
    wd = sv.walk_desc(sv.SV_SAMPLE, lgd, tkd, par, md, 0.7, 17, 2, None, alen, path, otok, wst)
    wa = torch.zeros(sv.lib.sv_verify_attention_workspace(ctypes.byref(ad)) + 256, dtype=torch.uint8, device="cuda")
    ww = torch.zeros(sv.lib.sv_tree_walk_workspace(ctypes.byref(wd)) + 256, dtype=torch.uint8, device="cuda")
    pa = ctypes.c_void_p(wa.data_ptr() + (-wa.data_ptr()) % 256)
    pw = ctypes.c_void_p(ww.data_ptr() + (-ww.data_ptr()) % 256)

    def launch(stream):
        assert sv.lib.sv_build_tree_mask(ctypes.c_void_p(par.data_ptr()), n, P, ctypes.c_void_p(bits.data_ptr()),
                                         ctypes.c_void_p(dep.data_ptr()), ctypes.c_void_p(pos.data_ptr()),
                                         ctypes.c_void_p(mst.data_ptr()), stream) == 0
        assert sv.lib.sv_verify_attention(ctypes.byref(ad), pa, wa.numel() - 256, stream) == 0
        assert sv.lib.sv_tree_walk(ctypes.byref(wd), pw, ww.numel() - 256, stream) == 0

    launch(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    outs = (bits, dep, pos, out, alen, path, otok, wst)
    ref = tuple(t.clone() for t in outs)
    assert int(mst.cpu()[0]) == 0 and int(wst.cpu()[0]) == 0

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        launch(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    other = synth.tree_logits(5, 2, 40, 3000, 3.0)
    other_par = synth.random_tree(6, 40, branch_p=0.7)
    other_tok = synth.node_tokens(6, other, other_par)
    for rep in range(5):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for j, (t, r) in enumerate(zip(outs, ref)):
            assert torch.equal(t, r), (rep, j)
        # eager walks and masks on other inputs (the binding's own workspace) between replays
        sv.sv_tree_walk(sv.SV_SAMPLE, dev_array(other), dev_array(other_tok.astype(np.int32)),
                        dev_array(np.asarray(other_par, np.int32)), 6, 0.9, rep, 0)
        sv.sv_build_tree_mask(dev_array(np.asarray(other_par, np.int32)), 11)
        torch.cuda.synchronize()


def test_processed_round_graph_replays_match_eager():
    """Penalties, top-k / top-p and the acceptance on the processed rows, captured once (rows
    copied into work buffers first, since the processing runs in place) and replayed with
    eager processing of other rows between replays: every replay equals the eager result."""
    B, g, V, T = 6, 4, 20000, 0.8
    acc = synth.accept_inputs(7, B=B, gamma=g, V=V, target_var=3.0, noise_var=1.0, tau=T)
    src_t, src_d, tok = dev_array(acc["target"]), dev_array(acc["draft"]), dev_array(acc["draft_tokens"])
    hist = dev_array(np.random.default_rng(3).integers(0, 500, (B, 300)).astype(np.int32))
    wt, wd = torch.empty_like(src_t), torch.empty_like(src_d)
    kt = torch.empty(B * (g + 1), dtype=torch.int32, device="cuda")
    kd = torch.empty(B * g, dtype=torch.int32, device="cuda")
    alen = torch.empty(B, dtype=torch.int32, device="cuda")
    otok = torch.empty((B, g + 1), dtype=torch.int32, device="cuda")
    pen = dict(repetition=1.3, frequency=0.2, presence=0.3)
    pds = [sv.penalty_desc(w, history=hist, draft_tokens=tok, **pen) for w in (wt, wd)]
    tds = [sv.trunc_desc(wt.reshape(-1, V), wt.reshape(-1, V), temperature=T, top_k=50, top_p=0.9, kept=kt),
           sv.trunc_desc(wd.reshape(-1, V), wd.reshape(-1, V), temperature=T, top_k=50, top_p=0.9, kept=kd)]
    sd = sv.accept_desc(sv.SV_SAMPLE, wt, wd, tok, T, 11, 2, None, alen, otok, None, None)
    npw = max(sv.lib.sv_penalize_workspace(ctypes.byref(d)) for d in pds)
    wp = torch.zeros(npw + 256, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(sv.lib.sv_spec_accept_workspace(ctypes.byref(sd)) + 256, dtype=torch.uint8, device="cuda")
    pp = ctypes.c_void_p(wp.data_ptr() + (-wp.data_ptr()) % 256)
    ps = ctypes.c_void_p(ws.data_ptr() + (-ws.data_ptr()) % 256)
    ntw = max(sv.lib.sv_truncate_workspace(ctypes.byref(d)) for d in tds)
    wtr = torch.zeros(ntw + 256, dtype=torch.uint8, device="cuda")
    pt = ctypes.c_void_p(wtr.data_ptr() + (-wtr.data_ptr()) % 256)

    def launch(stream):
        wt.copy_(src_t)
        wd.copy_(src_d)
        for d in pds:
            assert sv.lib.sv_penalize(ctypes.byref(d), pp, npw, stream) == 0
        for d in tds:
            assert sv.lib.sv_truncate(ctypes.byref(d), pt, ntw, stream) == 0
        assert sv.lib.sv_spec_accept(ctypes.byref(sd), ps, ws.numel() - 256, stream) == 0

    launch(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    ref = [x.clone() for x in (wt, wd, kt, kd, alen, otok)]

    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        launch(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    other = synth.accept_inputs(8, B=3, gamma=2, V=5000, target_var=2.0, noise_var=1.0, tau=T)
    for rep in range(4):
        for x in (wt, wd, kt, kd, alen, otok):
            x.zero_()
        gr.replay()
        torch.cuda.synchronize()
        for x, r in zip((wt, wd, kt, kd, alen, otok), ref):
            assert torch.equal(x, r), rep
        # eager processing of other rows (the binding's own workspace) between replays
        o = dev_array(other["target"])
        sv.sv_penalize(o, history=dev_array(np.arange(40, dtype=np.int32).reshape(1, 40).repeat(3, 0)),
                       draft_tokens=dev_array(other["draft_tokens"]), repetition=1.5)
        sv.sv_truncate(o, temperature=T, top_p=0.7, in_place=True)
        torch.cuda.synchronize()
