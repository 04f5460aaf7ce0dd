#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the verify
attention over every sequence's KV cache, then acceptance over the vocabulary (and, for
the tree workloads, the mask build and the tree walk).  The default workload is the
8B-like chain: batch 1, gamma = 5 drafts, 4096 cached tokens, 32 query / 8 KV heads of
128, bf16; vocabulary 128256 with fp32 logits, temperature 0.8, speculative sampling.

Inputs are resident in HBM before the timed region.  Each step reads a different one of
R device copies of the inputs (R * working set >= 1 GiB), so the 256 MB Infinity Cache
cannot serve repeated reads.  Kernel durations come from HIP events recorded on the
stream the library launches on; the main attention kernel's (the roofline's) from events
that hipExtLaunchKernel sets to the kernel's own start and end, the span a kernel trace
reports.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# how the roofline's kernel duration is taken
KERNEL_SPAN = "kernel start to end: hipExtLaunchKernel events on the launch stream, separate eager pass"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--split-keys", type=int, default=0)
    ap.add_argument("--kv-cache", choices=["auto", "ragged"], default="auto",
                    help="auto: dense cache for one sequence, ragged (kv_off) for a batch")
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9)
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of replaying HIP graphs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (reference for the HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of a known size: FETCH_SIZE / WRITE_SIZE of this
    kernel divided by 256 MiB gives the counters' scale factor on this GPU."""
    import torch
    n = 256 * 1024 * 1024 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 4 * n, "launches": 5}))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs on one device per process and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import draft_token_verification_attention_amd as sv
    import synth

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.WORKLOADS[args.workload]
    wl = args.workload
    if cfg["kind"] != "chain":
        return bench_tree(args, cfg, wl, dev)

    # ---------------- inputs (host, seeded) ----------------
    B, gamma = cfg["B"], cfg["gamma"]
    n_q = gamma + 1
    Hq, Hkv, D, V, tau = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["V"], cfg["tau"]
    P = synth.prefix_lengths(wl, cfg)
    max_prefix = int(cfg.get("P_hi", int(P.max())))
    att = synth.attention_inputs(wl, B=B, n_q=n_q, Hq=Hq, Hkv=Hkv, D=D, prefix_len=P, dtype=cfg["dtype"],
                                 qkv_scale=cfg["qkv_scale"])
    acc = synth.accept_inputs(wl, B=B, gamma=gamma, V=V, target_var=cfg["target_var"],
                              noise_var=cfg["noise_var"], tau=tau)
    bf = cfg["dtype"] == "bf16"

    def to_dev(a, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf16 else np.ascontiguousarray(a))
        t = t.view(torch.bfloat16) if bf16 else t
        return t.to(dev)

    base = dict(q=to_dev(att["q"], bf), k=to_dev(att["k"], bf), v=to_dev(att["v"], bf),
                target=to_dev(acc["target"]), draft=to_dev(acc["draft"]))
    # One sequence: a dense cache (kv_off NULL; the sequence owns max_prefix + n_q token
    # slots, which is what the packed buffer holds).  A batch: the packed ragged cache.
    dense = B == 1 and int(P[0]) == max_prefix and args.kv_cache != "ragged"
    kv_off = None if dense else to_dev(att["kv_off"].astype(np.int64))
    kv_sb = (max_prefix + n_q) * Hkv * D if dense else 0
    prefix = to_dev(P.astype(np.int32))
    toks = to_dev(acc["draft_tokens"].astype(np.int32))
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    R = max(1, int(math.ceil(args.rotate_bytes / set_bytes)))
    copies = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(R - 1)]
    scale = 1.0 / math.sqrt(D)
    esz = 2 if bf else 4

    # outputs and descriptors prepared once: the timed loop only launches
    out = torch.empty((B, n_q, Hq, D), dtype=base["q"].dtype, device=dev)
    acc_len = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    import ctypes
    adescs, sdescs = [], []
    for c in copies:
        adescs.append(sv.attn_desc(c["q"], c["k"], c["v"], kv_off, prefix, Hkv=Hkv, max_prefix=max_prefix,
                                   scale=scale, kv_sh=att["kv_sh"], kv_st=att["kv_st"], out=out,
                                   split_keys=args.split_keys, kv_sb=kv_sb))
        sdescs.append(sv.accept_desc(sv.SV_SAMPLE, c["target"], c["draft"], toks, tau, 1000 + wl, 0, None,
                                     acc_len, out_tok, None, status))
    ws_a = sv.lib.sv_verify_attention_workspace(ctypes.byref(adescs[0]))
    ws_s = sv.lib.sv_spec_accept_workspace(ctypes.byref(sdescs[0]))
    ws_att = torch.zeros(ws_a + 256, dtype=torch.uint8, device=dev)
    ws_acc = torch.zeros(ws_s + 256, dtype=torch.uint8, device=dev)
    pa = ctypes.c_void_p(ws_att.data_ptr() + (-ws_att.data_ptr()) % 256)
    ps = ctypes.c_void_p(ws_acc.data_ptr() + (-ws_acc.data_ptr()) % 256)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def launch(r, sh, ev=None):
        if ev is not None:
            ev[0].record()
        st = sv.lib.sv_verify_attention(ctypes.byref(adescs[r]), pa, ws_a, sh)
        if ev is not None:
            ev[1].record()
        st2 = sv.lib.sv_spec_accept(ctypes.byref(sdescs[r]), ps, ws_s, sh)
        if ev is not None:
            ev[2].record()
        if st or st2:
            raise RuntimeError("launch failed: %d %d" % (st, st2))

    for i in range(args.warmup):
        launch(i % R, sh)
    torch.cuda.synchronize()

    ms_per_step = timed_steps(launch, R, args, sh)

    # Kernel durations: HIP events on the launch stream, same K steps.  The library's
    # measurement hooks record one more event right after the main attention kernel (the
    # attention call splits into its main kernel and the split combine) and give the main
    # kernel's own start and end (hipExtLaunchKernel events: the span a kernel trace reports,
    # without the dispatch ahead of the kernel).
    # Two passes over the same K steps: the first with plain launches (call and combine
    # intervals), the second with the kernel-span events (whose launch path adds host work
    # between the events around the call).
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    for e in events:
        for k in (1, 4, 5):
            e[k].record()  # creates the events the library records
    torch.cuda.synchronize()
    for span in (False, True):
        for i in range(args.steps):
            ev = events[i]
            if span:
                sv.lib.sv_set_attention_timing(ctypes.c_void_p(ev[4].cuda_event), ctypes.c_void_p(ev[5].cuda_event))
            else:
                sv.lib.sv_set_attention_mark(ctypes.c_void_p(ev[1].cuda_event))
                ev[0].record()
            st = sv.lib.sv_verify_attention(ctypes.byref(adescs[(args.warmup + i) % R]), pa, ws_a, sh)
            if not span:
                ev[2].record()
            st2 = sv.lib.sv_spec_accept(ctypes.byref(sdescs[(args.warmup + i) % R]), ps, ws_s, sh)
            if not span:
                ev[3].record()
            if st or st2:
                raise RuntimeError("launch failed: %d %d" % (st, st2))
        sv.lib.sv_set_attention_mark(None)
        sv.lib.sv_set_attention_timing(None, None)
        torch.cuda.synchronize()
    main_ms = float(np.mean([e[4].elapsed_time(e[5]) for e in events]))
    main_call_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    comb_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    att_ms = float(np.mean([e[0].elapsed_time(e[2]) for e in events]))
    acc_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))

    drafts = B * gamma
    value = drafts / (ms_per_step * 1e-3)
    kv_tokens = int((P.astype(np.int64) + n_q).sum())
    att_bytes = esz * (B * n_q * Hq * D + 2 * kv_tokens * Hkv * D) + esz * B * n_q * Hq * D
    acc_bytes = 4 * V * B * (2 * gamma + 1)
    main_gbs = att_bytes / (main_ms * 1e-3) / 1e9

    line = {
        "metric": "draft tokens verified/sec on 1 MI355X; achieved HBM GB/s as % of peak",
        "value": round(value, 1),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": B, "gamma": gamma, "cached_context": int(P.max()),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "vocab": V, "temperature": tau,
                   "mode": "sample", "kv_cache": "dense" if dense else "ragged (kv_off)",
                   "rotated_input_copies": R, "launch": "eager" if args.eager else "hip_graph"},
        "roofline": {"bound": "hbm", "achieved": round(main_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(main_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl),
                     "kernel": "attn_bf16_kernel", "kernel_ms": round(main_ms, 5),
                     "timing": KERNEL_SPAN, "algorithmic_bytes": att_bytes},
        "kernels_ms": {"attn_bf16_kernel": round(main_ms, 5), "attn_bf16_kernel_with_dispatch": round(main_call_ms, 5),
                       "attn_combine_kernel": round(comb_ms, 5), "sv_spec_accept": round(acc_ms, 5)},
        "attention": {"kernel_ms": round(att_ms, 5), "algorithmic_bytes": att_bytes,
                      "achieved_GBs": round(att_bytes / (att_ms * 1e-3) / 1e9, 1)},
        "accept": {"kernel_ms": round(acc_ms, 5), "algorithmic_bytes": acc_bytes,
                   "achieved_GBs": round(acc_bytes / (acc_ms * 1e-3) / 1e9, 1)},
    }

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(att, acc, cfg, scale, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def timed_steps(launch, R, args, sh):
    """Warm up, then time exactly args.steps steps (wall clock between two device
    synchronizations); step i reads input copy i mod R.  Unless --eager, the steps are
    replayed from HIP graphs that each hold S consecutive steps (S the largest divisor of
    the step count up to 10), so the host's per-replay cost is spread over S steps; the
    kernels and their arguments are exactly those of the eager launches."""
    import ctypes
    import torch
    K = args.steps
    if args.eager:
        for i in range(args.warmup):
            launch(i % R, sh)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            launch((args.warmup + i) % R, sh)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K
    S = max(d for d in range(1, min(10, K) + 1) if K % d == 0)
    graphs = []
    for r in range(R):  # graph r: the S steps starting at copy r
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for k in range(S):
                launch((r + k) % R, cs)
        graphs.append(g)
    for m in range(max(1, args.warmup // S)):
        graphs[(m * S) % R].replay()
    torch.cuda.synchronize()
    first = args.warmup
    t0 = time.perf_counter()
    for m in range(K // S):
        graphs[(first + m * S) % R].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / K


def bench_tree(args, cfg, wl, dev):
    """A tree round: the mask build from the parent array, the tree attention over the
    cache + node tokens, and the tree walk (sampling, the workload's temperature) over
    the per-node target logits.  Draft tokens verified per step = drafted nodes."""
    import ctypes
    import torch
    import draft_token_verification_attention_amd as sv
    import synth

    parents, paths = synth.build_tree(cfg)
    n = len(parents)
    Hq, Hkv, D, V, tau, P = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["V"], cfg["tau"], cfg["P"]
    att = synth.attention_inputs(wl, B=1, n_q=n, Hq=Hq, Hkv=Hkv, D=D, prefix_len=[P], dtype="bf16",
                                 qkv_scale=cfg["qkv_scale"])
    lg = synth.tree_logits(wl, 1, n, V, cfg["target_var"])
    toks = synth.node_tokens(wl, lg, parents, synth.path_ranks(paths))
    depth = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        depth[i] = depth[parents[i]] + 1
    max_depth = int(depth.max())

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    base = dict(q=bf(att["q"]), k=bf(att["k"]), v=bf(att["v"]), logits=torch.from_numpy(lg).to(dev))
    del lg
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    R = max(1, int(math.ceil(args.rotate_bytes / set_bytes)))
    copies = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(R - 1)]
    par_d = torch.from_numpy(parents.astype(np.int32)).to(dev)
    toks_d = torch.from_numpy(toks.astype(np.int32)).to(dev)
    kv_off = torch.from_numpy(att["kv_off"].astype(np.int64)).to(dev)
    prefix = torch.tensor([P], dtype=torch.int32, device=dev)
    words = (n + 31) // 32
    bits = torch.empty((n, words), dtype=torch.int32, device=dev)
    dep_d = torch.empty(n, dtype=torch.int32, device=dev)
    pos_d = torch.empty(n, dtype=torch.int64, device=dev)
    mstat = torch.empty(1, dtype=torch.int32, device=dev)
    out = torch.empty((1, n, Hq, D), dtype=torch.bfloat16, device=dev)
    acc_len = torch.empty(1, dtype=torch.int32, device=dev)
    path = torch.empty((1, max_depth + 1), dtype=torch.int32, device=dev)
    out_tok = torch.empty((1, max_depth + 1), dtype=torch.int32, device=dev)
    wstat = torch.empty(1, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)
    adescs = [sv.attn_desc(c["q"], c["k"], c["v"], kv_off, prefix, Hkv=Hkv, max_prefix=P, scale=scale,
                           kv_sh=att["kv_sh"], kv_st=att["kv_st"], out=out, tree_bits=bits, tree_sb=0,
                           split_keys=args.split_keys) for c in copies]
    wdescs = [sv.walk_desc(sv.SV_SAMPLE, c["logits"], toks_d, par_d, max_depth, tau, 1000 + wl, 0, None,
                           acc_len, path, out_tok, wstat) for c in copies]
    ws_a = sv.lib.sv_verify_attention_workspace(ctypes.byref(adescs[0]))
    ws_w = sv.lib.sv_tree_walk_workspace(ctypes.byref(wdescs[0]))
    ws_att = torch.zeros(ws_a + 256, dtype=torch.uint8, device=dev)
    ws_wlk = torch.zeros(ws_w + 256, dtype=torch.uint8, device=dev)
    pa = ctypes.c_void_p(ws_att.data_ptr() + (-ws_att.data_ptr()) % 256)
    pw = ctypes.c_void_p(ws_wlk.data_ptr() + (-ws_wlk.data_ptr()) % 256)
    sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def launch(r, sh, ev=None):
        if ev is not None:
            ev[0].record()
        st0 = sv.lib.sv_build_tree_mask(ctypes.c_void_p(par_d.data_ptr()), n, P, ctypes.c_void_p(bits.data_ptr()),
                                        ctypes.c_void_p(dep_d.data_ptr()), ctypes.c_void_p(pos_d.data_ptr()),
                                        ctypes.c_void_p(mstat.data_ptr()), sh)
        if ev is not None:
            ev[1].record()
        st1 = sv.lib.sv_verify_attention(ctypes.byref(adescs[r]), pa, ws_a, sh)
        if ev is not None:
            ev[3].record()
        st2 = sv.lib.sv_tree_walk(ctypes.byref(wdescs[r]), pw, ws_w, sh)
        if ev is not None:
            ev[4].record()
        if st0 or st1 or st2:
            raise RuntimeError("launch failed: %d %d %d" % (st0, st1, st2))

    for i in range(args.warmup):
        launch(i % R, sh)
    torch.cuda.synchronize()
    ms_per_step = timed_steps(launch, R, args, sh)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    for e in events:
        for k in (2, 5, 6):
            e[k].record()  # creates the events the library records
    torch.cuda.synchronize()
    # two passes, as for the chain workloads: plain launches, then the kernel-span events
    for i in range(args.steps):
        sv.lib.sv_set_attention_mark(ctypes.c_void_p(events[i][2].cuda_event))
        launch((args.warmup + i) % R, sh, events[i])
    sv.lib.sv_set_attention_mark(None)
    torch.cuda.synchronize()
    for i in range(args.steps):
        sv.lib.sv_set_attention_timing(ctypes.c_void_p(events[i][5].cuda_event),
                                       ctypes.c_void_p(events[i][6].cuda_event))
        launch((args.warmup + i) % R, sh)
    sv.lib.sv_set_attention_timing(None, None)
    torch.cuda.synchronize()
    mask_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    main_ms = float(np.mean([e[5].elapsed_time(e[6]) for e in events]))
    main_call_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    comb_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in events]))
    walk_ms = float(np.mean([e[3].elapsed_time(e[4]) for e in events]))

    drafted = n - 1
    value = drafted / (ms_per_step * 1e-3)
    anc = int((depth + 1).sum())  # sum over nodes of the ancestor-or-self count
    att_flops = 4.0 * D * Hq * (n * P + anc)
    att_bytes = 2 * (n * Hq * D + 2 * (P + n) * Hkv * D) + 2 * n * Hq * D + 4 * n * words
    main_tflops = att_flops / (main_ms * 1e-3) / 1e12
    main_gbs = att_bytes / (main_ms * 1e-3) / 1e9
    walk_rows = int(to_host_int(acc_len)) + 1
    mfma = {"bound": "mfma", "achieved": round(main_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(main_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(wl),
            "kernel": "attn_bf16_kernel", "kernel_ms": round(main_ms, 5), "timing": KERNEL_SPAN,
            "algorithmic_flops": att_flops}
    hbm = {"bound": "hbm", "achieved": round(main_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(main_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl),
           "kernel": "attn_bf16_kernel", "kernel_ms": round(main_ms, 5), "timing": KERNEL_SPAN,
           "algorithmic_bytes": att_bytes}
    line = {
        "metric": "draft tokens verified/sec on 1 MI355X; achieved HBM GB/s as % of peak",
        "value": round(value, 1), "unit": "draft tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": 1, "tree_nodes": drafted, "cached_context": P,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "vocab": V, "temperature": tau,
                   "mode": "sample", "rotated_input_copies": R, "launch": "eager" if args.eager else "hip_graph"},
        "roofline": mfma if wl == 5 else hbm,
        "roofline_other": hbm if wl == 5 else mfma,
        "kernels_ms": {"tree_mask_kernel": round(mask_ms, 5), "attn_bf16_kernel": round(main_ms, 5),
                       "attn_bf16_kernel_with_dispatch": round(main_call_ms, 5),
                       "attn_combine_kernel": round(comb_ms, 5), "sv_tree_walk": round(walk_ms, 5)},
        "walk": {"kernel_ms": round(walk_ms, 5), "rows_visited": walk_rows,
                 "algorithmic_bytes": 4 * V * walk_rows},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline_tree(att, cfg, wl, parents, toks, scale, args.cpu_seconds)
    print(json.dumps(line), flush=True)


def to_host_int(t):
    return int(t.cpu().numpy().ravel()[0])


def cpu_baseline_tree(att, cfg, wl, parents, toks, scale, seconds):
    """The oracle on a bounded sample: the mask, the fp64 attention of a seeded sample of
    rows (timed, then scaled to every row) and the tree walk, repeated for ~`seconds`."""
    import oracle
    import synth
    threads = os.cpu_count() or 1
    oracle.set_threads(threads)
    n, Hq = len(parents), cfg["Hq"]
    total_rows = n * Hq
    r = np.random.default_rng(wl)
    nsample = min(total_rows, 4096)
    pick = r.choice(total_rows, size=nsample, replace=False)
    rows = np.stack([np.zeros(nsample, np.int64), pick // Hq, pick % Hq], 1).astype(np.int32)
    lg = synth.tree_logits(wl, 1, n, cfg["V"], cfg["target_var"]) if n <= 128 else None
    t_mask = t_att = t_walk = 0.0
    reps = 0
    t0 = time.perf_counter()
    while True:
        ta = time.perf_counter()
        bits = oracle.tree_mask(parents, cfg["P"])[0]
        tb = time.perf_counter()
        oracle.attention(att, scale=scale, tree_bits=bits, tree_sb=0, rows=rows)
        tc = time.perf_counter()
        if lg is not None:
            oracle.tree_walk(oracle.SAMPLE, lg, toks, parents, cfg["tau"], seed=1000 + wl, step=reps)
        td = time.perf_counter()
        t_mask += tb - ta
        t_att += tc - tb
        t_walk += td - tc
        reps += 1
        if time.perf_counter() - t0 >= seconds:
            break
    step_s = (t_mask + t_att * total_rows / nsample + t_walk) / reps
    return {"value": round((n - 1) / step_s, 3), "unit": "draft tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d reps of: mask, fp64 attention of %d of %d rows (time scaled to all rows)%s"
                      % (reps, nsample, total_rows, ", tree walk" if lg is not None else
                         "; walk not sampled (its 2.4 GB logits stay off the host leg)")}


# HBM bytes per launch of attn_bf16_kernel (2 x FETCH_SIZE + WRITE_SIZE, the FETCH_SIZE
# counter reading half the bytes of a plain copy of known size on this GPU), from the
# rocprofv3 --pmc runs summarized under profiles/, and the SHA-256 of the attention source
# they were taken on: a changed kernel reports null until the counters are taken again.
TRAFFIC = {2: 19146491, 4: 1110644725}
TRAFFIC_SRC_SHA256 = "f0181d9ba00dab5aead0be6b439625055d682b4177dd223d0d4fe6d7c20343a0"


def measured_traffic(wl):
    import hashlib
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "draft_token_verification_attention_amd",
                       "csrc", "attention.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if sha != TRAFFIC_SRC_SHA256 or wl not in TRAFFIC:
        return None
    return TRAFFIC[wl]


def cpu_baseline(att, acc, cfg, scale, seconds):
    """The fp64 oracle, as it stands, on the host cores: whole steps of the same workload
    (attention over every row, then sampling acceptance), repeated for ~`seconds`."""
    import oracle
    threads = os.cpu_count() or 1
    oracle.set_threads(threads)
    gamma, tau = cfg["gamma"], cfg["tau"]
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.attention(att, scale=scale)
        oracle.spec_accept(oracle.SAMPLE, acc["target"], acc["draft"], acc["draft_tokens"], tau, seed=1000, step=n)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = (time.perf_counter() - t0) / n
    return {"value": round(cfg["B"] * gamma / dt, 2), "unit": "draft tokens/s", "cores": threads,
            "kind": "oracle", "sample": "%d whole steps of the same workload (all attention rows + acceptance)" % n}


if __name__ == "__main__":
    main()
