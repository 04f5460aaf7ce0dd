#!/usr/bin/env python3
"""Benchmark of the speculative-decoding verify step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the verify
attention over every sequence's KV cache, then acceptance over the vocabulary (and, for
the tree workloads, the mask build and the tree walk).  The default workload is the
batched chain: 64 sequences, gamma = 4 drafts each, cached contexts uniform in
[512, 8192], 32 query / 8 KV heads of 128, bf16; vocabulary 128256 with fp32 logits,
temperature 1.0, speculative sampling with a Philox stream per sequence.

Inputs are resident in HBM before the timed region.  Each step reads a different one of
R device copies of the inputs (R * working set >= 1.1 GB), so the 256 MB Infinity Cache
cannot serve repeated reads.  The timed steps replay HIP graphs of consecutive steps.
Kernel durations come from HIP events on the stream the library launches on: the
attention call takes events in its descriptor that hipExtLaunchKernel sets to its
kernels' own start and end (the span a kernel trace reports).

The line also carries: the roofline of the attention pass (main kernel + split combine,
the dominant cost), the CPU oracle timed on the host (all cores and one thread, on a
bounded sample) with a parity verdict of the GPU step against it (decisions bit-exact
except near-threshold draws, which are counted; attention max-abs error), and, unless
--no-extra, short runs of the 8B-like chain and the full Cartesian tree (its MFMA
utilisation against the bf16 dense peak).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4] [--no-cpu] [--no-extra]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
KERNEL_SPAN = ("kernel start to end: hipExtLaunchKernel events on the launch stream, "
               "separate eager pass over the same steps")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the short runs of the other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--split-keys", type=int, default=0)
    ap.add_argument("--kv-cache", choices=["auto", "ragged"], default="auto",
                    help="auto: dense cache for one sequence, ragged (kv_off) for a batch")
    ap.add_argument("--rotate-bytes", type=float, default=1.1e9)
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of replaying HIP graphs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy 5 times (reference for the HBM byte counters)")
    ap.add_argument("--latency-floor", action="store_true",
                    help="only time plain device operations of the 8B chain's attention size (16.9 MB): a copy, "
                         "a one-pass reduction, and a 4-byte copy (the launch floor)")
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


def latency_floor(reps=200):
    """What one sequence's attention is measured against: plain device operations over the
    8B chain's attention bytes (16,900,096: Q, K/V of 4102 keys x 8 KV heads x 128, O), each
    launched back to back `reps` times, median of HIP event intervals (the kernel trace of the
    same run gives the kernels' own spans)."""
    import torch
    n = 16900096 // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    tiny_s = torch.ones(2, dtype=torch.bfloat16, device="cuda")
    tiny_d = torch.empty_like(tiny_s)
    out = torch.empty((), dtype=torch.float32, device="cuda")
    ops = {"copy_16.9MB": lambda: dst.copy_(src),
           "sum_16.9MB": lambda: torch.sum(src, dim=0, dtype=torch.float32, out=out),
           "copy_4B": lambda: tiny_d.copy_(tiny_s)}
    res = {}
    for name, op in ops.items():
        for _ in range(20):
            op()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            op()
            e1.record()
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
        res[name + "_us"] = round(1e3 * t[len(t) // 2], 2)
    print(json.dumps({"latency_floor": res, "bytes": 16900096, "reps": reps}))


def host_threads() -> int:
    """Host threads this process may use: its CPU affinity, capped by OMP_NUM_THREADS."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.latency_floor:
        latency_floor()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library runs on one device per process and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import draft_token_verification_attention_amd  # noqa: F401  (fails loudly without the library)

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    line = run_workload(args.workload, args, dev, args.steps, args.warmup, cpu=not args.no_cpu, headline=True)
    if not args.no_extra:
        extra = {}
        for wl in (2, 3, 5):
            if wl == args.workload:
                continue
            r = run_workload(wl, args, dev, 50, 5, cpu=False, headline=False)
            extra[r["config"]["workload"]] = {k: r[k] for k in ("value", "unit", "ms_per_step", "roofline",
                                                                 "roofline_other", "kernels_ms", "next_rows")
                                              if k in r}
        line["other_workloads"] = extra
    print(json.dumps(line), flush=True)


def run_workload(wl, args, dev, steps, warmup, cpu, headline):
    import synth
    cfg = synth.WORKLOADS[wl]
    if cfg["kind"] == "chain":
        return bench_chain(args, cfg, wl, dev, steps, warmup, cpu)
    return bench_tree(args, cfg, wl, dev, steps, warmup, cpu)


def _bf16_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


def _f32_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def _aligned(buf):
    return ctypes.c_void_p(buf.data_ptr() + (-buf.data_ptr()) % 256)


def _ev(e):
    return ctypes.c_void_p(e.cuda_event)


def attention_timing(sv, adescs, ws, R, first, steps, run_rest, sh):
    """Per-kernel durations over the same steps the timed region ran, in two eager passes:
    events around the calls (dispatch included), then the descriptor's kernel-span events
    (main kernel start/end, end of the call's last kernel).  ws = (workspace, bytes) of the
    attention call; run_rest(r) launches the rest of the step after it.  Medians."""
    import torch
    n_ev = 8
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    for e in events:
        for k in (4, 5, 6):
            e[k].record()  # creates the events the library records
    torch.cuda.synchronize()
    for span in (False, True):
        for i in range(steps):
            ev = events[i]
            d = adescs[(first + i) % R]
            if span:
                d.ev_kernel_start, d.ev_kernel_stop, d.ev_call_stop = _ev(ev[4]), _ev(ev[5]), _ev(ev[6])
            else:
                ev[0].record()
            st = sv.lib.sv_verify_attention(ctypes.byref(d), ws[0], ws[1], sh)
            d.ev_kernel_start = d.ev_kernel_stop = d.ev_call_stop = None
            if not span:
                ev[1].record()
            run_rest((first + i) % R)
            if not span:
                ev[2].record()
            if st:
                raise RuntimeError("attention launch failed: %d" % st)
        torch.cuda.synchronize()
    t = lambda a, b: float(np.median([e[a].elapsed_time(e[b]) for e in events]))  # noqa: E731
    return dict(main=t(4, 5), attn_span=t(4, 6), combine=t(5, 6), attn_call=t(0, 1), rest=t(1, 2))


def median_event_ms(call, steps, sh):
    """Median over `steps` eager calls of the time between events recorded on the launch
    stream right before and right after each call (dispatch included)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(3):
        call(i)
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(ev):
        e0.record()
        call(i)
        e1.record()
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))


def time_accept_rule(sv, copies, toks, tau, seed, rule, shape, steps, sh, dev):
    """sv_spec_accept under another rule on the same inputs (the GPU's own inputs, rotated)."""
    import torch
    B, gamma, V = shape
    R = len(copies)
    acc_len = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    descs = [sv.accept_desc(sv.SV_SAMPLE, c["target"], c["draft"], toks, tau, seed, 0, None, acc_len, out_tok, None,
                            status, rule) for c in copies]
    nb = sv.lib.sv_spec_accept_workspace(ctypes.byref(descs[0]))
    ws = torch.zeros(nb + 256, dtype=torch.uint8, device=dev)
    pw = _aligned(ws)

    def call(i):
        if sv.lib.sv_spec_accept(ctypes.byref(descs[i % R]), pw, nb, sh):
            raise RuntimeError("acceptance launch failed")
    ms = median_event_ms(call, steps, sh)
    rows = (2 * gamma + 1) if rule != sv.SV_RULE_GUMBEL else (gamma + 1)
    nbytes = 4 * V * B * rows
    out = {"kernel_ms": round(ms, 5), "value": round(B * gamma / (ms * 1e-3), 1), "unit": "draft tokens/s (acceptance alone)",
           "algorithmic_bytes": nbytes, "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "mean_accepted": float(acc_len.float().mean().item())}
    if rule == sv.SV_RULE_GUMBEL:
        out["note"] = ("ALU-bound: a Philox4x64-10 block per four tokens and two fp32 logarithms per token (fp64 scores only for the few tokens near each chunk's best); "
                       "drafts from the workload's own sampler (independent noise), which changes no cost")
    return out


def time_truncate(sv, copies, tau, top_k, top_p, steps, sh, dev):
    """sv_truncate on both models' rows of the round (target [B][gamma+1][V] and draft
    [B][gamma][V]; two calls per step, into separate output buffers so the inputs stay as they
    are).  Algorithmic bytes: every logit read once and written once."""
    import torch
    R = len(copies)
    outs = {k: torch.empty_like(copies[0][k]) for k in ("target", "draft")}
    kept = {k: torch.empty(copies[0][k].numel() // copies[0][k].shape[-1], dtype=torch.int32, device=dev)
            for k in ("target", "draft")}
    V = copies[0]["target"].shape[-1]
    descs = [[sv.trunc_desc(c[k].reshape(-1, V), outs[k].reshape(-1, V), temperature=tau, top_k=top_k,
                            top_p=top_p, kept=kept[k]) for k in ("target", "draft")] for c in copies]

    nb = max(sv.lib.sv_truncate_workspace(ctypes.byref(d)) for dd in descs for d in dd)
    ws = torch.zeros(nb + 256, dtype=torch.uint8, device=dev)
    pw = _aligned(ws)

    def call(i):
        for d in descs[i % R]:
            if sv.lib.sv_truncate(ctypes.byref(d), pw, nb, sh):
                raise RuntimeError("truncate launch failed")
    ms = median_event_ms(call, steps, sh)
    rows = sum(kept[k].numel() for k in kept)
    nbytes = 8 * V * rows
    return {"kernel_ms": round(ms, 5), "rows": rows, "top_k": top_k, "top_p": top_p,
            "algorithmic_bytes": nbytes, "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "mean_kept": round(float(torch.cat([kept["target"], kept["draft"]]).float().mean().item()), 1),
            "bound": "hbm (the row is read 2 to 3 times: selection passes, then a gather pass that writes)"}


def time_penalize(sv, base, toks, hist_tokens, steps, sh, dev):
    """sv_penalize on both models' rows of the round (two calls per step), each sequence with a
    history of hist_tokens random tokens and its drafts as the rows' prefixes.  It runs in
    place on a scratch copy of the rows (repeated calls compound the penalty, which changes
    no cost).  Work is per history entry, not per logit."""
    import torch
    B = toks.shape[0]
    V = base["target"].shape[-1]
    rows = {k: base[k].clone() for k in ("target", "draft")}
    g = torch.Generator(device="cpu").manual_seed(17)
    hist = torch.randint(0, V, (B, hist_tokens), generator=g, dtype=torch.int32).to(dev)
    descs = [sv.penalty_desc(rows[k], history=hist, draft_tokens=toks, repetition=1.2, frequency=0.3, presence=0.2)
             for k in ("target", "draft")]
    nb = max(sv.lib.sv_penalize_workspace(ctypes.byref(d)) for d in descs)
    ws = torch.zeros(nb + 256, dtype=torch.uint8, device=dev)
    pw = _aligned(ws)

    def call(i):
        for d in descs:
            if sv.lib.sv_penalize(ctypes.byref(d), pw, nb, sh):
                raise RuntimeError("penalize launch failed")
    ms = median_event_ms(call, steps, sh)
    nrows = sum(r.shape[0] * r.shape[1] for r in rows.values())
    return {"kernel_ms": round(ms, 5), "rows": nrows, "history_tokens": hist_tokens, "launches": 4,
            "bound": "scattered logits (two dependent launches per call: the history counted in LDS, then "
                     "about one read and write of a logit per distinct history token per row)"}


def time_commit(sv, k, v, kv_off, prefix, acc_len, path, n_q, Hkv, D, kv_sh, kv_st, kv_sb, esize, steps, sh, dev):
    """sv_kv_commit on the given caches (new lengths to a separate buffer, so every call
    moves the same rows).  Algorithmic bytes: the moved K and V rows, read and written."""
    import torch
    B = prefix.numel()
    new_len = torch.empty(B, dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    d = sv.commit_desc(k, v, kv_off, prefix, acc_len, n_q=n_q, Hkv=Hkv, D=D, kv_sh=kv_sh, kv_st=kv_st, kv_sb=kv_sb,
                       path=path, new_len=new_len, dev_status=status)

    def call(i):
        if sv.lib.sv_kv_commit(ctypes.byref(d), sh):
            raise RuntimeError("commit launch failed")
    ms = median_event_ms(call, steps, sh)
    moved = 0
    if path is not None:
        J = acc_len.cpu().numpy()
        pth = path.cpu().numpy()
        moved = int(sum(int((pth[b, 1:J[b] + 1] != np.arange(1, J[b] + 1)).sum()) for b in range(B)))
    nbytes = moved * Hkv * D * esize * 2 * 2
    return {"kernel_ms": round(ms, 5), "rows_moved": moved, "algorithmic_bytes": nbytes,
            "achieved_GBs": round(nbytes / (ms * 1e-3) / 1e9, 3) if nbytes else 0.0,
            "bound": "latency (one block per sequence; a few KB to move)"}


def timed_steps(launch, R, steps, warmup, eager, sh):
    """Warm up, then time exactly `steps` steps (wall clock between two device
    synchronizations); step i reads input copy i mod R.  Unless eager, the steps are
    replayed from HIP graphs that each hold S consecutive steps (S the largest divisor of
    the step count up to 10), so the host's per-replay cost is spread over S steps; the
    kernels and their arguments are exactly those of the eager launches."""
    import torch
    K = steps
    if eager:
        for i in range(warmup):
            launch(i % R, sh)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            launch((warmup + i) % R, sh)
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
    for m in range(max(1, warmup // S)):
        graphs[(m * S) % R].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for m in range(K // S):
        graphs[(warmup + m * S) % R].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / K


# --------------------------------------------------------------------------- #
def bench_chain(args, cfg, wl, dev, steps, warmup, cpu):
    import torch
    import draft_token_verification_attention_amd as sv
    import synth

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
    todev = (lambda a: _bf16_dev(a, dev)) if bf else (lambda a: _f32_dev(a, dev))
    base = dict(q=todev(att["q"]), k=todev(att["k"]), v=todev(att["v"]),
                target=_f32_dev(acc["target"], dev), draft=_f32_dev(acc["draft"], dev))
    # One sequence: a dense cache (kv_off NULL; the sequence owns max_prefix + n_q token
    # slots, which is what the packed buffer holds).  A batch: the packed ragged cache.
    dense = B == 1 and int(P[0]) == max_prefix and args.kv_cache != "ragged"
    kv_off = None if dense else _f32_dev(att["kv_off"].astype(np.int64), dev)
    kv_sb = (max_prefix + n_q) * Hkv * D if dense else 0
    prefix = _f32_dev(P.astype(np.int32), dev)
    toks = _f32_dev(acc["draft_tokens"].astype(np.int32), dev)
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    R = max(1, int(math.ceil(args.rotate_bytes / set_bytes)))
    copies = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(R - 1)]
    scale = 1.0 / math.sqrt(D)
    esz = 2 if bf else 4
    seed = 1000 + wl

    # outputs and descriptors prepared once: the timed loop only launches
    out = torch.empty((B, n_q, Hq, D), dtype=base["q"].dtype, device=dev)
    acc_len = torch.empty(B, dtype=torch.int32, device=dev)
    out_tok = torch.empty((B, n_q), dtype=torch.int32, device=dev)
    status = torch.empty(B, dtype=torch.int32, device=dev)
    adescs, sdescs = [], []
    for c in copies:
        adescs.append(sv.attn_desc(c["q"], c["k"], c["v"], kv_off, prefix, Hkv=Hkv, max_prefix=max_prefix,
                                   scale=scale, kv_sh=att["kv_sh"], kv_st=att["kv_st"], out=out,
                                   split_keys=args.split_keys, kv_sb=kv_sb))
        sdescs.append(sv.accept_desc(sv.SV_SAMPLE, c["target"], c["draft"], toks, tau, seed, 0, None,
                                     acc_len, out_tok, None, status))
    ws_a = sv.lib.sv_verify_attention_workspace(ctypes.byref(adescs[0]))
    ws_s = sv.lib.sv_spec_accept_workspace(ctypes.byref(sdescs[0]))
    ws_att = torch.zeros(ws_a + 256, dtype=torch.uint8, device=dev)
    ws_acc = torch.zeros(ws_s + 256, dtype=torch.uint8, device=dev)
    pa, ps = _aligned(ws_att), _aligned(ws_acc)
    sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def launch(r, sh):
        st = sv.lib.sv_verify_attention(ctypes.byref(adescs[r]), pa, ws_a, sh)
        st2 = sv.lib.sv_spec_accept(ctypes.byref(sdescs[r]), ps, ws_s, sh)
        if st or st2:
            raise RuntimeError("launch failed: %d %d" % (st, st2))

    for i in range(warmup):
        launch(i % R, sh)
    torch.cuda.synchronize()
    ms_per_step = timed_steps(launch, R, steps, warmup, args.eager, sh)

    def rest(r):
        if sv.lib.sv_spec_accept(ctypes.byref(sdescs[r]), ps, ws_s, sh):
            raise RuntimeError("acceptance launch failed")
    t = attention_timing(sv, adescs, (pa, ws_a), R, warmup, steps, rest, sh)

    drafts = B * gamma
    value = drafts / (ms_per_step * 1e-3)
    kv_tokens = int((P.astype(np.int64) + n_q).sum())
    att_bytes = esz * (B * n_q * Hq * D + 2 * kv_tokens * Hkv * D) + esz * B * n_q * Hq * D
    acc_bytes = 4 * V * B * (2 * gamma + 1)
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9  # noqa: E731
    traffic = measured_traffic(wl)
    line = {
        "metric": "draft tokens verified/sec on 1 MI355X; achieved HBM GB/s as % of peak",
        "value": round(value, 1),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": B, "gamma": gamma,
                   "cached_context": ("uniform [%d, %d]" % (cfg["P_lo"], cfg["P_hi"])) if "P_lo" in cfg
                   else int(P.max()),
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "vocab": V, "temperature": tau,
                   "mode": "sample", "kv_cache": "dense" if dense else "ragged (kv_off)",
                   "rotated_input_copies": R, "launch": "eager" if args.eager else "hip_graph"},
        "roofline": {"bound": "hbm", "achieved": round(gbs(att_bytes, t["attn_span"]), 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs(att_bytes, t["attn_span"]) / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else traffic["attention"],
                     "kernel": "attention pass: attn_bf16_kernel + attn_combine_kernel" if bf else "attn_f32_kernel",
                     "kernel_ms": round(t["attn_span"], 5), "timing": KERNEL_SPAN + "; main kernel start to "
                     "the end of the call's last kernel, median over the steps", "algorithmic_bytes": att_bytes,
                     "main_kernel_only": {"kernel_ms": round(t["main"], 5),
                                          "achieved": round(gbs(att_bytes, t["main"]), 1),
                                          "frac": round(gbs(att_bytes, t["main"]) / HBM_PEAK_GBS, 4),
                                          "traffic": None if traffic is None else traffic["main"]}},
        "kernels_ms": {"attn_bf16_kernel": round(t["main"], 5), "attn_combine_kernel": round(t["combine"], 5),
                       "attention_call_with_dispatch": round(t["attn_call"], 5),
                       "sv_spec_accept": round(t["rest"], 5)},
        "attention": {"kernel_ms": round(t["attn_span"], 5), "algorithmic_bytes": att_bytes,
                      "achieved_GBs": round(gbs(att_bytes, t["attn_span"]), 1)},
        "accept": {"kernel_ms": round(t["rest"], 5), "algorithmic_bytes": acc_bytes,
                   "achieved_GBs": round(gbs(acc_bytes, t["rest"]), 1)},
    }
    if bf:
        line["next_rows"] = {
            "block_verification": time_accept_rule(sv, copies, toks, tau, seed, sv.SV_RULE_BLOCK, (B, gamma, V),
                                                   steps, sh, dev),
            "gumbel_verification": time_accept_rule(sv, copies, toks, tau, seed, sv.SV_RULE_GUMBEL, (B, gamma, V),
                                                    steps, sh, dev),
            "kv_commit_chain": time_commit(sv, base["k"], base["v"], kv_off, prefix, acc_len, None, n_q, Hkv, D,
                                           att["kv_sh"], att["kv_st"], kv_sb, esz, steps, sh, dev),
            "truncate_top_k_top_p": time_truncate(sv, copies, tau, 50, 0.9, steps, sh, dev),
            "truncate_top_p": time_truncate(sv, copies, tau, 0, 0.9, steps, sh, dev),
            "penalize_history_4096": time_penalize(sv, base, toks, 4096, steps, sh, dev),
        }
    if cpu:
        # the GPU's own outputs for the step on copy 0 (seed, step 0), for the parity verdict
        launch(0, sh)
        torch.cuda.synchronize()
        gpu = dict(out=out.float().cpu().numpy(), accept_len=acc_len.cpu().numpy(),
                   out_tokens=out_tok.cpu().numpy(), status=status.cpu().numpy())
        line["cpu_baseline"] = cpu_baseline_chain(att, acc, cfg, scale, seed, gpu, args.cpu_seconds)
    return line


def bench_tree(args, cfg, wl, dev, steps, warmup, cpu):
    """A tree round: the mask build from the parent array, the tree attention over the
    cache + node tokens, and the tree walk (sampling, the workload's temperature) over
    the per-node target logits.  Draft tokens verified per step = drafted nodes."""
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

    base = dict(q=_bf16_dev(att["q"], dev), k=_bf16_dev(att["k"], dev), v=_bf16_dev(att["v"], dev),
                logits=_f32_dev(lg, dev))
    lg_host = lg if cpu and n <= 128 else None
    del lg
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    R = max(1, int(math.ceil(args.rotate_bytes / set_bytes)))
    copies = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(R - 1)]
    par_d = _f32_dev(parents.astype(np.int32), dev)
    toks_d = _f32_dev(toks.astype(np.int32), dev)
    kv_off = _f32_dev(att["kv_off"].astype(np.int64), dev)
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
    seed = 1000 + wl
    adescs = [sv.attn_desc(c["q"], c["k"], c["v"], kv_off, prefix, Hkv=Hkv, max_prefix=P, scale=scale,
                           kv_sh=att["kv_sh"], kv_st=att["kv_st"], out=out, tree_bits=bits, tree_sb=0,
                           split_keys=args.split_keys) for c in copies]
    wdescs = [sv.walk_desc(sv.SV_SAMPLE, c["logits"], toks_d, par_d, max_depth, tau, seed, 0, None,
                           acc_len, path, out_tok, wstat) for c in copies]
    ws_a = sv.lib.sv_verify_attention_workspace(ctypes.byref(adescs[0]))
    ws_w = sv.lib.sv_tree_walk_workspace(ctypes.byref(wdescs[0]))
    ws_att = torch.zeros(ws_a + 256, dtype=torch.uint8, device=dev)
    ws_wlk = torch.zeros(ws_w + 256, dtype=torch.uint8, device=dev)
    pa, pw = _aligned(ws_att), _aligned(ws_wlk)
    sh = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    vp = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731

    def mask(sh):
        return sv.lib.sv_build_tree_mask(vp(par_d), n, P, vp(bits), vp(dep_d), vp(pos_d), vp(mstat), sh)

    def launch(r, sh):
        st0 = mask(sh)
        st1 = sv.lib.sv_verify_attention(ctypes.byref(adescs[r]), pa, ws_a, sh)
        st2 = sv.lib.sv_tree_walk(ctypes.byref(wdescs[r]), pw, ws_w, sh)
        if st0 or st1 or st2:
            raise RuntimeError("launch failed: %d %d %d" % (st0, st1, st2))

    for i in range(warmup):
        launch(i % R, sh)
    torch.cuda.synchronize()
    ms_per_step = timed_steps(launch, R, steps, warmup, args.eager, sh)

    def rest(r):
        if sv.lib.sv_tree_walk(ctypes.byref(wdescs[r]), pw, ws_w, sh):
            raise RuntimeError("walk launch failed")
    t = attention_timing(sv, adescs, (pa, ws_a), R, warmup, steps, rest, sh)
    # the mask build alone
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        ev[2 * i].record()
        mask(sh)
        ev[2 * i + 1].record()
    torch.cuda.synchronize()
    mask_ms = float(np.median([ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(steps)]))

    drafted = n - 1
    value = drafted / (ms_per_step * 1e-3)
    anc = int((depth + 1).sum())  # sum over nodes of the ancestor-or-self count
    att_flops = 4.0 * D * Hq * (n * P + anc)
    att_bytes = 2 * (n * Hq * D + 2 * (P + n) * Hkv * D) + 2 * n * Hq * D + 4 * n * words
    traffic = measured_traffic(wl)
    tr_attn = None if traffic is None else traffic["attention"]
    span = t["attn_span"]
    mfma = {"bound": "mfma", "achieved": round(att_flops / (span * 1e-3) / 1e12, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(att_flops / (span * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": tr_attn, "kernel": "attention pass: attn_bf16_kernel + attn_combine_kernel",
            "kernel_ms": round(span, 5), "timing": KERNEL_SPAN, "algorithmic_flops": att_flops,
            "main_kernel_only": {"kernel_ms": round(t["main"], 5),
                                 "frac": round(att_flops / (t["main"] * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}}
    hbm = {"bound": "hbm", "achieved": round(att_bytes / (span * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(att_bytes / (span * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": tr_attn,
           "kernel": "attention pass: attn_bf16_kernel + attn_combine_kernel", "kernel_ms": round(span, 5),
           "timing": KERNEL_SPAN, "algorithmic_bytes": att_bytes,
           "main_kernel_only": {"kernel_ms": round(t["main"], 5),
                                "frac": round(att_bytes / (t["main"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    walk_rows = int(acc_len.cpu().numpy()[0]) + 1
    # next rows: the KV commit of the walked branch (on a copy of the caches), and for the
    # small tree the walk by recursive rejection (draft logits = target + N(0, 1) noise)
    # the commit gathers the tree's deepest branch (the longest the walk can accept; a sampled
    # walk of one step often accepts few nodes)
    leaf = int(np.argmax(depth))
    branch = []
    while leaf >= 0:
        branch.append(leaf)
        leaf = int(parents[leaf])
    branch = branch[::-1]
    cpath = torch.full((1, max_depth + 1), -1, dtype=torch.int32)
    cpath[0, :len(branch)] = torch.tensor(branch, dtype=torch.int32)
    cacc = torch.tensor([len(branch) - 1], dtype=torch.int32, device=dev)
    kc, vc = base["k"].clone(), base["v"].clone()
    nxt = {"kv_commit_tree": time_commit(sv, kc, vc, kv_off, prefix, cacc, cpath.to(dev), n, Hkv, D, att["kv_sh"],
                                         att["kv_st"], 0, 2, steps, sh, dev)}
    nxt["kv_commit_tree"]["branch"] = branch
    del kc, vc
    if n <= 128:
        lg_d = base["logits"]
        noise = torch.from_numpy(synth.normal(wl, "draft_noise", (1, n, V))).to(dev)
        dr_d = lg_d + noise
        kids = np.bincount(parents[1:], minlength=n)
        mk = int(kids.max())
        rdesc = sv.walk_desc(sv.SV_SAMPLE, lg_d, toks_d, par_d, max_depth, tau, seed, 0, None, acc_len, path, out_tok,
                             wstat, sv.SV_WALK_RRS, dr_d, mk)
        nb = sv.lib.sv_tree_walk_workspace(ctypes.byref(rdesc))
        wsr = torch.zeros(nb + 256, dtype=torch.uint8, device=dev)
        pr = _aligned(wsr)

        def rcall(i):
            rdesc.rng.step = i
            if sv.lib.sv_tree_walk(ctypes.byref(rdesc), pr, nb, sh):
                raise RuntimeError("rrs walk failed")
        ms = median_event_ms(rcall, steps, sh)
        nxt["rrs_walk"] = {"kernel_ms": round(ms, 5), "max_children": mk,
                           "launches": (max_depth + 1) * (1 + mk),
                           "note": "node tokens of the workload's drafter; draft logits = target + N(0,1)",
                           "bound": "latency (launches per level: one node pass and max_children try passes)"}
        del noise, dr_d
    line = {
        "metric": "draft tokens verified/sec on 1 MI355X; achieved HBM GB/s as % of peak",
        "value": round(value, 1), "unit": "draft tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": 1, "tree_nodes": drafted, "cached_context": P,
                   "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "vocab": V, "temperature": tau,
                   "mode": "sample", "rotated_input_copies": R, "launch": "eager" if args.eager else "hip_graph"},
        "roofline": mfma if wl == 5 else hbm,
        "roofline_other": hbm if wl == 5 else mfma,
        "kernels_ms": {"tree_mask_kernel": round(mask_ms, 5), "attn_bf16_kernel": round(t["main"], 5),
                       "attn_combine_kernel": round(t["combine"], 5),
                       "attention_call_with_dispatch": round(t["attn_call"], 5), "sv_tree_walk": round(t["rest"], 5)},
        "walk": {"kernel_ms": round(t["rest"], 5), "rows_visited": walk_rows, "algorithmic_bytes": 4 * V * walk_rows},
        "next_rows": nxt,
    }
    if cpu:
        launch(0, sh)
        torch.cuda.synchronize()
        gpu = dict(out=out.float().cpu().numpy(), path=path.cpu().numpy(), accept_len=acc_len.cpu().numpy(),
                   out_tokens=out_tok.cpu().numpy())
        line["cpu_baseline"] = cpu_baseline_tree(att, cfg, wl, parents, toks, lg_host, scale, seed, gpu,
                                                 args.cpu_seconds)
    return line


# --------------------------------------------------------------------------- #
# HBM bytes per launch (2 x FETCH_SIZE + WRITE_SIZE, the FETCH_SIZE counter reading half the
# bytes of a plain copy of known size on this GPU) from the rocprofv3 --pmc runs summarized
# under profiles/, with the SHA-256 of the attention source they were taken on: a changed
# kernel reports null until the counters are taken again.  "attention" = main + combine.
TRAFFIC = {4: {"main": 1103875984, "attention": 1114254469}, 2: {"main": 18523994, "attention": 20082557},
           3: {"main": 12744732, "attention": 16869067}, 5: {"main": 779440131, "attention": 779440131}}
TRAFFIC_SRC_SHA256 = "1da0c4c16669d3df29669342ac71374c7675655c3a0617a6cfe80a1f66b73ead"


def measured_traffic(wl):
    import hashlib
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "draft_token_verification_attention_amd",
                       "csrc", "attention.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if sha != TRAFFIC_SRC_SHA256 or wl not in TRAFFIC:
        return None
    return TRAFFIC[wl]


def _parity_accept(ref, gpu):
    flagged = ref["flags"] != 0
    same = (ref["accept_len"] == gpu["accept_len"]) & np.all(ref["out_tokens"] == gpu["out_tokens"], axis=1)
    return {"sequences": int(len(same)), "bit_exact": int(same.sum()), "near_threshold": int(flagged.sum()),
            "mismatched_near_threshold": int((~same & flagged).sum()),
            "mismatched_other": int((~same & ~flagged).sum())}


def cpu_baseline_chain(att, acc, cfg, scale, seed, gpu, seconds):
    """The fp64 oracle, as it stands, on the host: whole steps of the same workload on all
    host threads (attention of every row, then sampling acceptance), repeated for about
    `seconds`; then one thread on a bounded sample (the attention rows and acceptance of
    the first sequences, scaled to the whole step).  The first all-threads step runs on
    the inputs, seed and step of the GPU step whose outputs `gpu` holds: its results give
    the parity verdict."""
    import oracle
    threads = host_threads()
    oracle.set_threads(threads)
    B, gamma, tau = cfg["B"], cfg["gamma"], cfg["tau"]
    n = 0
    parity = None
    t0 = time.perf_counter()
    while True:
        o, _, rows = oracle.attention(att, scale=scale)
        r = oracle.spec_accept(oracle.SAMPLE, acc["target"], acc["draft"], acc["draft_tokens"], tau, seed=seed,
                               step=n)
        if n == 0:
            got = gpu["out"][rows[:, 0], rows[:, 1], rows[:, 2]]
            parity = {"accept": _parity_accept(r, gpu), "gpu_status_nonzero": int((gpu["status"] != 0).sum()),
                      "attention_rows": int(len(rows)), "attention_max_abs": float(np.abs(got - o).max()),
                      "attention_max_abs_over_max_out": float(np.abs(got - o).max() / np.abs(o).max()),
                      "attention_bound": 2e-2 if att["dtype"] == "bf16" else 1e-4}
            parity["verdict"] = bool(parity["accept"]["mismatched_other"] == 0 and parity["gpu_status_nonzero"] == 0
                                     and parity["attention_max_abs"] <= parity["attention_bound"])
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt_all = (time.perf_counter() - t0) / n
    # one thread: the first k sequences, attention rows and acceptance timed apart and
    # scaled to the whole step by their share of the cached keys and of the sequences
    oracle.set_threads(1)
    k = max(1, min(B, 2))
    rows = np.array([(b, i, h) for b in range(k) for i in range(att["n_q"]) for h in range(att["Hq"])], np.int32)
    keys_all = float((att["prefix_len"].astype(np.int64) + att["n_q"]).sum())
    keys_k = float((att["prefix_len"][:k].astype(np.int64) + att["n_q"]).sum())
    m, ta, tc = 0, 0.0, 0.0
    t1 = time.perf_counter()
    while True:
        t2 = time.perf_counter()
        oracle.attention(att, scale=scale, rows=rows)
        t3 = time.perf_counter()
        oracle.spec_accept(oracle.SAMPLE, acc["target"][:k], acc["draft"][:k], acc["draft_tokens"][:k], tau,
                           seed=seed, step=m)
        tc += time.perf_counter() - t3
        ta += t3 - t2
        m += 1
        if time.perf_counter() - t1 >= seconds:
            break
    dt_one = (ta * keys_all / keys_k + tc * B / k) / m
    oracle.set_threads(threads)
    return {"value": round(B * gamma / dt_all, 3), "unit": "draft tokens/s", "cores": threads, "kind": "oracle",
            "sample": "%d whole steps of the same workload (every attention row + acceptance of every sequence)"
                      % n,
            "single_thread": {"value": round(B * gamma / dt_one, 3), "cores": 1,
                              "sample": "%d reps of the attention rows and the acceptance of the first %d of %d "
                                        "sequences, timed apart and scaled by their share of the cached keys "
                                        "(x%.2f) and of the sequences (x%.1f)"
                                        % (m, k, B, keys_all / keys_k, B / k)},
            "host_cpu": host_cpu_model(), "parity": parity}


def cpu_baseline_tree(att, cfg, wl, parents, toks, lg, scale, seed, gpu, seconds):
    """The oracle on a bounded sample: the mask, the fp64 attention of a seeded sample of
    rows (timed, then scaled to every row) and the tree walk, repeated for ~`seconds`;
    the first repetition's rows and walk (seed and step of the GPU step whose outputs
    `gpu` holds) give the parity verdict."""
    import oracle
    threads = host_threads()
    oracle.set_threads(threads)
    n, Hq = len(parents), cfg["Hq"]
    total_rows = n * Hq
    r = np.random.default_rng(wl)
    nsample = min(total_rows, 4096)
    pick = np.sort(r.choice(total_rows, size=nsample, replace=False))
    rows = np.stack([np.zeros(nsample, np.int64), pick // Hq, pick % Hq], 1).astype(np.int32)
    t_mask = t_att = t_walk = 0.0
    reps = 0
    parity = None
    t0 = time.perf_counter()
    while True:
        ta = time.perf_counter()
        bits = oracle.tree_mask(parents, cfg["P"])[0]
        tb = time.perf_counter()
        o, _, _ = oracle.attention(att, scale=scale, tree_bits=bits, tree_sb=0, rows=rows)
        tc = time.perf_counter()
        w = None
        if lg is not None:
            w = oracle.tree_walk(oracle.SAMPLE, lg, toks, parents, cfg["tau"], seed=seed, step=reps)
        td = time.perf_counter()
        if reps == 0:
            got = gpu["out"][rows[:, 0], rows[:, 1], rows[:, 2]]
            parity = {"attention_rows": int(nsample), "attention_max_abs": float(np.abs(got - o).max()),
                      "attention_bound": 2e-2}
            ok = parity["attention_max_abs"] <= 2e-2
            if w is not None:
                same = bool(np.array_equal(w["path"], gpu["path"]) and np.array_equal(w["out_tokens"], gpu["out_tokens"]))
                parity["walk"] = {"bit_exact": same, "near_threshold": int((w["flags"] != 0).sum())}
                ok = ok and (same or bool(w["flags"][0]))
            parity["verdict"] = bool(ok)
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
                         "; walk not sampled (its 2.4 GB logits stay off the host leg)"),
            "host_cpu": host_cpu_model(), "parity": parity}


if __name__ == "__main__":
    main()
