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
stream the library launches on.

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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline leg")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--split-keys", type=int, default=0)
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
        print("bench.py measures one GPU: this build has no multi-GPU path (see DESIGN.md on sharding); "
              "run with --gpus 1", file=sys.stderr)
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
        print("tree workloads are measured by bench_tree (not yet wired)", file=sys.stderr)
        sys.exit(2)

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
    kv_off = to_dev(att["kv_off"].astype(np.int64))
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
                                   split_keys=args.split_keys))
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

    # One HIP graph per input copy: a step is one graph replay (the attention kernels and the
    # acceptance kernels, captured on torch's capture stream; no memset nodes).
    graphs = []
    if not args.eager:
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                launch(r, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % R].replay()
        torch.cuda.synchronize()

    # timed region: exactly K steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if graphs:
            graphs[(args.warmup + i) % R].replay()
        else:
            launch((args.warmup + i) % R, sh)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Kernel durations: HIP events on the launch stream, same K steps.  The library's
    # measurement hook records one more event right after the main attention kernel, so the
    # attention call splits into its main kernel and the split combine.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in events:
        e[1].record()  # creates the event the library will record
    torch.cuda.synchronize()
    for i in range(args.steps):
        sv.lib.sv_set_attention_mark(ctypes.c_void_p(events[i][1].cuda_event))
        ev = events[i]
        ev[0].record()
        st = sv.lib.sv_verify_attention(ctypes.byref(adescs[(args.warmup + i) % R]), pa, ws_a, sh)
        ev[2].record()
        st2 = sv.lib.sv_spec_accept(ctypes.byref(sdescs[(args.warmup + i) % R]), ps, ws_s, sh)
        ev[3].record()
        if st or st2:
            raise RuntimeError("launch failed: %d %d" % (st, st2))
    sv.lib.sv_set_attention_mark(None)
    torch.cuda.synchronize()
    main_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in events]))
    comb_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in events]))
    att_ms = main_ms + comb_ms
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
                   "mode": "sample", "rotated_input_copies": R, "launch": "eager" if args.eager else "hip_graph"},
        "roofline": {"bound": "hbm", "achieved": round(main_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(main_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl),
                     "kernel": "attn_bf16_kernel", "kernel_ms": round(main_ms, 5),
                     "algorithmic_bytes": att_bytes},
        "kernels_ms": {"attn_bf16_kernel": round(main_ms, 5), "attn_combine_kernel": round(comb_ms, 5),
                       "sv_spec_accept": round(acc_ms, 5)},
        "attention": {"kernel_ms": round(att_ms, 5), "algorithmic_bytes": att_bytes,
                      "achieved_GBs": round(att_bytes / (att_ms * 1e-3) / 1e9, 1)},
        "accept": {"kernel_ms": round(acc_ms, 5), "algorithmic_bytes": acc_bytes,
                   "achieved_GBs": round(acc_bytes / (acc_ms * 1e-3) / 1e9, 1)},
    }

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(att, acc, cfg, scale, args.cpu_seconds)
    print(json.dumps(line), flush=True)


# HBM bytes per launch of attn_bf16_kernel (2 x FETCH_SIZE + WRITE_SIZE, the FETCH_SIZE
# counter reading half the bytes of a plain copy of known size on this GPU), from the
# rocprofv3 --pmc runs summarized under profiles/, and the SHA-256 of the attention source
# they were taken on: a changed kernel reports null until the counters are taken again.
TRAFFIC = {2: 19184474, 4: 1128595583}
TRAFFIC_SRC_SHA256 = "feddf9da971373ac9862f47a7ecddd282c880e8a9988f6dd24097bc1577af88c"


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
