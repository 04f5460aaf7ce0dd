"""Helpers for the GPU parity tests: move synth inputs to the device, run the C-ABI
library through its binding, bring results back.  No verify arithmetic here."""
import numpy as np
import torch

import draft_token_verification_attention_amd as sv

DEV = "cuda"


def dev_array(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dense_cache(inp: dict, slots: int):
    """The packed K/V of `inp` re-laid as a dense [B][slots][Hkv][D] cache whose unused token
    slots hold NaN (so a kernel that lets them reach the result fails the comparison)."""
    B, Hkv, D, n_q = inp["B"], inp["Hkv"], inp["D"], inp["n_q"]
    out = []
    for name in ("k", "v"):
        src = inp[name]
        dst = np.full((B, slots, Hkv, D), np.nan, dtype=np.float32)
        if src.dtype != np.float32:  # bf16 bit patterns (uint16): NaN is 0x7fc0
            dst = np.full((B, slots, Hkv, D), 0x7FC0, dtype=src.dtype)
        for b in range(B):
            t = min(int(inp["prefix_len"][b]) + n_q, slots)
            o = int(inp["kv_off"][b])
            dst[b, :t] = src[o:o + t * Hkv * D].reshape(t, Hkv, D)
        out.append(dst.reshape(-1))
    return out[0], out[1], slots * Hkv * D


def attention_on_gpu(inp: dict, scale: float, tree_bits=None, tree_sb: int = 0, split_keys: int = 0,
                     max_prefix=None, dense: bool = False):
    bf = inp["dtype"] == "bf16"
    q = dev_array(inp["q"], bf)
    pl = dev_array(inp["prefix_len"].astype(np.int32))
    tb = None if tree_bits is None else dev_array(np.ascontiguousarray(tree_bits).view(np.int32))
    mp = int(inp["prefix_len"].max()) if max_prefix is None else int(max_prefix)
    if dense:  # kv_off NULL: sequence b at element b * kv_sb, max_prefix + n_q slots each
        kd, vd, kv_sb = dense_cache(inp, mp + inp["n_q"])
        k, v, kv_off = dev_array(kd, bf), dev_array(vd, bf), None
    else:
        k, v, kv_sb = dev_array(inp["k"], bf), dev_array(inp["v"], bf), 0
        kv_off = dev_array(inp["kv_off"].astype(np.int64))
    out, lse = sv.sv_verify_attention(q, k, v, kv_off, pl, Hkv=inp["Hkv"], max_prefix=mp, scale=scale,
                                      kv_sh=inp["kv_sh"], kv_st=inp["kv_st"], tree_bits=tb, tree_sb=tree_sb,
                                      want_lse=True, split_keys=split_keys, kv_sb=kv_sb)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


def rows_of(out: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Pick (b, i, h) rows out of a [B][n_q][Hq][...] array."""
    return out[rows[:, 0], rows[:, 1], rows[:, 2]]


def to_host(d: dict) -> dict:
    torch.cuda.synchronize()
    return {k: (None if v is None else v.cpu().numpy()) for k, v in d.items()}
