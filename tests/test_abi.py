"""CPU checks of the C-ABI library: it loads, exports every symbol include/specverify.h
declares, and its host-side argument checks return the documented status codes without
touching a device (no launch happens on these paths)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")

sv = pytest.importorskip("draft_token_verification_attention_amd")


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SV_API\s+[\w\s\*]+?\b(sv_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_symbols()
    assert len(names) == len(sv.EXPORTS), names
    for n in names:
        assert hasattr(sv.lib, n), n
    assert set(names) == set(sv.EXPORTS)


def test_library_keeps_no_mutable_state():
    """The only data symbols of the built library are the kernels' host-side handles, the
    toolchain's own registration and runtime symbols, and sv_spec_accept_static's fixed
    device array with the per-device record of its address: no other file-scope or
    function-local static variable carries state from one call to the next."""
    import subprocess
    out = subprocess.run(["nm", "-C", sv.LIB_PATH], check=True, capture_output=True, text=True).stdout
    data = [ln.split(" ", 2)[2] for ln in out.splitlines() if re.match(r"^[0-9a-f]+ [bBdD] ", ln)]
    allowed = re.compile(r"^(_DYNAMIC|_GLOBAL_OFFSET_TABLE_|__\w+(\.\w+)?|DW\.ref\.__\w+|.*_kernel(<.*>)?\(.*\)|"
                         # sv_spec_accept_static's fixed device array and the record of its address
                         r"scratch|\(anonymous namespace\)::g_scratch_(ptr|mutex))$")
    stray = [d for d in data if not allowed.match(d)]
    assert not stray, stray


def test_status_strings():
    assert sv.lib.sv_status_string(0) == b"SV_OK"
    assert sv.lib.sv_status_string(3) == b"SV_ERR_WORKSPACE"
    assert sv.lib.sv_status_string(99) == b"SV_UNKNOWN_STATUS"


FAKE = 0x100000  # never dereferenced: every case below fails before a launch


def _attn(**kw):
    d = sv.sv_attn_desc()
    d.dtype, d.mask = sv.SV_BF16, sv.SV_MASK_CAUSAL
    d.B, d.n_q, d.Hq, d.Hkv, d.D, d.max_prefix, d.scale = 1, 6, 32, 8, 128, 4096, 0.088
    d.q = d.k = d.v = d.kv_off = d.prefix_len = d.out = FAKE
    d.q_sb, d.q_st, d.q_sh = 6 * 32 * 128, 32 * 128, 128
    d.kv_sh, d.kv_st = 128, 8 * 128
    d.o_sb, d.o_st, d.o_sh = 6 * 32 * 128, 32 * 128, 128
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("change,status", [
    (dict(D=96), sv.SV_ERR_UNSUPPORTED),
    (dict(Hq=30), sv.SV_ERR_INVALID_ARG),
    (dict(n_q=0), sv.SV_ERR_INVALID_ARG),
    (dict(q=None), sv.SV_ERR_INVALID_ARG),
    (dict(mask=sv.SV_MASK_TREE), sv.SV_ERR_INVALID_ARG),        # tree without bits
    (dict(kv_st=1001), sv.SV_ERR_UNSUPPORTED),                   # not a multiple of 8 elements
    (dict(q=FAKE + 8), sv.SV_ERR_UNSUPPORTED),                   # misaligned
    (dict(max_prefix=-1), sv.SV_ERR_INVALID_ARG),
    (dict(scale=0.0), sv.SV_ERR_INVALID_ARG),
    (dict(scale=-0.088), sv.SV_ERR_INVALID_ARG),
    (dict(scale=float("nan")), sv.SV_ERR_INVALID_ARG),
    (dict(dtype=7), sv.SV_ERR_INVALID_ARG),
    (dict(kv_off=None, kv_sb=-8), sv.SV_ERR_INVALID_ARG),        # dense cache, negative stride
    (dict(kv_off=None, kv_sb=1001), sv.SV_ERR_UNSUPPORTED),      # dense cache, unaligned stride
    (dict(kv_off=None, kv_sb=4102 * 1024), sv.SV_ERR_WORKSPACE), # dense cache: valid
    ({}, sv.SV_ERR_WORKSPACE),                                   # valid, but no workspace
    (dict(B=70000), sv.SV_ERR_UNSUPPORTED),                      # few rows per KV head: grid's sequence limit
])
def test_attention_argument_checks(change, status):
    d = _attn(**change)
    assert sv.lib.sv_verify_attention(ctypes.byref(d), None, 0, None) == status


def test_attention_workspace_sizes():
    d = _attn()
    n = sv.lib.sv_verify_attention_workspace(ctypes.byref(d))
    assert n > 0 and n % 256 == 0
    assert sv.lib.sv_verify_attention_workspace(ctypes.byref(_attn(D=96))) == 0
    f = _attn(dtype=sv.SV_F32)
    assert sv.lib.sv_verify_attention_workspace(ctypes.byref(f)) == 0
    b0 = _attn(B=0)
    assert sv.lib.sv_verify_attention(ctypes.byref(b0), None, 0, None) == sv.SV_OK   # empty batch: no-op


def _acc(**kw):
    d = sv.sv_accept_desc()
    d.mode, d.B, d.gamma, d.V, d.temperature = sv.SV_SAMPLE, 4, 5, 128256, 0.8
    d.target_logits = d.draft_logits = d.draft_tokens = d.accept_len = d.out_tokens = FAKE
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("change,status", [
    (dict(gamma=0), sv.SV_ERR_INVALID_ARG),
    (dict(gamma=65), sv.SV_ERR_UNSUPPORTED),
    (dict(V=0), sv.SV_ERR_INVALID_ARG),
    (dict(temperature=-1.0), sv.SV_ERR_INVALID_ARG),
    (dict(temperature=float("nan")), sv.SV_ERR_INVALID_ARG),
    (dict(draft_logits=None), sv.SV_ERR_INVALID_ARG),           # sampling needs draft logits
    (dict(mode=5), sv.SV_ERR_INVALID_ARG),
    ({}, sv.SV_ERR_WORKSPACE),
    (dict(B=0), sv.SV_OK),
])
def test_accept_argument_checks(change, status):
    d = _acc(**change)
    assert sv.lib.sv_spec_accept(ctypes.byref(d), None, 0, None) == status


def test_accept_workspace_grows_with_batch_and_vocab():
    a = sv.lib.sv_spec_accept_workspace(ctypes.byref(_acc()))
    b = sv.lib.sv_spec_accept_workspace(ctypes.byref(_acc(B=64)))
    c = sv.lib.sv_spec_accept_workspace(ctypes.byref(_acc(V=1000)))
    assert 0 < c < a < b


def _walk(**kw):
    d = sv.sv_walk_desc()
    d.mode, d.B, d.n, d.V, d.max_depth, d.temperature = sv.SV_GREEDY, 1, 65, 128256, 4, 0.7
    d.logits = d.tokens = d.parents = d.accept_len = d.path = d.out_tokens = FAKE
    for k, v in kw.items():
        setattr(d, k, v)
    return d


@pytest.mark.parametrize("change,status", [
    (dict(n=0), sv.SV_ERR_INVALID_ARG),
    (dict(max_depth=-1), sv.SV_ERR_INVALID_ARG),
    (dict(max_depth=64), sv.SV_ERR_UNSUPPORTED),
    (dict(parents=None), sv.SV_ERR_INVALID_ARG),
    ({}, sv.SV_ERR_WORKSPACE),
    (dict(B=0), sv.SV_OK),
])
def test_walk_argument_checks(change, status):
    d = _walk(**change)
    assert sv.lib.sv_tree_walk(ctypes.byref(d), None, 0, None) == status


def test_tree_mask_argument_checks():
    L = sv.lib
    assert L.sv_build_tree_mask(None, 5, 0, FAKE, FAKE, FAKE, FAKE, None) == sv.SV_ERR_INVALID_ARG
    assert L.sv_build_tree_mask(FAKE, 0, 0, FAKE, FAKE, FAKE, FAKE, None) == sv.SV_ERR_INVALID_ARG
    assert L.sv_build_tree_mask(FAKE, 5, -1, FAKE, FAKE, FAKE, FAKE, None) == sv.SV_ERR_INVALID_ARG


def test_oracle_and_library_share_nothing():
    """The oracle never imports the HIP package and the package never imports the oracle."""
    pkg = os.path.join(ROOT, "draft_token_verification_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                assert "oracle" not in open(os.path.join(dirpath, f)).read().replace("oracle.c", ""), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c")):
            txt = open(os.path.join(ROOT, "oracle", f)).read()
            assert "import draft_token_verification_attention_amd" not in txt
            assert "specverify.h" not in txt and "sv_common" not in txt


def test_static_accept_rejects_calls_beyond_its_scratch():
    """The size check of sv_spec_accept_static runs on the host before any runtime call."""
    d = sv.sv_accept_desc()
    d.mode, d.B, d.gamma, d.V, d.temperature = 1, 4096, 4, 128256, 1.0
    assert sv.lib.sv_spec_accept_workspace(ctypes.byref(d)) > sv.SV_STATIC_SCRATCH_BYTES
    assert sv.lib.sv_spec_accept_static(ctypes.byref(d), None) == sv.SV_ERR_WORKSPACE
    d.B = 64
    assert sv.lib.sv_spec_accept_workspace(ctypes.byref(d)) <= sv.SV_STATIC_SCRATCH_BYTES


def test_struct_layouts_match_the_header(tmp_path):
    """Every descriptor the binding declares has the C header's field offsets and size (a
    small C program built against include/specverify.h prints them)."""
    import shutil
    import subprocess
    if not shutil.which("gcc"):
        pytest.skip("no C compiler")
    structs = {"sv_philox": sv.sv_philox, "sv_attn_desc": sv.sv_attn_desc, "sv_accept_desc": sv.sv_accept_desc,
               "sv_walk_desc": sv.sv_walk_desc, "sv_commit_desc": sv.sv_commit_desc,
               "sv_trunc_desc": sv.sv_trunc_desc, "sv_penalty_desc": sv.sv_penalty_desc}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "specverify.h"', "int main(void) {"]
    for name, cls in structs.items():
        lines.append('printf("%s sizeof %%zu\\n", sizeof(%s));' % (name, name))
        for field, _ in cls._fields_:
            lines.append('printf("%s %s %%zu\\n", offsetof(%s, %s));' % (name, field, name, field))
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        s, f, v = ln.split()
        got[(s, f)] = int(v)
    for name, cls in structs.items():
        assert got[(name, "sizeof")] == ctypes.sizeof(cls), name
        for field, _ in cls._fields_:
            assert got[(name, field)] == getattr(cls, field).offset, (name, field)
