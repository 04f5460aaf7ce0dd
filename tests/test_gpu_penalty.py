"""GPU parity of sv_penalize (repetition, frequency, presence; drafted prefix as context)
against oracle.penalize: bit-exact rows (both sides evaluate the same fp64 expression and
round once).  Cases: vocabularies up to 128256, histories from empty to 20000 entries (both
ways of counting: in LDS up to 8192 entries, in a vocabulary-sized array beyond) with repeats
and out-of-range entries, per-sequence history lengths (0, clamped,
negative), drafts from none to 64, one workspace across calls (left zero), bad arguments,
and the whole processed round: penalties, top-k / top-p, then the acceptance, against the
oracle's same three steps.
"""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import draft_token_verification_attention_amd as sv  # noqa: E402
from svgpu import dev_array, to_host  # noqa: E402
from test_gpu_accept import _assert_parity, near_threshold_limit  # noqa: E402


def _inputs(seed, B, n, V, H, g, spread=None):
    lg = synth.logit_rows(seed, B * n, V, 4.0).reshape(B, n, V)
    r = np.random.default_rng(seed)
    hist = r.integers(-2, V + 2, (B, H)).astype(np.int32) if H else None
    if H:
        k = min(H, 50)
        hist[:, :k] = r.integers(0, min(V, spread or 20), (B, k))    # repeats
    drafts = r.integers(0, min(V, 30), (B, g)).astype(np.int32) if g else None
    return lg, hist, drafts


def _gpu(lg, hist, drafts, hist_len=None, **pen):
    x = dev_array(lg)
    sv.sv_penalize(x, history=None if hist is None else dev_array(hist),
                   hist_len=None if hist_len is None else dev_array(hist_len),
                   draft_tokens=None if drafts is None else dev_array(drafts), **pen)
    torch.cuda.synchronize()
    return x.cpu().numpy()


PENS = [dict(repetition=1.3), dict(repetition=1.0, frequency=0.4, presence=0.3),
        dict(repetition=0.7, frequency=-0.25, presence=1.5), dict(repetition=1.2, frequency=0.1, presence=0.2)]


@pytest.mark.parametrize("V,B,H,g", [(7, 8, 12, 4), (1000, 16, 300, 5), (32000, 8, 2500, 4), (128256, 4, 5000, 16),
                                     (128256, 2, 0, 64), (5000, 4, 1024, 0), (5000, 4, 1025, 1),
                                     (32000, 3, 8192, 4), (32000, 3, 8193, 4), (128256, 2, 20000, 8)])
def test_penalize_parity(V, B, H, g):
    n = g + 1 if g else 3
    lg, hist, drafts = _inputs(V + H + g, B, n, V, H, g)
    for pen in PENS:
        ref = oracle.penalize(lg, history=hist, drafts=drafts, **pen)
        got = _gpu(lg, hist, drafts, **pen)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), pen


def test_history_lengths_and_draft_rows():
    V, B, g = 2000, 6, 4
    lg, hist, drafts = _inputs(5, B, g, V, 1500, g)
    hl = np.array([0, 1500, 9999, -3, 700, 1024], np.int32)
    pen = dict(repetition=1.25, frequency=0.3, presence=0.15)
    ref = oracle.penalize(lg, history=hist, hist_len=hl, drafts=drafts, **pen)
    got = _gpu(lg, hist, drafts, hist_len=hl, **pen)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_one_workspace_across_calls():
    """The workspace contract: whatever lies after the counter region (other entry points
    leave partial results there; here, garbage written before every call) does not change
    the result, and the counter region reads zero after each call.  Calls of other shapes
    share one explicit workspace."""
    import ctypes
    pen = dict(repetition=1.4, frequency=0.2, presence=0.1)
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device="cuda")
    for seed, B, V, H in [(1, 5, 4000, 800), (2, 5, 4000, 3000), (3, 3, 9000, 2500), (4, 7, 1500, 0),
                          (5, 2, 20000, 5000), (6, 5, 4000, 2048), (7, 2, 30000, 9000), (8, 4, 4000, 1200)]:
        ws[128 * 1024:].random_(0, 256)
        lg, hist, drafts = _inputs(seed, B, 4, V, H, 3, spread=V)
        ref = oracle.penalize(lg, history=hist, drafts=drafts, **pen)
        x = dev_array(lg)
        h = None if hist is None else dev_array(hist)
        d = sv.penalty_desc(x, history=h, draft_tokens=dev_array(drafts), **pen)
        nb = sv.lib.sv_penalize_workspace(ctypes.byref(d))
        assert 0 < nb <= ws.numel()
        st = sv.lib.sv_penalize(ctypes.byref(d), ctypes.c_void_p(ws.data_ptr()), nb,
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0
        torch.cuda.synchronize()
        assert np.array_equal(x.cpu().numpy().view(np.uint32), ref.view(np.uint32)), seed
        assert int(torch.count_nonzero(ws[:128 * 1024]).item()) == 0, seed


def test_off_and_empty():
    lg, hist, drafts = _inputs(6, 3, 4, 500, 100, 3)
    assert np.array_equal(_gpu(lg, hist, drafts), lg)
    x = torch.zeros((0, 4, 10), dtype=torch.float32, device="cuda")
    sv.sv_penalize(x, repetition=1.5)


def test_bad_arguments():
    x = dev_array(synth.logit_rows(7, 4, 10, 1.0).reshape(2, 2, 10))
    for kw in (dict(repetition=0.0), dict(repetition=-1.0), dict(repetition=float("nan")),
               dict(repetition=float("inf")), dict(frequency=float("inf")), dict(presence=float("nan"))):
        with pytest.raises(sv.SpecVerifyError):
            sv.sv_penalize(x, **kw)
    with pytest.raises(sv.SpecVerifyError):   # more than 64 drafts
        sv.sv_penalize(x, draft_tokens=torch.zeros((2, 65), dtype=torch.int32, device="cuda"), repetition=1.2)


@pytest.mark.parametrize("V,B,g", [(1000, 96, 4), (32000, 24, 5)])
def test_processed_round(V, B, g):
    """Penalties (history and drafted prefix), then top-k / top-p, then the round, on both
    models' rows, on the GPU, equal the oracle's same three steps.  Drafts come from the
    drafter's processed rows."""
    T, k, p = 0.9, 60, 0.92
    pen = dict(repetition=1.3, frequency=0.2, presence=0.4)
    a = synth.accept_inputs(V + 5, B=B, gamma=g, V=V, target_var=3.0, noise_var=1.0, tau=T)
    hist = np.random.default_rng(V).integers(0, 200, (B, 64)).astype(np.int32)
    # drafts: the drafter's own sequential processed sampling (its row i sees x_0..x_{i-1})
    u = np.clip(synth.rng(V, "misc").random(size=(B, g, V)), 1e-300, 1.0 - 1e-16)
    toks = np.zeros((B, g), np.int32)
    for i in range(g):
        row = oracle.penalize(a["draft"][:, i:i + 1], history=np.concatenate([hist, toks[:, :i]], axis=1), **pen)
        row = oracle.truncate(row, T, top_k=k, top_p=p)["out"]
        toks[:, i] = synth.gumbel_draw(row[:, 0], T, u[:, i])
    tp = oracle.truncate(oracle.penalize(a["target"], history=hist, drafts=toks, **pen), T, top_k=k, top_p=p)
    dq = oracle.truncate(oracle.penalize(a["draft"], history=hist, drafts=toks, **pen), T, top_k=k, top_p=p)
    ref = oracle.spec_accept(oracle.SAMPLE, tp["out"], dq["out"], toks, T, seed=9, step=0)
    near = (tp["flags"].reshape(B, g + 1) != 0).any(axis=1) | (dq["flags"].reshape(B, g) != 0).any(axis=1)
    assert near.sum() <= near_threshold_limit(B * (2 * g + 1))

    tgt, dft = dev_array(a["target"]), dev_array(a["draft"])
    h, x = dev_array(hist), dev_array(toks)
    for rows in (tgt, dft):
        sv.sv_penalize(rows, history=h, draft_tokens=x, **pen)
        sv.sv_truncate(rows, temperature=T, top_k=k, top_p=p, in_place=True)
    got = to_host(sv.sv_spec_accept(oracle.SAMPLE, tgt, dft, x, T, 9, 0))
    keep = ~near
    _assert_parity({kk: v[keep] for kk, v in ref.items() if v is not None},
                   {kk: v[keep] for kk, v in got.items() if v is not None}, "processed V=%d" % V)


def test_full_batch_of_the_batched_chain():
    """The batched chain's rows at full size (64 sequences, 320 target and 256 draft rows of
    128256 logits) with a 4096-token history per sequence, as bench.py times them."""
    cfg = synth.WORKLOADS[4]
    a = synth.accept_inputs(4, B=cfg["B"], gamma=cfg["gamma"], V=cfg["V"], target_var=cfg["target_var"],
                            noise_var=cfg["noise_var"], tau=cfg["tau"])
    hist = np.random.default_rng(17).integers(0, cfg["V"], (cfg["B"], 4096)).astype(np.int32)
    pen = dict(repetition=1.2, frequency=0.3, presence=0.2)
    for name in ("target", "draft"):
        ref = oracle.penalize(a[name], history=hist, drafts=a["draft_tokens"], **pen)
        got = _gpu(a[name], hist, a["draft_tokens"], **pen)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), name
