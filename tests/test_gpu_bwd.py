"""GPU parity of the SMA backward (and of the training forward's statistics)
against the fp64 oracle on the same seeded inputs.

Bar: bfloat16 inputs with fp32 accumulation, so every output tensor meets
max|gpu - ref| <= 2e-2 * max|ref| (the gradients are f32 tensors, but the
kernels round their MFMA operands to bf16 as the forward does); the gate
gradient is a scalar and meets |gpu - ref| <= 2e-2 * |ref| (the readout o
it sums is kept in f32 by the training forward, so the cancellation in
Σ dy·o does not amplify a bf16 rounding).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from ssm_state_attention_amd import api, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF = torch.bfloat16


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def assert_parity(gpu, ref, what):
    g = gpu if isinstance(gpu, np.ndarray) else synth.as_f64(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = float(np.max(np.abs(g - ref))) if g.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = 2e-2 * scale
    print(f"{what}: max err {err:.3e} bound {bound:.3e} (max|ref| {scale:.3e})", flush=True)
    assert err <= bound, f"{what}: max err {err:.3e} > bound {bound:.3e}"


def _pn_to_np(t):
    """Library layout [..., P, N] -> oracle layout [..., N, P]."""
    return np.swapaxes(synth.as_f64(t), -1, -2)


def _inputs(seed, B, L, H, G, N, P, S, qscale, mem_std):
    """Prefill token inputs (synth recipe), memories N(0, mem_std²) and an
    upstream gradient dy ~ N(0, 1), all bf16."""
    inp = synth.draw_prefill(seed, B, L, H, G, N, P, io=BF, qscale=qscale)
    inp["dH"] = synth.draw_state(seed + 1, (B, H, L // S, P, N), mem_std, BF)
    inp["dy"] = synth.draw_state(seed + 2, (B, L, H, P), 1.0, BF)
    inp["y_ssd"] = synth.draw_state(seed + 3, (B, L, H, P), 1.0, BF)
    return inp


def _gpu_train(d, gate, S):
    B, L, H, P = d["E"].shape
    y = torch.empty(B, L, H, P, dtype=BF, device=DEV)
    o = torch.empty(B, L, H, P, dtype=torch.float32, device=DEV)
    lse = torch.empty(B, H, L, dtype=torch.float32, device=DEV)
    api.dart_sma_fwd_train(d["Q"], d["E"], d["C"], d["dH"], d["y_ssd"], gate, y, o, lse, S)
    grads = api.dart_sma_bwd(d["Q"], d["E"], d["C"], d["dH"], o, lse, d["dy"], gate, S)
    torch.cuda.synchronize()
    return y, o, lse, grads


@pytest.mark.parametrize("B,L,H,G,N,P,S,qscale,mem_std", [
    (1, 256, 2, 1, 32, 32, 64, 1.0, 0.05),      # heads share a group; 4 chunks
    (2, 384, 4, 2, 64, 64, 128, 30.0, 0.05),    # sharpened softmax
    (1, 768, 3, 3, 128, 64, 256, 1.0, 0.05),    # the layer's N, P, S
    (2, 512, 8, 1, 128, 64, 128, 100.0, 0.02),  # one group of 8 heads, sharpened
    (2, 640, 8, 4, 128, 64, 128, 30.0, 0.05),   # 8 (batch, group) pairs: the XCD-dealt grid; 5 chunks
])
def test_sma_backward(B, L, H, G, N, P, S, qscale, mem_std):
    _need_gpu()
    print(f"sma backward case B{B} L{L} H{H} G{G} N{N} P{P} S{S} qscale{qscale}", flush=True)
    gate = 0.7
    inp = _inputs(11, B, L, H, G, N, P, S, qscale, mem_std)
    d = {k: v.to(DEV) for k, v in inp.items()}
    y, o, lse, gr = _gpu_train(d, gate, S)
    # the training forward's y is the plain forward's, bit for bit
    y_plain = torch.empty_like(y)
    api.dart_sma_fwd(d["Q"], d["E"], d["C"], d["dH"], d["y_ssd"], gate, y_plain, S)
    torch.cuda.synchronize()
    assert torch.equal(y, y_plain)
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    dHo = np.swapaxes(n["dH"], -1, -2)
    o_ref = oracle.sma(n["Q"], n["E"], n["C"], dHo, S)
    lse_ref = oracle.sma_logsumexp(n["Q"], n["E"], n["C"], dHo, S)
    assert_parity(o, o_ref, "o")
    assert_parity(synth.as_f64(lse) * math.log(2.0), lse_ref, "lse")
    _, do, dg = oracle.gated_backward(n["dy"], o_ref, gate)
    dQ, dE, dC, ddH = oracle.sma_backward(n["Q"], n["E"], n["C"], dHo, S, do)
    assert_parity(gr["dQ"], dQ, "dQ")
    assert_parity(gr["dE"], dE, "dE")
    assert_parity(gr["dC"], dC, "dC")
    assert_parity(_pn_to_np(gr["ddH"]), ddH, "ddH")
    dg_gpu = float(gr["dgate"].item())
    print(f"dgate {dg_gpu:.6e} ref {dg:.6e}", flush=True)
    assert abs(dg_gpu - dg) <= 2e-2 * abs(dg)


def test_sma_backward_rejects_unsupported():
    _need_gpu()
    d = {k: v.to(DEV) for k, v in _inputs(12, 1, 64, 1, 1, 32, 32, 32, 1.0, 0.05).items()}
    with pytest.raises(ValueError, match="unsupported"):
        _gpu_train(d, 0.5, 32)  # chunk of 32 tokens: not a whole 64-token tile


def test_sma_backward_full_size_sampled_group():
    """The Mamba-2 ~370M layer shape (batch 4, 32 heads in groups of 8,
    L=8192, S=256, N=128, P=64): the whole backward on the GPU; the oracle
    computes one (batch, group) in full (its 8 heads, so dQ and dC are the
    group sums) and the GPU's tensors for it are compared."""
    _need_gpu()
    B, L, H, G, N, P, S, gate = 4, 8192, 32, 4, 128, 64, 256, 0.5
    inp = _inputs(13, B, L, H, G, N, P, S, 1.0, 0.05)
    d = {k: v.to(DEV) for k, v in inp.items()}
    y, o, lse, gr = _gpu_train(d, gate, S)
    b, g = 2, 1
    hs = slice(g * 8, g * 8 + 8)
    sl = {"Q": inp["Q"][b:b + 1, :, g:g + 1], "C": inp["C"][b:b + 1, :, g:g + 1],
          "E": inp["E"][b:b + 1, :, hs], "dy": inp["dy"][b:b + 1, :, hs],
          "dH": inp["dH"][b:b + 1, hs]}
    n = {k: synth.as_f64(v) for k, v in sl.items()}
    dHo = np.swapaxes(n["dH"], -1, -2)
    o_ref = oracle.sma(n["Q"], n["E"], n["C"], dHo, S)
    assert_parity(o[b:b + 1, :, hs], o_ref, "full-size o (one group)")
    _, do, _ = oracle.gated_backward(n["dy"], o_ref, gate)
    dQ, dE, dC, ddH = oracle.sma_backward(n["Q"], n["E"], n["C"], dHo, S, do)
    assert_parity(gr["dQ"][b:b + 1, :, g:g + 1], dQ, "full-size dQ (one group)")
    assert_parity(gr["dC"][b:b + 1, :, g:g + 1], dC, "full-size dC (one group)")
    assert_parity(gr["dE"][b:b + 1, :, hs], dE, "full-size dE (one group)")
    assert_parity(_pn_to_np(gr["ddH"][b:b + 1, hs]), ddH, "full-size ddH (one group)")
    # the gate gradient over the whole layer, from the GPU's own o (a
    # property: dgate = Σ dy·o, whatever o is)
    prod = synth.as_f64(d["dy"]) * synth.as_f64(o)
    dg_prop, l1 = float(np.sum(prod)), float(np.sum(np.abs(prod)))
    # f32 summation of the 33.5 M products in the kernels' order: within
    # 1e-4 of the sum of their magnitudes
    assert abs(float(gr["dgate"].item()) - dg_prop) <= 1e-4 * l1


# ------------------------------------------------------------ scan backward
def _scan_case(seed, B, L, H, G, N, P, S, with_extra=True):
    inp = synth.draw_prefill(seed, B, L, H, G, N, P, io=BF)
    M = L // S
    extra = {
        "dy": synth.draw_state(seed + 5, (B, L, H, P), 1.0, BF),
        "ddH": synth.draw_state(seed + 6, (B, H, M, P, N), 1.0, torch.float32),
        "dhf": synth.draw_state(seed + 7, (B, H, P, N), 1.0, torch.float32),
        "dCs": synth.draw_state(seed + 8, (B, L, G, N), 1.0, torch.float32),
    }
    return inp, extra


def _oracle_scan(inp, extra, S, with_extra):
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    ddH = np.swapaxes(synth.as_f64(extra["ddH"]), -1, -2) if with_extra else None
    dhf = np.swapaxes(synth.as_f64(extra["dhf"]), -1, -2) if with_extra else None
    ref = oracle.ssd_backward(n["x"], n["dt"], n["A"], n["Bm"], n["C"], S,
                              synth.as_f64(extra["dy"]), ddH, dhf)
    if with_extra:
        ref["dC"] = ref["dC"] + synth.as_f64(extra["dCs"])
    return ref


def _check_scan(gr, ref, what):
    for k in ("dx", "ddt", "dA", "dB", "dC"):
        assert_parity(gr[k], ref[k], f"{what} {k}")
    assert_parity(_pn_to_np(gr["dh0"]), ref["dh0"], f"{what} dh0")


@pytest.mark.parametrize("B,L,H,G,N,P,S,with_extra", [
    (1, 256, 2, 1, 32, 32, 64, True),      # heads share B/C; one key block per chunk
    (2, 384, 4, 2, 64, 64, 128, True),     # two blocks per chunk
    (1, 768, 3, 3, 128, 64, 256, True),    # the layer's N, P, S
    (2, 512, 8, 1, 128, 64, 128, False),   # one group of 8 heads; dy only
])
def test_scan_backward(B, L, H, G, N, P, S, with_extra):
    _need_gpu()
    print(f"scan backward case B{B} L{L} H{H} G{G} N{N} P{P} S{S} extra{with_extra}", flush=True)
    inp, extra = _scan_case(21, B, L, H, G, N, P, S)
    d = {k: v.to(DEV) for k, v in inp.items()}
    e = {k: v.to(DEV) for k, v in extra.items()}
    fwd = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.5, S)
    gr = api.dart_scan_bwd(d["x"], d["dt"], d["A"], d["Bm"], d["C"], fwd["acum"], fwd["H_in"],
                           e["dy"], S, ddH=e["ddH"] if with_extra else None,
                           dh_final=e["dhf"] if with_extra else None,
                           dC_sma=e["dCs"] if with_extra else None)
    torch.cuda.synchronize()
    _check_scan(gr, _oracle_scan(inp, extra, S, with_extra), "scan")


def test_prefill_backward_end_to_end():
    """SMA backward feeding the scan backward (ddH and the SMA part of dC),
    against the oracle's chain: sma_backward, then ssd_backward with the
    SMA's memory gradient."""
    _need_gpu()
    B, L, H, G, N, P, S, gate = 2, 512, 4, 2, 128, 64, 128, 0.7
    inp = synth.draw_prefill(31, B, L, H, G, N, P, io=BF, qscale=30.0)
    dy = synth.draw_state(32, (B, L, H, P), 1.0, BF)
    d = {k: v.to(DEV) for k, v in inp.items()}
    fwd = api.prefill_train(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    gr = api.prefill_backward(fwd, d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"],
                              gate, S, dy.to(DEV))
    torch.cuda.synchronize()
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    dH = oracle.chunk_states(n["x"], n["dt"], n["A"], n["Bm"], S)
    o = oracle.sma(n["Q"], n["E"], n["C"], dH, S)
    _, do, dg = oracle.gated_backward(synth.as_f64(dy), o, gate)
    dQ, dE, dC_s, ddH = oracle.sma_backward(n["Q"], n["E"], n["C"], dH, S, do)
    ref = oracle.ssd_backward(n["x"], n["dt"], n["A"], n["Bm"], n["C"], S, synth.as_f64(dy), ddH)
    ref["dC"] = ref["dC"] + dC_s
    for k in ("dx", "ddt", "dA", "dB", "dC"):
        assert_parity(gr[k], ref[k], f"end-to-end {k}")
    assert_parity(gr["dQ"], dQ, "end-to-end dQ")
    assert_parity(gr["dE"], dE, "end-to-end dE")
    assert abs(float(gr["dgate"].item()) - dg) <= 2e-2 * abs(dg)


def test_scan_backward_full_size_sampled_group():
    """The ~370M layer shape: the whole scan backward on the GPU; one
    (batch, group) (8 heads, so dB and dC are complete group sums) against
    the oracle; dA sums over the batch and is checked at the small shapes."""
    _need_gpu()
    B, L, H, G, N, P, S = 4, 8192, 32, 4, 128, 64, 256
    inp, extra = _scan_case(41, B, L, H, G, N, P, S)
    d = {k: v.to(DEV) for k, v in inp.items()}
    e = {k: v.to(DEV) for k, v in extra.items()}
    fwd = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.5, S)
    gr = api.dart_scan_bwd(d["x"], d["dt"], d["A"], d["Bm"], d["C"], fwd["acum"], fwd["H_in"],
                           e["dy"], S, ddH=e["ddH"], dh_final=e["dhf"], dC_sma=e["dCs"])
    torch.cuda.synchronize()
    b, g = 1, 3
    hs = slice(g * 8, g * 8 + 8)
    sl = {"x": inp["x"][b:b + 1, :, hs], "dt": inp["dt"][b:b + 1, :, hs], "A": inp["A"][hs],
          "Bm": inp["Bm"][b:b + 1, :, g:g + 1], "C": inp["C"][b:b + 1, :, g:g + 1]}
    ex = {"dy": extra["dy"][b:b + 1, :, hs], "ddH": extra["ddH"][b:b + 1, hs],
          "dhf": extra["dhf"][b:b + 1, hs], "dCs": extra["dCs"][b:b + 1, :, g:g + 1]}
    ref = _oracle_scan(sl, ex, S, True)
    assert_parity(gr["dx"][b:b + 1, :, hs], ref["dx"], "full-size dx (one group)")
    assert_parity(gr["ddt"][b:b + 1, :, hs], ref["ddt"], "full-size ddt (one group)")
    assert_parity(gr["dB"][b:b + 1, :, g:g + 1], ref["dB"], "full-size dB (one group)")
    assert_parity(gr["dC"][b:b + 1, :, g:g + 1], ref["dC"], "full-size dC (one group)")
    assert_parity(_pn_to_np(gr["dh0"][b:b + 1, hs]), ref["dh0"], "full-size dh0 (one group)")


def test_backward_single_chunk():
    """One chunk: no memory is visible, so every SMA gradient and dgate are
    zero and the scan backward is the intra-chunk term plus the state
    gradients of one chunk."""
    _need_gpu()
    B, L, H, G, N, P, S, gate = 2, 128, 2, 1, 64, 64, 128, 0.5
    inp = synth.draw_prefill(51, B, L, H, G, N, P, io=BF)
    dy = synth.draw_state(52, (B, L, H, P), 1.0, BF)
    dhf = synth.draw_state(53, (B, H, P, N), 1.0, torch.float32)
    d = {k: v.to(DEV) for k, v in inp.items()}
    fwd = api.prefill_train(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    gr = api.prefill_backward(fwd, d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"],
                              gate, S, dy.to(DEV), dh_final=dhf.to(DEV))
    torch.cuda.synchronize()
    assert float(gr["dgate"].item()) == 0.0
    assert not bool(gr["dQ"].any()) and not bool(gr["dE"].any())
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    ref = oracle.ssd_backward(n["x"], n["dt"], n["A"], n["Bm"], n["C"], S, synth.as_f64(dy),
                              None, np.swapaxes(synth.as_f64(dhf), -1, -2))
    for k in ("dx", "ddt", "dA", "dB", "dC"):
        assert_parity(gr[k], ref[k], f"single chunk {k}")
    assert_parity(_pn_to_np(gr["dh0"]), ref["dh0"], "single chunk dh0")


# ------------------------------------------------------------ f32 io
# The f32 backward runs plain f32 kernels (every compiled f32 shape, any chunk
# size).  Bar: max|gpu - ref| <= 1e-4 · max(1, max|ref|) per tensor: the fp32
# bar of 1e-4 absolute, relative to the tensor's scale where gradients that
# sum many products exceed 1.
F32 = torch.float32


def assert_parity_f32(gpu, ref, what):
    g = gpu if isinstance(gpu, np.ndarray) else synth.as_f64(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = float(np.max(np.abs(g - ref))) if g.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = 1e-4 * max(1.0, scale)
    print(f"{what}: max err {err:.3e} bound {bound:.3e} (max|ref| {scale:.3e})", flush=True)
    assert err <= bound, f"{what}: max err {err:.3e} > bound {bound:.3e}"


@pytest.mark.parametrize("B,L,H,G,N,P,S,qscale,mem_std", [
    (1, 1024, 1, 1, 16, 16, 64, 1.0, 0.05),     # the tiny fp32 layer's shape (16 chunks)
    (2, 288, 3, 3, 32, 32, 96, 30.0, 0.05),     # S = 96, sharpened
    (1, 256, 4, 2, 32, 32, 32, 100.0, 0.05),    # 32-token chunks, heads sharing a group
    (2, 64, 2, 1, 16, 16, 64, 1.0, 0.05),       # one chunk: no memory visible, zero gradients
])
def test_sma_backward_f32(B, L, H, G, N, P, S, qscale, mem_std):
    _need_gpu()
    print(f"f32 sma backward case B{B} L{L} H{H} G{G} N{N} P{P} S{S} qscale{qscale}", flush=True)
    gate = 0.7
    inp = synth.draw_prefill(14, B, L, H, G, N, P, io=F32, qscale=qscale)
    inp["dH"] = synth.draw_state(15, (B, H, L // S, P, N), mem_std, F32)
    inp["dy"] = synth.draw_state(16, (B, L, H, P), 1.0, F32)
    inp["y_ssd"] = synth.draw_state(17, (B, L, H, P), 1.0, F32)
    d = {k: v.to(DEV) for k, v in inp.items()}
    y = torch.empty(B, L, H, P, dtype=F32, device=DEV)
    o = torch.empty(B, L, H, P, dtype=F32, device=DEV)
    lse = torch.empty(B, H, L, dtype=F32, device=DEV)
    api.dart_sma_fwd_train(d["Q"], d["E"], d["C"], d["dH"], d["y_ssd"], gate, y, o, lse, S)
    gr = api.dart_sma_bwd(d["Q"], d["E"], d["C"], d["dH"], o, lse, d["dy"], gate, S)
    torch.cuda.synchronize()
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    dHo = np.swapaxes(n["dH"], -1, -2)
    o_ref = oracle.sma(n["Q"], n["E"], n["C"], dHo, S)
    assert_parity_f32(o, o_ref, "o")
    _, do, dg = oracle.gated_backward(n["dy"], o_ref, gate)
    dQ, dE, dC, ddH = oracle.sma_backward(n["Q"], n["E"], n["C"], dHo, S, do)
    assert_parity_f32(gr["dQ"], dQ, "dQ")
    assert_parity_f32(gr["dE"], dE, "dE")
    assert_parity_f32(gr["dC"], dC, "dC")
    assert_parity_f32(_pn_to_np(gr["ddH"]), ddH, "ddH")
    dg_gpu = float(gr["dgate"].item())
    print(f"dgate {dg_gpu:.6e} ref {dg:.6e}", flush=True)
    assert abs(dg_gpu - dg) <= 1e-4 * max(1.0, abs(dg))


@pytest.mark.parametrize("B,L,H,G,N,P,S,with_extra", [
    (1, 1024, 1, 1, 16, 16, 64, True),     # the tiny fp32 layer's shape
    (2, 288, 3, 3, 32, 32, 96, True),      # S = 96
    (1, 256, 4, 2, 32, 32, 32, False),     # 32-token chunks, shared B/C; dy only
    (1, 512, 2, 1, 16, 16, 256, True),     # 256-token chunks
    (2, 64, 2, 2, 32, 32, 64, True),       # one chunk
])
def test_scan_backward_f32(B, L, H, G, N, P, S, with_extra):
    _need_gpu()
    print(f"f32 scan backward case B{B} L{L} H{H} G{G} N{N} P{P} S{S} extra{with_extra}",
          flush=True)
    inp = synth.draw_prefill(22, B, L, H, G, N, P, io=F32)
    M = L // S
    extra = {"dy": synth.draw_state(23, (B, L, H, P), 1.0, F32),
             "ddH": synth.draw_state(24, (B, H, M, P, N), 1.0, F32),
             "dhf": synth.draw_state(25, (B, H, P, N), 1.0, F32),
             "dCs": synth.draw_state(26, (B, L, G, N), 1.0, F32)}
    d = {k: v.to(DEV) for k, v in inp.items()}
    e = {k: v.to(DEV) for k, v in extra.items()}
    fwd = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.5, S)
    gr = api.dart_scan_bwd(d["x"], d["dt"], d["A"], d["Bm"], d["C"], fwd["acum"], fwd["H_in"],
                           e["dy"], S, ddH=e["ddH"] if with_extra else None,
                           dh_final=e["dhf"] if with_extra else None,
                           dC_sma=e["dCs"] if with_extra else None)
    torch.cuda.synchronize()
    ref = _oracle_scan(inp, extra, S, with_extra)
    for k in ("dx", "ddt", "dA", "dB", "dC"):
        assert_parity_f32(gr[k], ref[k], f"f32 scan {k}")
    assert_parity_f32(_pn_to_np(gr["dh0"]), ref["dh0"], "f32 scan dh0")


def test_prefill_backward_end_to_end_f32():
    """The tiny fp32 layer (batch 1, 1 head, L=1024, S=64, N=P=16): the
    whole prefill backward (SMA feeding the scan) against the oracle's
    chain."""
    _need_gpu()
    B, L, H, G, N, P, S, gate = 1, 1024, 1, 1, 16, 16, 64, 0.5
    inp = synth.draw_prefill(0, B, L, H, G, N, P, io=F32)
    dy = synth.draw_state(33, (B, L, H, P), 1.0, F32)
    d = {k: v.to(DEV) for k, v in inp.items()}
    fwd = api.prefill_train(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    gr = api.prefill_backward(fwd, d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"],
                              gate, S, dy.to(DEV))
    torch.cuda.synchronize()
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    dH = oracle.chunk_states(n["x"], n["dt"], n["A"], n["Bm"], S)
    o = oracle.sma(n["Q"], n["E"], n["C"], dH, S)
    _, do, dg = oracle.gated_backward(synth.as_f64(dy), o, gate)
    dQ, dE, dC_s, ddH = oracle.sma_backward(n["Q"], n["E"], n["C"], dH, S, do)
    ref = oracle.ssd_backward(n["x"], n["dt"], n["A"], n["Bm"], n["C"], S, synth.as_f64(dy), ddH)
    ref["dC"] = ref["dC"] + dC_s
    for k in ("dx", "ddt", "dA", "dB", "dC"):
        assert_parity_f32(gr[k], ref[k], f"f32 end-to-end {k}")
    assert_parity_f32(gr["dQ"], dQ, "f32 end-to-end dQ")
    assert_parity_f32(gr["dE"], dE, "f32 end-to-end dE")
    assert abs(float(gr["dgate"].item()) - dg) <= 1e-4 * max(1.0, abs(dg))
