"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Bar: fp32 max|gpu - ref| <= 1e-4; bfloat16 (fp32 accumulate)
max|gpu - ref| <= 2e-2 * max|ref|, per output tensor.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from ssm_state_attention_amd import api, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def assert_parity(gpu, ref, io, what):
    g = gpu if isinstance(gpu, np.ndarray) else synth.as_f64(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = float(np.max(np.abs(g - ref))) if g.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    bound = 1e-4 if io == torch.float32 else 2e-2 * scale
    print(f"{what}: max err {err:.3e} bound {bound:.3e} (max|ref| {scale:.3e})", flush=True)
    assert err <= bound, f"{what}: max err {err:.3e} > bound {bound:.3e}"


def _np(d):
    return {k: synth.as_f64(v) for k, v in d.items()}


def _to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def _pn_to_np(t):
    """Library state layout [..., P, N] -> oracle layout [..., N, P]."""
    return np.swapaxes(synth.as_f64(t), -1, -2)


def run_prefill_case(B, L, H, G, N, P, S, io, seed=0, gate=0.5, qscale=1.0, h0_std=0.0,
                     decayed=False):
    _need_gpu()
    print(f"prefill case B{B} L{L} H{H} G{G} N{N} P{P} S{S} {io} seed{seed} "
          f"qscale{qscale} h0_std{h0_std} decayed{decayed}", flush=True)
    inp = synth.draw_prefill(seed, B, L, H, G, N, P, io=io, qscale=qscale)
    h0 = None
    if h0_std:
        h0 = synth.draw_state(seed + 1, (B, H, P, N), h0_std, torch.float32)
    d = _to_dev(inp)
    out = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S,
                      h0=None if h0 is None else h0.to(DEV), decayed=decayed)
    torch.cuda.synchronize()
    n = _np(inp)
    ref = oracle.prefill(n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"], n["E"], gate, S,
                         h0=None if h0 is None else _pn_to_np(h0), decayed=decayed)
    assert_parity(_pn_to_np(out["dH_f32"]), ref["dH"], io, "dH_f32")
    assert_parity(_pn_to_np(out["dH"]), ref["dH"], io, "dH")
    assert_parity(_pn_to_np(out["H_in"]), ref["H_in"][:, :, :-1], io, "H_in")
    assert_parity(_pn_to_np(out["h_final"]), ref["h_final"], io, "h_final")
    assert_parity(out["y_ssd"], ref["y_ssd"], io, "y_ssd")
    assert_parity(out["y"], ref["y"], io, "y")
    # the SMA branch alone, so that a wrong readout cannot hide under y_ssd
    o_gpu = (synth.as_f64(out["y"]) - synth.as_f64(out["y_ssd"])) / gate
    if io == torch.float32:
        assert_parity(o_gpu, ref["o"], io, "o")
    return out, ref


def test_config0_fp32_tiny_layer():
    """Tiny DART layer fp32: batch 1, 1 head, L=1024, S=64, N=16, P=16, g=0.5, seed 0."""
    run_prefill_case(1, 1024, 1, 1, 16, 16, 64, torch.float32)


def test_config1_bf16_prefill():
    """Prefill bf16: batch 1, 8 heads, L=4096, S=256, N=128, P=64."""
    run_prefill_case(1, 4096, 8, 8, 128, 64, 256, torch.bfloat16)


@pytest.mark.parametrize("B,L,H,G,N,P,S,io", [
    (1, 32, 1, 1, 32, 32, 32, torch.bfloat16),        # M = 1: SMA output is zero
    (2, 64, 3, 1, 32, 32, 32, torch.bfloat16),        # M = 2, B·H not a multiple of 8
    (3, 96, 5, 5, 64, 64, 32, torch.bfloat16),        # ragged pair count, 1-wave tiles
    (1, 384, 4, 2, 64, 64, 128, torch.bfloat16),      # 4-wave tiles, grouped B/C/Q
    (2, 512, 2, 2, 128, 128, 256, torch.bfloat16),    # largest shape, one token block/wave
    (1, 768, 3, 3, 128, 64, 256, torch.bfloat16),     # M = 3
    (2, 288, 3, 3, 32, 32, 96, torch.float32),        # S not a power of two, M = 3
    (1, 384, 2, 2, 64, 64, 96, torch.bfloat16),       # S = 96 (three 1-wave tiles), M = 4
    (1, 320, 2, 1, 16, 16, 32, torch.float32),
    (1, 768, 6, 2, 128, 64, 256, torch.bfloat16),     # 3 heads per group: the chunk output's
    (1, 768, 10, 2, 64, 64, 256, torch.bfloat16),     # ring of 3 head slots wraps (5 heads, N=64)
])
def test_prefill_shapes(B, L, H, G, N, P, S, io):
    run_prefill_case(B, L, H, G, N, P, S, io, seed=B * 100 + L + H)


@pytest.mark.parametrize("B,L,H,G,N,P,S,io,qscale", [
    (2, 288, 3, 3, 32, 32, 96, torch.float32, 1e2),   # S = 96, M = 3
    (1, 384, 2, 2, 64, 64, 96, torch.bfloat16, 1e3),  # S = 96, M = 4, 1-wave tiles
])
def test_prefill_sharpened_chunk96(B, L, H, G, N, P, S, io, qscale):
    """Chunks of 96 tokens (not a power of two) with memories visible and a
    sharpened softmax: the SMA readout o alone against the oracle."""
    out, ref = run_prefill_case(B, L, H, G, N, P, S, io, seed=5 + L, qscale=qscale, gate=1.0)
    o_gpu = synth.as_f64(out["y"]) - synth.as_f64(out["y_ssd"])
    assert_parity(o_gpu, ref["o"], io, "o (sharpened, S=96)")


@pytest.mark.parametrize("qscale", [1e2, 1e4])
def test_prefill_sharpened_grouped_xcd_mapping(qscale):
    """Batch x groups a multiple of 8 with several heads per group: the SMA
    launch places the heads of one (batch, group) side by side on one XCD
    (the mapping the ~370M-layer benchmark shape uses).  Sharpened scores
    make the readout o sensitive to the score path; o is checked alone."""
    out, ref = run_prefill_case(2, 2048, 16, 4, 128, 64, 256, torch.bfloat16, seed=13,
                                qscale=qscale, gate=1.0)
    o_gpu = synth.as_f64(out["y"]) - synth.as_f64(out["y_ssd"])
    assert_parity(o_gpu, ref["o"], torch.bfloat16, "o (sharpened, grouped XCD mapping)")


@pytest.mark.parametrize("io,N,P,S", [(torch.bfloat16, 128, 64, 256), (torch.float32, 16, 16, 64),
                                      (torch.bfloat16, 64, 64, 64)])
def test_prefill_large_decay(io, N, P, S):
    """Per-token decays dt·|A| of 8 to 16 (far outside the synthetic recipe):
    inside a 16-token block the log-decay spans more than 2^7, so the
    intra-chunk weights must be formed without factors that overflow."""
    _need_gpu()
    B, H, G, L = 1, 4, 2, 4 * S
    inp = synth.draw_prefill(17, B, L, H, G, N, P, io=io, qscale=10.0)
    rng = np.random.default_rng(18)
    inp["dt"] = torch.from_numpy(rng.uniform(0.5, 1.0, (B, L, H))).to(torch.float32)
    inp["A"] = torch.full((H,), -16.0, dtype=torch.float32)
    d = _to_dev(inp)
    gate = 0.5
    out = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    torch.cuda.synchronize()
    n = _np(inp)
    ref = oracle.prefill(n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"], n["E"], gate, S)
    assert_parity(_pn_to_np(out["dH_f32"]), ref["dH"], io, "dH_f32 (large decay)")
    assert_parity(_pn_to_np(out["h_final"]), ref["h_final"], io, "h_final (large decay)")
    assert_parity(out["y_ssd"], ref["y_ssd"], io, "y_ssd (large decay)")
    assert_parity(out["y"], ref["y"], io, "y (large decay)")


@pytest.mark.parametrize("qscale", [1e2, 1e4])
def test_prefill_sharpened_softmax(qscale):
    """Scaled queries make the softmax nearly one-hot, so a wrong score
    (scale, key axis, index) moves y far beyond the tolerance."""
    out, ref = run_prefill_case(2, 1024, 4, 2, 128, 64, 256, torch.bfloat16, seed=7,
                                qscale=qscale, gate=1.0)
    o_gpu = synth.as_f64(out["y"]) - synth.as_f64(out["y_ssd"])
    assert_parity(o_gpu, ref["o"], torch.bfloat16, "o (sharpened)")


@pytest.mark.parametrize("B,L,H,G,N,P,S,io,qscale", [
    (1, 768, 3, 3, 128, 64, 256, torch.bfloat16, 1.0),   # M = 3, 8-wave tiles
    (2, 512, 2, 2, 128, 128, 256, torch.bfloat16, 1.0),  # one token block per wave
    (1, 384, 4, 2, 64, 64, 128, torch.bfloat16, 1e2),    # sharpened, grouped B/C/Q
    (2, 64, 3, 1, 32, 32, 32, torch.bfloat16, 1.0),      # M = 2
    (2, 288, 3, 3, 32, 32, 96, torch.float32, 1e2),      # S not a power of two, M = 3
    (1, 320, 2, 1, 16, 16, 32, torch.float32, 1.0),      # M = 10: old memories decay to ~0
])
def test_prefill_decayed(B, L, H, G, N, P, S, io, qscale):
    """The decay-included SMA variant (dart_sma_fwd_decayed) against the
    oracle's sma_decayed, through the whole prefill."""
    out, ref = run_prefill_case(B, L, H, G, N, P, S, io, seed=7 + L, qscale=qscale,
                                decayed=True)
    assert out["y"].isfinite().all()


def test_prefill_sharpened_fp32():
    run_prefill_case(1, 256, 2, 1, 32, 32, 32, torch.float32, seed=8, qscale=1e3)


def test_prefill_with_initial_state():
    run_prefill_case(2, 512, 4, 4, 64, 64, 128, torch.bfloat16, seed=9, h0_std=0.05)
    run_prefill_case(1, 256, 1, 1, 16, 16, 64, torch.float32, seed=10, h0_std=0.5)


def test_gate_zero_returns_ssm_output():
    """g = 0 removes the SMA branch: y equals y_ssd rounded to the io type."""
    _need_gpu()
    inp = _to_dev(synth.draw_prefill(11, 1, 1024, 4, 4, 128, 64, io=torch.bfloat16))
    out = api.prefill(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["C"], inp["Q"], inp["E"],
                      0.0, 256)
    torch.cuda.synchronize()
    assert torch.equal(out["y"], out["y_ssd"].to(torch.bfloat16))


def test_memories_rounded_from_f32():
    """The io-typed memories are the f32 memories rounded to nearest even."""
    _need_gpu()
    inp = _to_dev(synth.draw_prefill(12, 1, 512, 2, 2, 128, 64, io=torch.bfloat16))
    out = api.prefill(inp["x"], inp["dt"], inp["A"], inp["Bm"], inp["C"], inp["Q"], inp["E"],
                      0.5, 256)
    torch.cuda.synchronize()
    assert torch.equal(out["dH"], out["dH_f32"].to(torch.bfloat16))


# ------------------------------------------------------------------ decode
def _decode_case(B, H, G, N, P, S, max_chunks, n_chunks, pos, io, seed, gate=0.5, qscale=1.0):
    _need_gpu()
    print(f"decode case B{B} H{H} G{G} N{N} P{P} S{S} max{max_chunks} n{n_chunks} pos{pos} "
          f"{io} seed{seed}", flush=True)
    st = api.new_decode_state(B, H, G, N, P, S, max_chunks, io, DEV)
    st["cache"].copy_(synth.draw_state(seed, (B, H, max_chunks, P, N), 0.01, io))
    st["h"].copy_(synth.draw_state(seed + 1, (B, H, P, N), 0.01, torch.float32))
    st["dH_cur"].copy_(synth.draw_state(seed + 2, (B, H, P, N), 0.01, torch.float32))
    st["n_chunks"].copy_(torch.tensor(n_chunks, dtype=torch.int32))
    st["pos"].copy_(torch.tensor(pos, dtype=torch.int32))
    ostate = {"cache": _pn_to_np(st["cache"]), "h": _pn_to_np(st["h"]),
              "dH_cur": _pn_to_np(st["dH_cur"]), "n_chunks": np.array(n_chunks),
              "pos": np.array(pos)}
    tok = synth.draw_decode_token(seed + 3, B, H, G, N, P, io=io, qscale=qscale)
    d = _to_dev(tok)
    y = api.decode_step(st, d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate)
    torch.cuda.synchronize()
    n = _np(tok)
    y_ref, new = oracle.decode_step(ostate, n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"],
                                    n["E"], gate, S, cache_bf16=io == torch.bfloat16)
    assert_parity(y, y_ref, io, "decode y")
    if qscale != 1.0:
        # the SMA readout alone: y - C·h over the updated state, against the
        # oracle's readout (its y at gate g minus its y at gate 0, over g)
        y0_ref, _ = oracle.decode_step(ostate, n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"],
                                       n["E"], 0.0, S, cache_bf16=io == torch.bfloat16)
        Ch = n["C"][:, oracle.group_of_head(H, G)]
        y_ssd_gpu = np.einsum("bhn,bhnp->bhp", Ch, _pn_to_np(st["h"]))
        assert_parity((synth.as_f64(y) - y_ssd_gpu) / gate, (y_ref - y0_ref) / gate, io,
                      "decode o (sharpened)")
    assert_parity(_pn_to_np(st["h"]), new["h"], io, "decode h")
    assert_parity(_pn_to_np(st["dH_cur"]), new["dH_cur"], io, "decode dH_cur")
    assert_parity(_pn_to_np(st["cache"]), new["cache"], io, "decode cache")
    assert st["n_chunks"].cpu().tolist() == list(new["n_chunks"])
    assert st["pos"].cpu().tolist() == list(new["pos"])
    return st


@pytest.mark.parametrize("io,N,P", [(torch.bfloat16, 128, 64), (torch.bfloat16, 64, 64),
                                    (torch.bfloat16, 128, 128), (torch.float32, 16, 16),
                                    (torch.float32, 32, 32)])
def test_decode_small(io, N, P):
    """Few (sequence, head) pairs: the chunk range is split across
    workgroups and merged by the combine kernel; one sequence closes its
    chunk (append), one starts from an empty cache."""
    _decode_case(3, 4, 2, N, P, 64, 12, [5, 0, 11], [63, 0, 17], io, seed=20)


def test_decode_sharpened():
    _decode_case(2, 4, 4, 128, 64, 256, 16, [16, 9], [3, 255], torch.bfloat16, seed=21,
                 qscale=1e4)


@pytest.mark.parametrize("qscale", [1.0, 1e4])
def test_decode_many_pairs_single_split(qscale):
    """Enough pairs that each workgroup streams its whole cache (no combine);
    with sharpened scores the readout is checked alone."""
    _decode_case(32, 32, 32, 128, 64, 256, 8, list(range(1, 9)) * 4, [255, 0] * 16,
                 torch.bfloat16, seed=22, qscale=qscale, gate=1.0 if qscale != 1.0 else 0.5)


def test_decode_cache_full_sets_flag():
    """Closing a chunk with a full cache appends nothing, raises the
    workspace flag and saturates n_chunks; nothing is written out of bounds."""
    _need_gpu()
    B, H, N, P, S, mx = 2, 2, 64, 64, 32, 3
    st = api.new_decode_state(B, H, H, N, P, S, mx, torch.bfloat16, DEV)
    st["cache"].copy_(synth.draw_state(30, (B, H, mx, P, N), 0.01, torch.bfloat16))
    before = st["cache"].clone()
    st["n_chunks"].fill_(mx)
    st["pos"].fill_(S - 1)
    d = _to_dev(synth.draw_decode_token(31, B, H, H, N, P, io=torch.bfloat16))
    assert not api.cache_overflowed(st)
    with pytest.raises(RuntimeError, match="decode cache full"):
        api.decode_step(st, d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.5,
                        check_overflow=True)
    torch.cuda.synchronize()
    assert torch.equal(st["cache"], before)
    assert int(st["workspace"][:4].view(torch.int32).item()) == 1
    assert api.cache_overflowed(st)
    assert st["n_chunks"].tolist() == [mx] * B and st["pos"].tolist() == [0] * B


@pytest.mark.parametrize("io,N,P,S,cap", [(torch.bfloat16, 128, 64, 64, 3),
                                           (torch.bfloat16, 128, 64, 64, 16),
                                           (torch.float32, 16, 16, 32, 3)])
def test_decode_continues_prefill(io, N, P, S, cap):
    """Prefill k chunks, then decode the next chunk token by token: decode
    outputs match the prefill of the longer sequence, and the appended
    memory matches the prefill's memory (GPU against GPU and oracle).  A
    cache of 3 slots is streamed by one workgroup per (sequence, head), whose
    last one advances the positions; 16 slots split each stream over several
    workgroups with separate combine and advance launches."""
    _need_gpu()
    B, H, G, k0, M = 2, 4, 2, 2, 3
    L = S * M
    inp = synth.draw_prefill(40, B, L, H, G, N, P, io=io, qscale=30.0)
    d = _to_dev(inp)
    gate = 0.75
    full = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    # the first k0 chunks alone: their memories and f32 final state seed decode
    pre = {k: v[:, :k0 * S].contiguous() if k != "A" else v for k, v in d.items()}
    head = api.prefill(pre["x"], pre["dt"], pre["A"], pre["Bm"], pre["C"], pre["Q"], pre["E"],
                       gate, S)
    st = api.new_decode_state(B, H, G, N, P, S, cap, io, DEV)
    st["cache"][:, :, :k0].copy_(head["dH"])
    st["h"].copy_(head["h_final"])
    st["n_chunks"].fill_(k0)
    ys = []
    for t in range(k0 * S, L):
        ys.append(api.decode_step(st, d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(),
                                  d["A"], d["Bm"][:, t].contiguous(), d["C"][:, t].contiguous(),
                                  d["Q"][:, t].contiguous(), d["E"][:, t].contiguous(), gate))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, dim=1)
    n = _np(inp)
    ref = oracle.prefill(n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"], n["E"], gate, S)
    assert_parity(y_dec, ref["y"][:, k0 * S:], io, "decoded y vs oracle prefill")
    assert_parity(y_dec, synth.as_f64(full["y"][:, k0 * S:]), io, "decoded y vs GPU prefill")
    assert_parity(_pn_to_np(st["cache"][:, :, k0]), ref["dH"][:, :, k0], io, "appended memory")
    assert_parity(_pn_to_np(st["h"]), ref["h_final"], io, "final state")
    assert st["n_chunks"].tolist() == [M] * B and st["pos"].tolist() == [0] * B


@pytest.mark.parametrize("io,N,P,S,k0,M", [(torch.bfloat16, 128, 64, 256, 2, 2),
                                             (torch.bfloat16, 64, 64, 64, 3, 2),
                                             (torch.float32, 16, 16, 32, 4, 3)])
def test_prefill_continuation(io, N, P, S, k0, M):
    """Chunked prefill: prefill k0 chunks, keep their memories in a decode
    cache and their final state, then prefill the next M chunks from there;
    the continued outputs, memories and final state match the oracle's
    prefill of the whole sequence."""
    _need_gpu()
    B, H, G = 2, 4, 2
    L = (k0 + M) * S
    print(f"continuation {io} N{N} P{P} S{S} k0={k0} M={M}", flush=True)
    inp = synth.draw_prefill(60 + k0, B, L, H, G, N, P, io=io, qscale=10.0)
    d = _to_dev(inp)
    gate = 0.5
    part = lambda lo, hi: {k: (v if k == "A" else v[:, lo:hi].contiguous()) for k, v in d.items()}
    pre, tail = part(0, k0 * S), part(k0 * S, L)
    head = api.prefill(pre["x"], pre["dt"], pre["A"], pre["Bm"], pre["C"], pre["Q"], pre["E"],
                       gate, S)
    cache = torch.zeros(B, H, k0 + M + 1, P, N, dtype=io, device=DEV)
    cache[:, :, :k0].copy_(head["dH"])
    cont = api.prefill_continue(tail["x"], tail["dt"], tail["A"], tail["Bm"], tail["C"],
                                tail["Q"], tail["E"], gate, S, cache, k0, head["h_final"])
    torch.cuda.synchronize()
    n = _np(inp)
    ref = oracle.prefill(n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"], n["E"], gate, S)
    assert_parity(_pn_to_np(cont["dH"]), ref["dH"][:, :, k0:], io, "continued memories")
    assert_parity(cont["y_ssd"], ref["y_ssd"][:, k0 * S:], io, "continued y_ssd")
    assert_parity(_pn_to_np(cont["h_final"]), ref["h_final"], io, "continued final state")
    assert_parity(cont["y"], ref["y"][:, k0 * S:], io, "continued y")


def test_sma_continuation_arbitrary_cache():
    """dart_sma_fwd_cont over prior memories that no prefill produced (a
    seeded cache with spare capacity) against the oracle's sma_continue."""
    _need_gpu()
    B, H, G, N, P, S, k0, M = 2, 3, 3, 32, 32, 32, 5, 3
    io = torch.float32
    L = M * S
    inp = synth.draw_prefill(70, B, L, H, G, N, P, io=io, qscale=10.0)
    d = _to_dev(inp)
    cache = synth.draw_state(71, (B, H, k0 + 2, P, N), 0.05, io, device=DEV)
    h0 = synth.draw_state(72, (B, H, P, N), 0.05, torch.float32, device=DEV)
    gate = 0.75
    cont = api.prefill_continue(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate,
                                S, cache, k0, h0)
    torch.cuda.synchronize()
    n = _np(inp)
    prior = _pn_to_np(cache)[:, :, :k0]
    dH = oracle.chunk_states(n["x"], n["dt"], n["A"], n["Bm"], S)
    o_ref = oracle.sma_continue(n["Q"], n["E"], n["C"], prior, dH, S)
    o_gpu = (synth.as_f64(cont["y"]) - synth.as_f64(cont["y_ssd"])) / gate
    assert_parity(o_gpu, o_ref, io, "continued SMA readout")


# ------------------------------------------------------ full-size samples
def _oracle_pair(n, b, h, H, G, S, gate, tokens=None):
    """Oracle outputs of one (batch, head) pair, from sliced inputs."""
    g = h // (H // G)
    sl = dict(x=n["x"][b:b + 1, :, h:h + 1], dt=n["dt"][b:b + 1, :, h:h + 1],
              A=n["A"][h:h + 1], Bm=n["Bm"][b:b + 1, :, g:g + 1], C=n["C"][b:b + 1, :, g:g + 1],
              Q=n["Q"][b:b + 1, :, g:g + 1], E=n["E"][b:b + 1, :, h:h + 1])
    dH = oracle.chunk_states(sl["x"], sl["dt"], sl["A"], sl["Bm"], S)
    H_in = oracle.state_pass(dH, sl["dt"], sl["A"], S)
    y_ssd = oracle.chunk_output(sl["x"], sl["dt"], sl["A"], sl["Bm"], sl["C"], H_in, S)
    o = oracle.sma(sl["Q"], sl["E"], sl["C"], dH, S, tokens=tokens)
    return dH[0, 0], H_in[0, 0], y_ssd[0, :, 0], o[0, :, 0], \
        oracle.gated_output(y_ssd, o, gate)[0, :, 0]


@pytest.mark.parametrize("qscale", [1.0, 1e3])
def test_config2_full_size_sampled_pairs(qscale):
    """Prefill bf16 at the Mamba-2 ~370M layer shape (batch 4, 32 heads,
    groups of 8 heads, L=8192, S=256, N=128, P=64), the configuration the
    benchmark times, in the launch configuration it times (heads of one
    (batch, group) side by side on one XCD); every output of three sampled
    (batch, head) pairs is checked against the oracle.  With sharpened
    queries (gate 1) the SMA readout o = y - y_ssd is also checked alone."""
    _need_gpu()
    B, L, H, G, N, P, S = 4, 8192, 32, 4, 128, 64, 256
    gate = 0.5 if qscale == 1.0 else 1.0
    print(f"c2 full size qscale {qscale}", flush=True)
    inp = synth.draw_prefill(0, B, L, H, G, N, P, io=torch.bfloat16, qscale=qscale)
    d = _to_dev(inp)
    out = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    torch.cuda.synchronize()
    n = _np(inp)
    io = torch.bfloat16
    for b, h in [(0, 0), (1, 13), (3, 31)]:
        dH, H_in, y_ssd, o, y = _oracle_pair(n, b, h, H, G, S, gate)
        assert_parity(_pn_to_np(out["dH"][b, h]), dH, io, f"c2 dH b{b} h{h}")
        assert_parity(_pn_to_np(out["H_in"][b, h]), H_in[:-1], io, f"c2 H_in b{b} h{h}")
        assert_parity(_pn_to_np(out["h_final"][b, h]), H_in[-1], io, f"c2 h_final b{b} h{h}")
        assert_parity(out["y_ssd"][b, :, h], y_ssd, io, f"c2 y_ssd b{b} h{h}")
        assert_parity(out["y"][b, :, h], y, io, f"c2 y b{b} h{h}")
        if qscale != 1.0:
            o_gpu = synth.as_f64(out["y"][b, :, h]) - synth.as_f64(out["y_ssd"][b, :, h])
            assert_parity(o_gpu, o, io, f"c2 o (sharpened) b{b} h{h}")


def test_config4_full_size_decode_all_pairs():
    """Decode bf16: batch 64, 32 heads, N=128, P=64, S=256, 128 cached chunks
    per sequence (4 GiB cache), one new token at the start of chunk 128;
    every (sequence, head) pair against the oracle, which is run one
    sequence at a time (its 64 MB slice of the cache)."""
    _need_gpu()
    B, H, N, P, S, mx = 64, 32, 128, 64, 256, 128
    io = torch.bfloat16
    st = api.new_decode_state(B, H, H, N, P, S, mx, io, DEV)
    st["cache"].copy_(synth.draw_state(50, (B, H, mx, P, N), 0.01, io, device=DEV))
    st["h"].copy_(synth.draw_state(51, (B, H, P, N), 0.01, torch.float32, device=DEV))
    st["dH_cur"].copy_(synth.draw_state(52, (B, H, P, N), 0.01, torch.float32, device=DEV))
    st["n_chunks"].fill_(mx)
    h_before, dHc_before = st["h"].clone(), st["dH_cur"].clone()
    tok = synth.draw_decode_token(53, B, H, H, N, P, io=io)
    d = _to_dev(tok)
    y = api.decode_step(st, d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.5)
    torch.cuda.synchronize()
    # pos 0 appends nothing: the cache after the step is the cache the step read
    n = _np(tok)
    y_ref = np.empty((B, H, P))
    h_ref = np.empty((B, H, N, P))
    for b in range(B):
        pre = {"cache": _pn_to_np(st["cache"][b:b + 1]), "h": _pn_to_np(h_before[b:b + 1]),
               "dH_cur": _pn_to_np(dHc_before[b:b + 1]), "n_chunks": np.array([mx]),
               "pos": np.array([0])}
        sl = {k: v[b:b + 1] for k, v in n.items() if k != "A"}
        yr, new = oracle.decode_step(pre, sl["x"], sl["dt"], n["A"], sl["Bm"], sl["C"], sl["Q"],
                                     sl["E"], 0.5, S)
        y_ref[b], h_ref[b] = yr[0], new["h"][0]
        if b % 16 == 15:
            print(f"c4 oracle: {b + 1} of {B} sequences", flush=True)
    assert_parity(y, y_ref, io, "c4 decode y (all pairs)")
    assert_parity(_pn_to_np(st["h"]), h_ref, io, "c4 decode h (all pairs)")
    assert st["n_chunks"].tolist() == [mx] * B and st["pos"].tolist() == [1] * B


@pytest.mark.parametrize("qscale", [1.0, 1e3])
def test_config3_long_context_sampled_tokens(qscale):
    """Long-context prefill bf16 (batch 1, 32 heads, L=65536, S=256, N=128,
    P=64: 256 chunk memories per head).  For three heads the oracle computes
    every memory and the SMA readout of 64 tokens spread over all chunk
    indices (first, middle and last chunks included: the last chunk's
    tokens attend 255 memories).  At qscale 1 the boundary states, y_ssd and
    y are checked too; with sharpened queries (gate 1) the readout
    o = y - y_ssd of the sampled tokens is checked alone."""
    _need_gpu()
    B, L, H, G, N, P, S = 1, 65536, 32, 32, 128, 64, 256
    gate = 0.5 if qscale == 1.0 else 1.0
    M = L // S
    print(f"c3 long context qscale {qscale}", flush=True)
    inp = synth.draw_prefill(3, B, L, H, G, N, P, io=torch.bfloat16, qscale=qscale)
    d = _to_dev(inp)
    out = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    chunks = np.unique(np.concatenate([[0, 1, 2, M // 2, M - 2, M - 1],
                                       rng.integers(0, M, 58)]))
    tokens = np.sort(chunks * S + rng.integers(0, S, chunks.size))
    tokens = np.unique(np.concatenate([tokens, [L - 1]]))
    io = torch.bfloat16
    for h in (0, 17, 31):
        sl = {k: synth.as_f64(v[:, :, h:h + 1]) for k, v in inp.items() if k != "A"}
        A = synth.as_f64(inp["A"][h:h + 1])
        dH = oracle.chunk_states(sl["x"], sl["dt"], A, sl["Bm"], S)
        o = oracle.sma(sl["Q"], sl["E"], sl["C"], dH, S, tokens=tokens)
        assert_parity(_pn_to_np(out["dH"][0, h]), dH[0, 0], io, f"c3 dH h{h}")
        if qscale == 1.0:
            H_in = oracle.state_pass(dH, sl["dt"], A, S)
            y_ssd = oracle.chunk_output(sl["x"], sl["dt"], A, sl["Bm"], sl["C"], H_in, S)
            y = oracle.gated_output(y_ssd, o, gate)
            assert_parity(_pn_to_np(out["H_in"][0, h]), H_in[0, 0, :-1], io, f"c3 H_in h{h}")
            assert_parity(_pn_to_np(out["h_final"][0, h]), H_in[0, 0, -1], io,
                          f"c3 h_final h{h}")
            assert_parity(out["y_ssd"][0, :, h], y_ssd[0, :, 0], io, f"c3 y_ssd h{h}")
            assert_parity(out["y"][0, tokens, h], y[0, tokens, 0], io, f"c3 y (sampled) h{h}")
        else:
            o_gpu = synth.as_f64(out["y"][0, tokens, h]) - synth.as_f64(out["y_ssd"][0, tokens, h])
            assert_parity(o_gpu, o[0, tokens, 0], io, f"c3 o (sharpened, sampled) h{h}")


def _sma_launches(d, out, gate, S, reps):
    """reps launches of dart_sma_fwd into fresh outputs (after one prefill)."""
    ys = []
    for _ in range(reps):
        y = torch.full_like(out["y"], float("nan"))
        api.dart_sma_fwd(d["Q"], d["E"], d["C"], out["dH"], out["y_ssd"], gate, y, S)
        ys.append(y)
    torch.cuda.synchronize()
    return ys


def test_grouped_sma_one_memory_tiles_repeated():
    """Heads sharing a group, two chunks: every tile of chunk 1 sees one
    memory, so o_t = C_tᵀ·dH[0] (the softmax weight is 1) and each head of
    a group is finished after a single step, the case where the direct
    loads of a head's y_ssd rows are newest.  o = y - y_ssd against the
    oracle on every token, and 20 launches bit-identical."""
    _need_gpu()
    B, L, H, G, N, P, S, gate = 4, 512, 32, 4, 128, 64, 256, 1.0
    inp = synth.draw_prefill(31, B, L, H, G, N, P, io=torch.bfloat16, qscale=10.0)
    d = _to_dev(inp)
    out = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    ys = _sma_launches(d, out, gate, S, 20)
    n = _np(inp)
    dH = oracle.chunk_states(n["x"], n["dt"], n["A"], n["Bm"], S)
    o_ref = oracle.sma(n["Q"], n["E"], n["C"], dH, S)
    for r, y in enumerate(ys):
        assert torch.equal(y, ys[0]), f"launch {r} differs from launch 0"
    o_gpu = synth.as_f64(ys[0]) - synth.as_f64(out["y_ssd"])
    assert_parity(o_gpu, o_ref, torch.bfloat16, "o (one memory per tile)")


def test_sma_repeated_launches_bit_identical():
    """The L=8K ~370M-layer shape: ten SMA launches over the same inputs give
    bit-identical outputs (no launch-to-launch variation from LDS staging)."""
    _need_gpu()
    B, L, H, G, N, P, S, gate = 4, 8192, 32, 4, 128, 64, 256, 0.5
    d = _to_dev(synth.draw_prefill(0, B, L, H, G, N, P, io=torch.bfloat16))
    out = api.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate, S)
    ys = _sma_launches(d, out, gate, S, 10)
    for r, y in enumerate(ys):
        assert torch.equal(y, ys[0]), f"launch {r} differs from launch 0"
