"""GPU: the one-pass chunk scan (dart_chunk_scan + dart_chunk_out) against the
two-pass path (dart_chunk_state + dart_state_pass) through the C ABI.

dart_chunk_scan documents its outputs as bit-identical to the two-pass
path's, so every output is compared with torch.equal, over the cases of its
launch: 4, 2 and 1 chunks per workgroup (M divisible by 4, by 2 only, odd),
the XCD-major block order ((batch·groups) % 8 == 0) and the plain order,
an initial state h0, chunks shorter than 256 tokens, P = 128 (two chunks per
workgroup at most), f32 io (the two-kernel recurrence over the workspace)
and a workspace holding garbage or the flags of earlier calls.  The two-pass
path itself is checked against the fp64 oracle in test_gpu_parity.py; the
fused path at the benchmark shape is also checked against the oracle here.
"""
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


def _two_pass(d, S, h0):
    x, Bm = d["x"], d["Bm"]
    B, L, H, P = x.shape
    N, M = Bm.shape[3], L // S
    f32 = dict(dtype=torch.float32, device=DEV)
    o = {"acum": torch.empty(B, H, M, S, **f32),
         "dH": torch.empty(B, H, M, P, N, dtype=x.dtype, device=DEV),
         "dH_f32": torch.empty(B, H, M, P, N, **f32),
         "H_in": torch.empty(B, H, M, P, N, dtype=x.dtype, device=DEV),
         "h_final": torch.empty(B, H, P, N, **f32),
         "y_ssd": torch.empty(B, L, H, P, dtype=x.dtype, device=DEV)}
    api.dart_chunk_state(x, d["dt"], d["A"], Bm, o["acum"], o["dH"], o["dH_f32"], S)
    api.dart_state_pass(x, d["dt"], Bm, d["C"], o["acum"], o["dH_f32"], h0, o["H_in"],
                        o["h_final"], o["y_ssd"], S)
    return o


def _one_pass(d, S, h0, ws, keep_f32):
    x, Bm = d["x"], d["Bm"]
    B, L, H, P = x.shape
    N, M = Bm.shape[3], L // S
    f32 = dict(dtype=torch.float32, device=DEV)
    o = {"acum": torch.full((B, H, M, S), float("nan"), **f32),
         "dH": torch.full((B, H, M, P, N), float("nan"), dtype=x.dtype, device=DEV),
         "dH_f32": torch.full((B, H, M, P, N), float("nan"), **f32) if keep_f32 else None,
         "H_in": torch.full((B, H, M, P, N), float("nan"), dtype=x.dtype, device=DEV),
         "h_final": torch.full((B, H, P, N), float("nan"), **f32),
         "y_ssd": torch.full((B, L, H, P), float("nan"), dtype=x.dtype, device=DEV)}
    api.dart_chunk_scan(x, d["dt"], d["A"], Bm, h0, o["acum"], o["dH"], o["dH_f32"], o["H_in"],
                        o["h_final"], ws, S)
    api.dart_chunk_out(x, d["dt"], Bm, d["C"], o["acum"], o["H_in"], o["y_ssd"], S)
    return o


def _failures(ws, io):
    """The workspace's count of waits that gave up (16-bit io only)."""
    return int(ws[:4].view(torch.int32).item()) if io == torch.bfloat16 else 0


CASES = [
    # B, L, H, G, N, P, S, io, h0_std     (chunks per workgroup, block order)
    (4, 4096, 8, 2, 128, 64, 256, torch.bfloat16, 0.0),    # M=16: 4/wg, XCD-major
    (1, 1536, 4, 1, 128, 64, 256, torch.bfloat16, 0.5),    # M=6: 2/wg, plain order, h0
    (2, 1280, 4, 2, 128, 64, 256, torch.bfloat16, 0.0),    # M=5: 1/wg
    (1, 960, 3, 3, 64, 64, 96, torch.bfloat16, 0.3),       # S=96, M=10: 2/wg
    (2, 2048, 8, 4, 128, 128, 128, torch.bfloat16, 0.0),   # P=128, M=16: 2/wg, XCD-major
    (1, 448, 2, 2, 32, 32, 64, torch.bfloat16, 0.0),       # M=7, small state
    (2, 256, 2, 1, 32, 32, 32, torch.bfloat16, 0.2),       # S=32 (shorter than a K-block), M=8
    (1, 65536, 32, 32, 128, 64, 256, torch.bfloat16, 0.0),  # long context: 64 links per chain
    (1, 1024, 2, 1, 16, 16, 64, torch.float32, 0.5),       # f32 io, two-kernel recurrence
    (1, 1024, 2, 1, 32, 32, 32, torch.float32, 0.0),       # f32 io, S=32
]


@pytest.mark.parametrize("B,L,H,G,N,P,S,io,h0_std", CASES)
def test_one_pass_equals_two_pass(B, L, H, G, N, P, S, io, h0_std):
    _need_gpu()
    print(f"chunk scan B{B} L{L} H{H} G{G} N{N} P{P} S{S} {io} h0_std{h0_std}", flush=True)
    d = {k: v.to(DEV) for k, v in synth.draw_prefill(90 + L + N, B, L, H, G, N, P, io=io).items()}
    h0 = synth.draw_state(91, (B, H, P, N), h0_std, torch.float32).to(DEV) if h0_std else None
    ref = _two_pass(d, S, h0)
    nbytes = api.dart_chunk_scan_workspace(api.prefill_dims(d["x"], d["Bm"], S))
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=DEV)  # any initial contents
    ws[:4].zero_()
    for rep in range(3):  # the same workspace again: the earlier calls' flags must not pass
        got = _one_pass(d, S, h0, ws, keep_f32=rep == 0)
        torch.cuda.synchronize()
        assert _failures(ws, io) == 0, "a hand-over wait gave up"
        for k, v in got.items():
            if v is not None:
                assert torch.equal(v, ref[k]), f"{k} differs from the two-pass path (call {rep})"


def test_one_pass_benchmark_shape_against_oracle_and_two_pass():
    """The prefill benchmark shape (batch 4, 32 heads in 4 groups, L=8192,
    S=256, N=128, P=64): bit-identical to the two-pass path, and the
    recurrence outputs of 3 sampled (batch, head) pairs against the oracle."""
    _need_gpu()
    B, L, H, G, N, P, S = 4, 8192, 32, 4, 128, 64, 256
    print("chunk scan at the benchmark shape", flush=True)
    inp = synth.draw_prefill(0, B, L, H, G, N, P, io=torch.bfloat16)
    d = {k: v.to(DEV) for k, v in inp.items()}
    ref = _two_pass(d, S, None)
    ws = torch.zeros(api.dart_chunk_scan_workspace(api.prefill_dims(d["x"], d["Bm"], S)),
                     dtype=torch.uint8, device=DEV)
    got = _one_pass(d, S, None, ws, keep_f32=False)
    torch.cuda.synchronize()
    assert _failures(ws, torch.bfloat16) == 0
    for k, v in got.items():
        if v is not None:
            assert torch.equal(v, ref[k]), f"{k} differs from the two-pass path"
    g = H // G
    for b, h in ((0, 0), (1, 13), (3, 31)):
        gi = h // g
        xs = synth.as_f64(inp["x"][b:b + 1, :, h:h + 1])
        dts = synth.as_f64(inp["dt"][b:b + 1, :, h:h + 1])
        A = synth.as_f64(inp["A"][h:h + 1])
        dH = oracle.chunk_states(xs, dts, A, synth.as_f64(inp["Bm"][b:b + 1, :, gi:gi + 1]), S)
        hs = oracle.state_pass(dH, dts, A, S)
        hin, hfin = hs[:, :, :-1], hs[:, :, -1]
        for name, gv, rv in (("H_in", got["H_in"][b, h], hin[0, 0]),
                             ("h_final", got["h_final"][b, h], hfin[0, 0])):
            gn = np.swapaxes(synth.as_f64(gv.cpu()), -1, -2)
            err = float(np.max(np.abs(gn - rv)))
            bound = 2e-2 * float(np.max(np.abs(rv)))
            print(f"(b{b}, h{h}) {name}: max err {err:.3e} bound {bound:.3e}", flush=True)
            assert err <= bound


@pytest.mark.parametrize("decayed", [False, True])
def test_prefill_one_pass_equals_default(decayed):
    """api.prefill(one_pass=True) gives the default path's outputs bit for
    bit (y through the SMA and gated add included), and prefill_train the
    same for what the backward reads."""
    _need_gpu()
    B, L, H, G, N, P, S = 2, 2048, 8, 2, 128, 64, 256
    print(f"prefill one_pass decayed={decayed}", flush=True)
    d = {k: v.to(DEV) for k, v in synth.draw_prefill(97, B, L, H, G, N, P, io=torch.bfloat16,
                                                      qscale=30.0).items()}
    h0 = synth.draw_state(98, (B, H, P, N), 0.3, torch.float32).to(DEV)
    args = (d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.5, S)
    a = api.prefill(*args, h0=h0, decayed=decayed)
    b = api.prefill(*args, h0=h0, decayed=decayed, one_pass=True)
    torch.cuda.synchronize()
    assert "dH_f32" not in b
    for k, v in b.items():
        assert torch.equal(v, a[k]), f"{k} differs"
    if not decayed:
        ta = api.prefill_train(*args, h0=h0)
        tb = api.prefill_train(*args, h0=h0, one_pass=True)
        torch.cuda.synchronize()
        for k, v in tb.items():
            assert torch.equal(v, ta[k]), f"prefill_train {k} differs"
