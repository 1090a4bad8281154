"""The allocation-free decode entry point (dart_sma_decode_noalloc) against
dart_sma_decode on the same inputs: identical kernels, so every output and
state tensor must match bit for bit.  Two calls in a row, the second with
fewer (sequence, head) pairs (more chunk splits), so stale scratch contents
from the first call cannot leak into the second."""
import pytest
import torch

from ssm_state_attention_amd import api, synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _state(seed, B, H, G, N, P, S, mx, io, n_chunks, pos):
    st = api.new_decode_state(B, H, G, N, P, S, mx, io, DEV)
    st["cache"].copy_(synth.draw_state(seed, (B, H, mx, P, N), 0.01, io, device=DEV))
    st["h"].copy_(synth.draw_state(seed + 1, (B, H, P, N), 0.01, torch.float32, device=DEV))
    st["dH_cur"].copy_(synth.draw_state(seed + 2, (B, H, P, N), 0.01, torch.float32,
                                        device=DEV))
    st["n_chunks"].copy_(torch.tensor(n_chunks, dtype=torch.int32))
    st["pos"].copy_(torch.tensor(pos, dtype=torch.int32))
    return st


def _both(seed, B, H, G, N, P, S, mx, io, n_chunks, pos, qscale):
    print(f"noalloc case B{B} H{H} G{G} N{N} P{P} S{S} max{mx} {io}", flush=True)
    ref = _state(seed, B, H, G, N, P, S, mx, io, n_chunks, pos)
    new = _state(seed, B, H, G, N, P, S, mx, io, n_chunks, pos)
    tok = {k: v.to(DEV) for k, v in
           synth.draw_decode_token(seed + 3, B, H, G, N, P, io=io, qscale=qscale).items()}
    args = (tok["x"], tok["dt"], tok["A"], tok["Bm"], tok["C"], tok["Q"], tok["E"], 0.75)
    y_ref = torch.empty(B, H, P, dtype=io, device=DEV)
    y_new = torch.full((B, H, P), float("nan"), dtype=io, device=DEV)
    api.dart_sma_decode(*args, ref["cache"], ref["h"], ref["dH_cur"], ref["n_chunks"],
                        ref["pos"], y_ref, ref["workspace"], S)
    full = torch.zeros(1, dtype=torch.int32, device=DEV)
    api.dart_sma_decode_noalloc(*args, new["cache"], new["h"], new["dH_cur"], new["n_chunks"],
                                new["pos"], y_new, S, cache_full=full)
    torch.cuda.synchronize()
    assert torch.equal(y_new, y_ref)
    for k in ("cache", "h", "dH_cur", "n_chunks", "pos"):
        assert torch.equal(new[k], ref[k]), k
    assert full.item() == int(api.cache_overflowed(ref))


def test_noalloc_decode_matches_workspace_decode():
    # call 1: 64 pairs, one sequence closes its chunk, one overflows its cache
    _both(80, 8, 8, 4, 128, 64, 64, 12, torch.bfloat16,
          [5, 0, 11, 12, 3, 7, 1, 9], [63, 0, 17, 63, 5, 63, 62, 1], 30.0)
    # call 2, right after: 6 pairs (more splits per pair), fp32 io
    _both(90, 2, 3, 3, 32, 32, 32, 9, torch.float32, [4, 9], [31, 2], 10.0)
    # call 3: the benchmark decode shape's element types at many pairs (one split)
    _both(100, 64, 32, 32, 128, 64, 256, 8, torch.bfloat16, list(range(8)) * 8,
          [255, 0, 3, 128] * 16, 1.0)


def test_noalloc_decode_replayed_from_a_captured_graph():
    """Callers under HIP graph capture are among those the allocation-free
    entry point serves: one decode step captured once and replayed five
    times (new token values copied into the captured inputs before each
    replay, eager work between the replays) matches dart_sma_decode run
    eagerly on a twin state, bit for bit, at every replay; sequence 0
    closes its chunk during the replays."""
    B, H, G, N, P, S, mx, io = 4, 8, 4, 128, 64, 64, 8, torch.bfloat16
    n_chunks, pos = [2, 5, 0, 7], [60, 3, 63, 10]
    print("noalloc graph replay case", flush=True)
    ref = _state(110, B, H, G, N, P, S, mx, io, n_chunks, pos)
    cap = _state(110, B, H, G, N, P, S, mx, io, n_chunks, pos)
    warm = _state(110, B, H, G, N, P, S, mx, io, n_chunks, pos)
    names = ("x", "dt", "A", "Bm", "C", "Q", "E")
    inp = {k: v.to(DEV) for k, v in synth.draw_decode_token(113, B, H, G, N, P, io=io).items()}
    args = tuple(inp[k] for k in names) + (0.75,)
    y_cap = torch.empty(B, H, P, dtype=io, device=DEV)
    # the first call on a device looks the scratch address up: not under capture
    api.dart_sma_decode_noalloc(*args, warm["cache"], warm["h"], warm["dH_cur"],
                                warm["n_chunks"], warm["pos"], torch.empty_like(y_cap), S)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        api.dart_sma_decode_noalloc(*args, cap["cache"], cap["h"], cap["dH_cur"],
                                    cap["n_chunks"], cap["pos"], y_cap, S)
    torch.cuda.synchronize()
    for rep in range(5):
        tok = synth.draw_decode_token(120 + rep, B, H, G, N, P, io=io)
        for k in names:
            inp[k].copy_(tok[k].to(DEV))
        graph.replay()
        y_ref = torch.empty(B, H, P, dtype=io, device=DEV)
        api.dart_sma_decode(*args, ref["cache"], ref["h"], ref["dH_cur"], ref["n_chunks"],
                            ref["pos"], y_ref, ref["workspace"], S)
        float(torch.randn(1 << 20, device=DEV).square().sum())  # eager work in between
        torch.cuda.synchronize()
        assert torch.equal(y_cap, y_ref), f"replay {rep}: y"
        for k in ("cache", "h", "dH_cur", "n_chunks", "pos"):
            assert torch.equal(cap[k], ref[k]), f"replay {rep}: {k}"
    assert int(cap["n_chunks"][0].item()) == 3  # sequence 0 closed its chunk
