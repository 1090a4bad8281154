"""GPU parity of the fp8 (E4M3) chunk-memory cache: the encoder against the
oracle's, bit for bit, and the fp8 decode step against the oracle's.

Bar: codes and scales bit-exact where both sides encode the same f32
memories; y, h and dH_cur as for the other parity tests (fp32 max-abs
<= 1e-4, bfloat16 <= 2e-2 * max|ref|).  A memory the decode step appends is
encoded from the GPU's f32 state on one side and the oracle's f64 state on
the other, so a code may differ where the value sits on a rounding
midpoint: there the two codes must be neighbours, the f64 value (divided by
the scale) within 2.56e-3 of their midpoint (1e-5 of the 256 that bounds
the scaled magnitudes), and at most one code in a thousand may differ.
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


def _pn_to_np(t):
    """Library layout [..., P, N] -> oracle layout [..., N, P]."""
    return np.swapaxes(synth.as_f64(t), -1, -2)


def _oracle_quantize(mem):
    """Oracle codes and scales of memories [..., R, C] (any element order:
    the encoding is per element with one scale per memory)."""
    lead = mem.shape[:-2]
    codes = np.empty(mem.shape, dtype=np.uint8)
    scales = np.empty(lead, dtype=np.float64)
    for idx in np.ndindex(*lead):
        codes[idx], scales[idx] = oracle.fp8_quantize_memory(mem[idx])
    return codes, scales


def _memories(seed, shape):
    """f32 memories with magnitudes spread over many binades: N(0, 1) values,
    each memory times 2^U with U uniform in [-40, 40]; memory 0 of every
    (batch, head) is all zero."""
    m = synth.draw_state(seed, shape, 1.0, torch.float32)
    rng = np.random.default_rng(seed + 1000)
    mag = np.exp2(rng.uniform(-40.0, 40.0, shape[:-2])).astype(np.float32)
    m = m * torch.from_numpy(mag)[..., None, None]
    m[:, :, 0] = 0.0
    return m


def _ties(shape, e, seed):
    """One memory of E4M3 midpoints times 2^e (ties of the encoder), with one
    entry at 200·2^e so that its scale is 2^e."""
    fin = np.unique(oracle.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    fin = fin[fin < 200.0]
    mids = 0.5 * (fin[1:] + fin[:-1])
    rng = np.random.default_rng(seed)
    v = rng.choice(np.concatenate([mids, -mids, fin, -fin]), size=shape)
    v.flat[0] = 200.0
    return torch.from_numpy((v * 2.0 ** e).astype(np.float32))


@pytest.mark.parametrize("io,N,P", [(torch.bfloat16, 128, 64), (torch.bfloat16, 128, 128),
                                    (torch.bfloat16, 64, 64), (torch.float32, 16, 16),
                                    (torch.float32, 32, 32)])
def test_fp8_store_bit_exact(io, N, P):
    """dart_cache_fp8_store against the oracle's encoder on the same f32
    memories: every code and scale equal; slots outside [first, first+n)
    untouched."""
    _need_gpu()
    B, H, n, first, mx = 2, 3, 5, 2, 9
    print(f"fp8 store case {io} N{N} P{P} B{B} H{H} n{n} first{first} max{mx}", flush=True)
    mem = _memories(60 + N + P, (B, H, n, P, N))
    mem[1, 2, 3] = _ties((P, N), -7, 61)
    mem[0, 1, 4] = _ties((P, N), 12, 62)
    cache8 = torch.full((B, H, mx, P, N), 0x5A, dtype=torch.uint8, device=DEV)
    scale = torch.full((B, H, mx), 3.0, dtype=torch.float32, device=DEV)
    api.dart_cache_fp8_store(mem.to(DEV), first, cache8, scale, H, 64, io)
    torch.cuda.synchronize()
    codes, scales = _oracle_quantize(mem.double().numpy())
    got = cache8[:, :, first:first + n].cpu().numpy()
    bad = np.argwhere(got != codes)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"
    assert np.array_equal(scale[:, :, first:first + n].cpu().numpy().astype(np.float64), scales)
    outside = torch.ones(mx, dtype=torch.bool)
    outside[first:first + n] = False
    assert bool((cache8[:, :, outside] == 0x5A).all())
    assert bool((scale[:, :, outside] == 3.0).all())


def _check_codes(codes_gpu, scale_gpu, mem_ref, what):
    """A memory encoded from the GPU's f32 values: scale equal to the
    oracle's and codes equal except on rounding midpoints (see the module
    docstring)."""
    codes_ref, s_ref = oracle.fp8_quantize_memory(mem_ref)
    assert float(scale_gpu) == s_ref, f"{what}: scale {float(scale_gpu)} vs {s_ref}"
    diff = np.flatnonzero(codes_gpu.ravel() != codes_ref.ravel())
    print(f"{what}: {diff.size} of {codes_ref.size} codes on a rounding midpoint", flush=True)
    assert diff.size <= max(2, codes_ref.size // 1000), f"{what}: {diff.size} codes differ"
    if diff.size:
        a = oracle.fp8_e4m3_decode(codes_gpu.ravel()[diff])
        b = oracle.fp8_e4m3_decode(codes_ref.ravel()[diff])
        v = mem_ref.ravel()[diff] / s_ref
        assert np.all(np.abs(v - 0.5 * (a + b)) <= 2.56e-3), what
        both = np.sort(np.stack([a, b]), axis=0)
        # neighbours: no E4M3 value strictly between them
        fin = np.unique(oracle.fp8_e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
        fin = np.concatenate([-fin[::-1], fin])
        for lo, hi in both.T:
            assert not np.any((fin > lo) & (fin < hi)), f"{what}: codes not neighbours"


def _decode_case_fp8(B, H, G, N, P, S, mx, n_chunks, pos, io, seed, gate=0.5, qscale=1.0):
    _need_gpu()
    print(f"fp8 decode case B{B} H{H} G{G} N{N} P{P} S{S} max{mx} n{n_chunks} pos{pos} "
          f"{io} seed{seed}", flush=True)
    st = api.new_decode_state(B, H, G, N, P, S, mx, io, DEV, fp8_cache=True)
    mem = synth.draw_state(seed, (B, H, mx, P, N), 0.01, torch.float32)
    api.store_memories(st, mem.to(DEV))
    st["h"].copy_(synth.draw_state(seed + 1, (B, H, P, N), 0.01, torch.float32))
    st["dH_cur"].copy_(synth.draw_state(seed + 2, (B, H, P, N), 0.01, torch.float32))
    st["n_chunks"].copy_(torch.tensor(n_chunks, dtype=torch.int32))
    st["pos"].copy_(torch.tensor(pos, dtype=torch.int32))
    codes, scales = _oracle_quantize(np.swapaxes(mem.double().numpy(), -1, -2))
    assert np.array_equal(np.swapaxes(st["cache8"].cpu().numpy(), -1, -2), codes)
    ostate = {"codes": codes, "scales": scales, "h": _pn_to_np(st["h"]),
              "dH_cur": _pn_to_np(st["dH_cur"]), "n_chunks": np.array(n_chunks),
              "pos": np.array(pos)}
    tok = synth.draw_decode_token(seed + 3, B, H, G, N, P, io=io, qscale=qscale)
    d = {k: v.to(DEV) for k, v in tok.items()}
    y = api.decode_step(st, d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], gate)
    torch.cuda.synchronize()
    n = {k: synth.as_f64(v) for k, v in tok.items()}
    y_ref, new = oracle.decode_step_fp8(ostate, n["x"], n["dt"], n["A"], n["Bm"], n["C"],
                                        n["Q"], n["E"], gate, S)
    assert_parity(y, y_ref, io, "fp8 decode y")
    assert_parity(_pn_to_np(st["h"]), new["h"], io, "fp8 decode h")
    assert_parity(_pn_to_np(st["dH_cur"]), new["dH_cur"], io, "fp8 decode dH_cur")
    assert st["n_chunks"].cpu().tolist() == list(new["n_chunks"])
    assert st["pos"].cpu().tolist() == list(new["pos"])
    # the f64 memory each closing token appends: the float-cache oracle step
    fstate = dict(ostate, cache=oracle.fp8_dequantize(codes, scales))
    del fstate["codes"], fstate["scales"]
    _, newf = oracle.decode_step(fstate, n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"],
                                 n["E"], gate, S, cache_bf16=False)
    c8 = np.swapaxes(st["cache8"].cpu().numpy(), -1, -2)
    sc = st["scale"].cpu().numpy().astype(np.float64)
    for b in range(B):
        k = n_chunks[b]
        keep = np.ones(mx, dtype=bool)
        if new["n_chunks"][b] == k + 1:
            keep[k] = False
            for h in range(H):
                _check_codes(c8[b, h, k], sc[b, h, k], newf["cache"][b, h, k],
                                f"appended b{b} h{h}")
        assert np.array_equal(c8[b][:, keep], codes[b][:, keep])
        assert np.array_equal(sc[b][:, keep], scales[b][:, keep])
    return st


@pytest.mark.parametrize("io,N,P", [(torch.bfloat16, 128, 64), (torch.bfloat16, 64, 64),
                                    (torch.bfloat16, 128, 128), (torch.float32, 16, 16),
                                    (torch.float32, 32, 32)])
def test_decode_fp8_small(io, N, P):
    """Chunk ranges split over workgroups; one sequence closes its chunk
    (fp8 append), one starts from an empty cache."""
    _decode_case_fp8(3, 4, 2, N, P, 64, 12, [5, 0, 11], [63, 0, 17], io, seed=70)


def test_decode_fp8_sharpened():
    _decode_case_fp8(2, 4, 4, 128, 64, 256, 16, [16, 9], [3, 255], torch.bfloat16, seed=71,
                     qscale=1e4)


def test_decode_fp8_many_pairs():
    """Enough pairs that each workgroup streams its whole cache; half the
    sequences append."""
    _decode_case_fp8(32, 32, 32, 128, 64, 256, 8, list(range(1, 9)) * 4, [255, 0] * 16,
                     torch.bfloat16, seed=72)


def test_decode_fp8_continues_prefill():
    """Prefill two chunks, encode their memories (dart_cache_fp8_store on
    the prefill's f32 memories), decode the third chunk token by token over
    the fp8 cache; against the oracle doing the same in f64."""
    _need_gpu()
    io, N, P, S = torch.bfloat16, 128, 64, 64
    B, H, G, k0, M = 2, 4, 2, 2, 3
    L, gate = S * M, 0.75
    inp = synth.draw_prefill(41, B, L, H, G, N, P, io=io, qscale=30.0)
    d = {k: v.to(DEV) for k, v in inp.items()}
    pre = {k: v[:, :k0 * S].contiguous() if k != "A" else v for k, v in d.items()}
    head = api.prefill(pre["x"], pre["dt"], pre["A"], pre["Bm"], pre["C"], pre["Q"], pre["E"],
                       gate, S)
    st = api.new_decode_state(B, H, G, N, P, S, M, io, DEV, fp8_cache=True)
    api.store_memories(st, head["dH_f32"])
    st["h"].copy_(head["h_final"])
    st["n_chunks"].fill_(k0)
    ys = []
    for t in range(k0 * S, L):
        ys.append(api.decode_step(st, d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(),
                                  d["A"], d["Bm"][:, t].contiguous(), d["C"][:, t].contiguous(),
                                  d["Q"][:, t].contiguous(), d["E"][:, t].contiguous(), gate))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, dim=1)
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    npre = {k: v[:, :k0 * S] if k != "A" else v for k, v in n.items()}
    ref = oracle.prefill(npre["x"], npre["dt"], npre["A"], npre["Bm"], npre["C"], npre["Q"],
                         npre["E"], gate, S)
    codes = np.zeros((B, H, M, N, P), dtype=np.uint8)
    scales = np.ones((B, H, M))
    codes[:, :, :k0], scales[:, :, :k0] = _oracle_quantize(ref["dH"])
    ostate = {"codes": codes, "scales": scales, "h": ref["h_final"],
              "dH_cur": np.zeros((B, H, N, P)), "n_chunks": np.array([k0] * B),
              "pos": np.zeros(B, dtype=np.int64)}
    y_ref = []
    for t in range(k0 * S, L):
        y_t, ostate = oracle.decode_step_fp8(ostate, n["x"][:, t], n["dt"][:, t], n["A"],
                                             n["Bm"][:, t], n["C"][:, t], n["Q"][:, t],
                                             n["E"][:, t], gate, S)
        y_ref.append(y_t)
    assert_parity(y_dec, np.stack(y_ref, axis=1), io, "fp8-cache decoded y")
    # every memory of the cache (two stored, one appended) against the f64
    # memories of the whole sequence: the GPU's memories carry the bfloat16
    # bar's error before they are encoded, so each value is within that bar
    # plus half an E4M3 grid step of the f64 memory
    full = oracle.prefill(n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"], n["E"], gate, S)
    c8 = np.swapaxes(st["cache8"].cpu().numpy(), -1, -2)
    sc = st["scale"].cpu().numpy().astype(np.float64)
    deq = oracle.fp8_dequantize(c8, sc)
    mem = full["dH"]
    for b in range(B):
        for h in range(H):
            for c in range(M):
                m = mem[b, h, c]
                err = np.abs(deq[b, h, c] - m)
                bound = np.abs(m) / 16.0 + sc[b, h, c] * 2.0 ** -10 + 2e-2 * np.max(np.abs(m))
                assert np.all(err <= bound), f"memory b{b} h{h} c{c}"
    assert st["n_chunks"].tolist() == [M] * B and st["pos"].tolist() == [0] * B


def test_decode_fp8_full_size_sampled():
    """fp8 cache at the decode benchmark shape: batch 64, 32 heads, N=128,
    P=64, 128 cached chunks per sequence (1 GiB of codes), bfloat16 io; the
    cache is filled by dart_cache_fp8_store in blocks of 16 chunks; every
    head of three sampled sequences against the oracle."""
    _need_gpu()
    B, H, N, P, S, mx = 64, 32, 128, 64, 256, 128
    io = torch.bfloat16
    st = api.new_decode_state(B, H, H, N, P, S, mx, io, DEV, fp8_cache=True)
    samples = (0, 17, 63)
    mem_s = {b: [] for b in samples}
    for blk in range(mx // 16):
        mem = synth.draw_state(90 + blk, (B, H, 16, P, N), 0.01, torch.float32, device=DEV)
        api.store_memories(st, mem, first=16 * blk)
        for b in samples:
            mem_s[b].append(mem[b].cpu())
        del mem
    st["h"].copy_(synth.draw_state(51, (B, H, P, N), 0.01, torch.float32, device=DEV))
    st["dH_cur"].copy_(synth.draw_state(52, (B, H, P, N), 0.01, torch.float32, device=DEV))
    st["n_chunks"].fill_(mx)
    pre = {}
    for b in samples:
        m = torch.cat(mem_s[b], dim=1)[None]  # [1,H,mx,P,N]
        codes, scales = _oracle_quantize(np.swapaxes(m.double().numpy(), -1, -2))
        assert np.array_equal(np.swapaxes(st["cache8"][b:b + 1].cpu().numpy(), -1, -2), codes)
        pre[b] = {"codes": codes, "scales": scales, "h": _pn_to_np(st["h"][b:b + 1]),
                  "dH_cur": _pn_to_np(st["dH_cur"][b:b + 1]), "n_chunks": np.array([mx]),
                  "pos": np.array([0])}
    tok = synth.draw_decode_token(53, B, H, H, N, P, io=io)
    d = {k: v.to(DEV) for k, v in tok.items()}
    y = api.decode_step(st, d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.5)
    torch.cuda.synchronize()
    n = {k: synth.as_f64(v) for k, v in tok.items()}
    for b in samples:
        sl = {k: v[b:b + 1] for k, v in n.items() if k != "A"}
        y_ref, new = oracle.decode_step_fp8(pre[b], sl["x"], sl["dt"], n["A"], sl["Bm"],
                                            sl["C"], sl["Q"], sl["E"], 0.5, S)
        assert_parity(y[b:b + 1], y_ref, io, f"fp8 decode y b{b}")
        assert_parity(_pn_to_np(st["h"][b:b + 1]), new["h"], io, f"fp8 decode h b{b}")


# ------------------------------------------- chunked prefill from the cache
def _spread_memories(seed, shape, std):
    """f64 memories in the oracle layout [..., N, P]: N(0, std²) values, each
    memory times 2^U with U uniform in [-3, 3], so that the scales differ."""
    rng = np.random.default_rng(seed)
    m = rng.standard_normal(shape) * std
    return m * np.exp2(rng.uniform(-3.0, 3.0, shape[:-2]))[..., None, None]


@pytest.mark.parametrize("N,P,S,k0,M", [(128, 64, 64, 3, 2), (64, 64, 64, 5, 3),
                                        (128, 128, 64, 2, 2), (32, 32, 32, 7, 2),
                                        (128, 64, 256, 1, 2), (128, 64, 64, 0, 2)])
def test_sma_continuation_fp8_cache(N, P, S, k0, M):
    """dart_sma_fwd_cont_fp8 on seeded inputs: prior memories encoded by the
    oracle (codes and scales uploaded as the cache, spare slots holding NaN
    codes that must never be read), new memories drawn directly, y_ssd = 0
    and gate 1, so y is the SMA readout itself; against the oracle's
    sma_continue over the decoded priors."""
    _need_gpu()
    io, B, H, G = torch.bfloat16, 2, 4, 2
    L, cap = M * S, k0 + 2
    print(f"fp8 continuation N{N} P{P} S{S} k0={k0} M={M}", flush=True)
    inp = synth.draw_prefill(120 + k0, B, L, H, G, N, P, io=io, qscale=10.0)
    prior = _spread_memories(121 + k0, (B, H, k0, N, P), 0.05)
    codes = np.full((B, H, cap, N, P), 0x7F, dtype=np.uint8)
    scales = np.full((B, H, cap), np.nan)
    if k0:
        codes[:, :, :k0], scales[:, :, :k0] = _oracle_quantize(prior)
    dH = synth.draw_state(122 + k0, (B, H, M, P, N), 0.05, io)
    cache8 = torch.from_numpy(np.ascontiguousarray(np.swapaxes(codes, -1, -2))).to(DEV)
    scale = torch.from_numpy(scales.astype(np.float32)).to(DEV)
    d = {k: v.to(DEV) for k, v in inp.items()}
    y_ssd = torch.zeros(B, L, H, P, dtype=io, device=DEV)
    y = torch.full((B, L, H, P), float("nan"), dtype=io, device=DEV)
    api.dart_sma_fwd_cont_fp8(d["Q"], d["E"], d["C"], cache8, scale, k0, dH.to(DEV), y_ssd, 1.0,
                              y, S)
    torch.cuda.synchronize()
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    deq = oracle.fp8_dequantize(codes[:, :, :k0], scales[:, :, :k0])
    o_ref = oracle.sma_continue(n["Q"], n["E"], n["C"], deq, _pn_to_np(dH), S)
    assert_parity(y, o_ref, io, "SMA readout over the fp8 cache")


def test_prefill_continuation_fp8_cache():
    """Chunked prefill over the fp8 cache, end to end: prefill k0 chunks,
    encode their f32 memories (dart_cache_fp8_store), continue the next M
    chunks from the fp8 cache and the final state.  Reference: the oracle's
    whole-sequence prefill for y_ssd and the new memories, with the SMA over
    the oracle's own encoding of its first k0 memories.  The two encodings
    start from memories that differ by rounding, so a code may differ by one
    step where a value sits near a midpoint; the bar on y absorbs that."""
    _need_gpu()
    io, N, P, S, k0, M = torch.bfloat16, 128, 64, 64, 3, 2
    B, H, G, gate = 2, 4, 2, 0.5
    L = (k0 + M) * S
    inp = synth.draw_prefill(130, B, L, H, G, N, P, io=io, qscale=10.0)
    d = {k: v.to(DEV) for k, v in inp.items()}
    part = lambda lo, hi: {k: (v if k == "A" else v[:, lo:hi].contiguous()) for k, v in d.items()}
    pre, tail = part(0, k0 * S), part(k0 * S, L)
    head = api.prefill(pre["x"], pre["dt"], pre["A"], pre["Bm"], pre["C"], pre["Q"], pre["E"],
                       gate, S)
    st = api.new_decode_state(B, H, G, N, P, S, k0 + M, io, DEV, fp8_cache=True)
    api.store_memories(st, head["dH_f32"])
    cont = api.prefill_continue(tail["x"], tail["dt"], tail["A"], tail["Bm"], tail["C"],
                                tail["Q"], tail["E"], gate, S, st["cache8"], k0, head["h_final"],
                                scale=st["scale"])
    torch.cuda.synchronize()
    n = {k: synth.as_f64(v) for k, v in inp.items()}
    ref = oracle.prefill(n["x"], n["dt"], n["A"], n["Bm"], n["C"], n["Q"], n["E"], gate, S)
    codes, scales = _oracle_quantize(ref["dH"][:, :, :k0])
    sl = slice(k0 * S, L)
    o_ref = oracle.sma_continue(n["Q"][:, sl], n["E"][:, sl], n["C"][:, sl],
                                oracle.fp8_dequantize(codes, scales), ref["dH"][:, :, k0:], S)
    assert_parity(cont["y"], ref["y_ssd"][:, sl] + gate * o_ref, io, "continued y (fp8 cache)")
    assert_parity(_pn_to_np(cont["h_final"]), ref["h_final"], io, "continued final state")
