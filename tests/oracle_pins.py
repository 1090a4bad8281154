"""Pins for the fp64 oracle: checks against facts the pages and the
mathematics fix, independent of the oracle's own formulas.

Each ``pin_*`` takes the oracle module (so that the mutation test can run the
same pins against a deliberately broken copy) and raises AssertionError when
the oracle disagrees.  Inputs are small and seeded; every pin finishes in well
under a second.
"""

import json
import math
import os

import numpy as np
import scipy.signal
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _inputs(seed, B=2, L=24, H=4, G=2, N=3, P=5, dt_const=None, A_zero=False):
    rng = np.random.default_rng(seed)
    A = np.zeros(H) if A_zero else -np.exp(rng.uniform(0.0, math.log(16.0), H))
    if dt_const is None:
        dt = np.exp(rng.uniform(math.log(1e-2), math.log(3e-1), (B, L, H)))
    else:
        dt = np.full((B, L, H), float(dt_const))
    x = rng.standard_normal((B, L, H, P))
    Bm = rng.standard_normal((B, L, G, N))
    C = rng.standard_normal((B, L, G, N))
    Q = rng.standard_normal((B, L, G, N))
    E = rng.standard_normal((B, L, H, P))
    return dict(A=A, dt=dt, x=x, Bm=Bm, C=C, Q=Q, E=E)


def _heads(T, H):
    """Grouped [B, L, G, N] -> per head, heads grouped contiguously."""
    G = T.shape[2]
    return np.stack([T[:, :, h // (H // G)] for h in range(H)], axis=2)


def _close(a, b, tol=1e-10, what=""):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert err <= tol * scale, f"{what}: max err {err:.3e} (scale {scale:.3e})"


# --------------------------------------------------------------- recurrence
def pin_recurrence_linear_attention(orc):
    """With A = 0 nothing decays and the SSM is causal linear attention:
    y_t = Σ_{j<=t} (C_t·B_j)·dt_j·x_j  (SSD duality, Pith review axiom
    ledger, paper Eq. 4)."""
    d = _inputs(1, A_zero=True)
    y, _, _ = orc.recurrence(d["x"], d["dt"], d["A"], d["Bm"], d["C"])
    Bh, Ch = _heads(d["Bm"], 4), _heads(d["C"], 4)
    B, L, H, P = d["x"].shape
    ref = np.zeros_like(y)
    for b in range(B):
        for h in range(H):
            for t in range(L):
                for j in range(t + 1):
                    ref[b, t, h] += (Ch[b, t, h] @ Bh[b, j, h]) * d["dt"][b, j, h] * d["x"][b, j, h]
    _close(y, ref, what="linear-attention closed form")


def pin_recurrence_lfilter(orc):
    """With constant dt the decay a = exp(dt·A) is constant, so every state
    entry is a first-order IIR filter h_t = a·h_{t-1} + u_t; scipy's lfilter
    evaluates it independently."""
    dtc = 0.07
    d = _inputs(2, dt_const=dtc)
    _, hfin, states = orc.recurrence(d["x"], d["dt"], d["A"], d["Bm"], d["C"],
                                     keep_states=True)
    B, L, H, P = d["x"].shape
    Bh = _heads(d["Bm"], H)
    N = Bh.shape[-1]
    for b in range(B):
        for h in range(H):
            a = math.exp(dtc * d["A"][h])
            for n in range(N):
                for p in range(P):
                    u = dtc * Bh[b, :, h, n] * d["x"][b, :, h, p]
                    ref = scipy.signal.lfilter([1.0], [1.0, -a], u)
                    _close(states[b, :, h, n, p], ref, what=f"lfilter b{b} h{h} n{n} p{p}")
    _close(hfin, states[:, -1], what="final state")


def pin_single_token(orc):
    """One token from a zero state: y_0 = dt_0·(C_0·B_0)·x_0."""
    d = _inputs(3, L=1)
    y, _, _ = orc.recurrence(d["x"], d["dt"], d["A"], d["Bm"], d["C"])
    Bh, Ch = _heads(d["Bm"], 4), _heads(d["C"], 4)
    ref = (d["dt"][:, 0, :, None] * np.einsum("bhn,bhn->bh", Ch[:, 0], Bh[:, 0])[..., None]
           * d["x"][:, 0])
    _close(y[:, 0], ref, what="single token")


# ------------------------------------------------------------ chunked scan
def pin_state_pass_matches_recurrence(orc):
    """The chunk-boundary states of the chunked scan equal the sequential
    recurrence's state at every chunk end, from a non-zero h0 too (the
    chunked scan is exact; Pith review axiom ledger)."""
    for S in (1, 4, 6):
        d = _inputs(4, L=24)
        rng = np.random.default_rng(40)
        h0 = rng.standard_normal((2, 4, 3, 5))
        _, hfin, states = orc.recurrence(d["x"], d["dt"], d["A"], d["Bm"], d["C"],
                                         h0=h0, keep_states=True)
        dH = orc.chunk_states(d["x"], d["dt"], d["A"], d["Bm"], S)
        H_in = orc.state_pass(dH, d["dt"], d["A"], S, h0)
        M = 24 // S
        _close(H_in[:, :, 0], h0, what="H_in[0]")
        for c in range(M):
            _close(H_in[:, :, c + 1], states[:, (c + 1) * S - 1], what=f"S={S} chunk {c}")
        _close(H_in[:, :, M], hfin, what="h_final")


def pin_chunk_states_unit_chunk(orc):
    """With S = 1 each chunk holds one token and nothing decays inside it:
    ΔH[c] = dt_c·B_c x_cᵀ."""
    d = _inputs(5, L=7)
    dH = orc.chunk_states(d["x"], d["dt"], d["A"], d["Bm"], 1)
    Bh = _heads(d["Bm"], 4)
    ref = np.einsum("blh,blhn,blhp->bhlnp", d["dt"], Bh, d["x"])
    _close(dH, ref, what="S=1 chunk states")


def pin_chunk_states_zero_state_start(orc):
    """ΔH[c] is the state the recurrence reaches at the end of chunk c when
    started from zero at the start of chunk c (definition of a chunk's
    contribution to the chunk-boundary state)."""
    S = 5
    d = _inputs(6, L=15)
    dH = orc.chunk_states(d["x"], d["dt"], d["A"], d["Bm"], S)
    for c in range(3):
        sl = slice(c * S, (c + 1) * S)
        _, hend, _ = orc.recurrence(d["x"][:, sl], d["dt"][:, sl], d["A"],
                                    d["Bm"][:, sl], d["C"][:, sl])
        _close(dH[:, :, c], hend, what=f"chunk {c}")


def pin_chunk_output_matches_recurrence(orc):
    """The quadratic (intra + inter chunk) output equals the recurrence at
    every token (SSD duality)."""
    for S in (1, 4, 8):
        d = _inputs(7, L=24)
        h0 = np.random.default_rng(70).standard_normal((2, 4, 3, 5))
        y_rec, _, _ = orc.recurrence(d["x"], d["dt"], d["A"], d["Bm"], d["C"], h0=h0)
        dH = orc.chunk_states(d["x"], d["dt"], d["A"], d["Bm"], S)
        H_in = orc.state_pass(dH, d["dt"], d["A"], S, h0)
        y = orc.chunk_output(d["x"], d["dt"], d["A"], d["Bm"], d["C"], H_in, S)
        _close(y, y_rec, what=f"chunked output S={S}")


# --------------------------------------------------------------------- SMA
def _mem(seed, B, H, M, N, P):
    return np.random.default_rng(seed).standard_normal((B, H, M, N, P))


def pin_sma_first_chunk_zero_and_single_memory(orc):
    """Tokens of chunk 0 see no completed chunk (readout zero); tokens of
    chunk 1 see exactly one memory, so the softmax weight is 1 and the
    readout is C_tᵀ ΔH[0] whatever the query and key."""
    S, M = 4, 3
    d = _inputs(8, L=S * M)
    dH = _mem(80, 2, 4, M, 3, 5)
    o = orc.sma(d["Q"], d["E"], d["C"], dH, S)
    _close(o[:, :S], np.zeros_like(o[:, :S]), what="chunk 0")
    Ch = _heads(d["C"], 4)
    ref = np.einsum("bthn,bhnp->bthp", Ch[:, S:2 * S], dH[:, :, 0])
    _close(o[:, S:2 * S], ref, what="single memory")


def pin_sma_uniform_when_query_zero(orc):
    """Q = 0 makes every score zero: uniform weights, readout
    C_tᵀ·mean_{c<k} ΔH[c]."""
    S, M = 3, 4
    d = _inputs(9, L=S * M)
    dH = _mem(90, 2, 4, M, 3, 5)
    o = orc.sma(np.zeros_like(d["Q"]), d["E"], d["C"], dH, S)
    Ch = _heads(d["C"], 4)
    for k in range(1, M):
        mean = dH[:, :, :k].mean(axis=2)
        ref = np.einsum("bthn,bhnp->bthp", Ch[:, k * S:(k + 1) * S], mean)
        _close(o[:, k * S:(k + 1) * S], ref, what=f"uniform chunk {k}")


def pin_sma_planted_query(orc):
    """A query aligned with the longest decoded key of a token makes the
    softmax one-hot: the readout becomes C_tᵀ ΔH[c*].  The key of memory c for
    token t is ΔH[c]·E_t (value axis contracted); with Q_t = λ·sqrt(N)·key*
    the score gap to every other memory is λ·(|key*|² - key_c·key*) > 0
    (Cauchy-Schwarz), and λ is set so that the gap is 40."""
    S, M, N, P = 2, 5, 3, 4
    B, H = 1, 2
    rng = np.random.default_rng(11)
    E = rng.standard_normal((B, S * M, H, P))
    C = rng.standard_normal((B, S * M, H, N))
    dH = rng.standard_normal((B, H, M, N, P))
    Q = np.zeros((B, S * M, H, N))
    target = {}
    for t in range(S, S * M):
        k = t // S
        for h in range(H):
            keys = np.array([dH[0, h, c] @ E[0, t, h] for c in range(k)])   # [k, N]
            cstar = int(np.argmax(np.linalg.norm(keys, axis=1)))
            kstar = keys[cstar]
            others = [keys[c] @ kstar for c in range(k) if c != cstar]
            gap = kstar @ kstar - (max(others) if others else 0.0)
            assert gap > 0
            Q[0, t, h] = (40.0 / gap) * math.sqrt(N) * kstar
            target[(t, h)] = cstar
    o = orc.sma(Q, E, C, dH, S)
    for t in range(S, S * M):
        for h in range(H):
            ref = C[0, t, h] @ dH[0, h, target[(t, h)]]
            _close(o[0, t, h], ref, tol=1e-8, what=f"planted t{t} h{h}")


def pin_sma_memory_order_invariant(orc):
    """Softmax attention is a set function of the (key, value) pairs: any
    permutation of the memories a token sees leaves its readout unchanged."""
    S, M = 3, 6
    d = _inputs(12, L=S * M)
    dH = _mem(120, 2, 4, M, 3, 5)
    perm = np.array([3, 0, 4, 1, 2, 5])  # last chunk stays (not visible to itself)
    o = orc.sma(d["Q"], d["E"], d["C"], dH, S)
    o2 = orc.sma(d["Q"], d["E"], d["C"], dH[:, :, perm], S)
    _close(o2[:, (M - 1) * S:], o[:, (M - 1) * S:], what="permuted memories")


def pin_sma_against_library_attention(orc):
    """When E_t is the same vector e for every token, keys K_c = ΔH[c]·e no
    longer depend on t and SMA is ordinary masked softmax attention with
    query Q_t, key K_c and value vec(ΔH[c]), followed by the contraction
    with C_t.  torch's scaled_dot_product_attention (scale 1/sqrt(N), the
    query width) computes the attention part independently."""
    S, M, N, P = 4, 5, 6, 3
    B, H, G = 2, 2, 1
    rng = np.random.default_rng(13)
    e = rng.standard_normal(P)
    E = np.broadcast_to(e, (B, S * M, H, P)).copy()
    Q = 3.0 * rng.standard_normal((B, S * M, G, N))
    C = rng.standard_normal((B, S * M, G, N))
    dH = rng.standard_normal((B, H, M, N, P))
    o = orc.sma(Q, E, C, dH, S)
    L = S * M
    tok_chunk = np.arange(L) // S
    mask = torch.from_numpy(np.arange(M)[None, :] < tok_chunk[:, None])      # [L, M]
    for b in range(B):
        for h in range(H):
            q = torch.from_numpy(Q[b, :, 0])                                    # [L, N]
            kk = torch.from_numpy(np.einsum("cnp,p->cn", dH[b, h], e))          # [M, N]
            v = torch.from_numpy(dH[b, h].reshape(M, N * P))                    # [M, N*P]
            u = torch.nn.functional.scaled_dot_product_attention(
                q[None], kk[None], v[None], attn_mask=mask[None]).numpy()[0]
            ref = np.einsum("tn,tnp->tp", C[b, :, 0], u.reshape(L, N, P))
            _close(o[b, S:, h], ref[S:], what=f"sdpa b{b} h{h}")


def pin_sma_bruteforce(orc):
    """Scalar per-token, per-chunk loops agree with the vectorised readout."""
    S, M = 2, 4
    d = _inputs(14, B=1, L=S * M, H=2, G=1, N=3, P=2)
    d["Q"] *= 4.0
    dH = _mem(140, 1, 2, M, 3, 2)
    _close(orc.sma(d["Q"], d["E"], d["C"], dH, S),
           orc.sma_bruteforce(d["Q"], d["E"], d["C"], dH, S), what="brute force")


# -------------------------------------------------------------------- gate
def pin_gate(orc):
    """g = 0 removes the SMA branch (y = y_ssd, the kernel-level form of the
    paper's 'SMA removed' ablation); y is affine in g."""
    S = 4
    d = _inputs(15, L=16)
    r0 = orc.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.0, S)
    r1 = orc.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 1.0, S)
    r7 = orc.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], 0.7, S)
    _close(r0["y"], r0["y_ssd"], what="g=0")
    _close(r7["y"], r0["y"] + 0.7 * (r1["y"] - r0["y"]), what="affine in g")
    assert np.max(np.abs(r1["y"] - r0["y"])) > 1e-3, "SMA branch has no effect"


# ------------------------------------------------------------ worked example
def pin_worked_scalar_example(orc):
    """Hand-derived scalar case (N = P = 1, S = 1, H = 1): every quantity is
    a short closed form written with math.exp.

    x = (1, 2, -1), dt = (0.5, 0.25, 0.2), A = -2, B = (1, 2, 1),
    C = (1, 1, 2), Q = (1, 1, 1), E = (1, 1, 3), h0 = 0.5, g = 0.5.
    Memories: ΔH = (0.5, 1.0, -0.2).
    States:   h_0 = e^{-1}·0.5 + 0.5,  h_1 = e^{-0.5}·h_0 + 1.0,
              h_2 = e^{-0.4}·h_1 - 0.2;  y_ssd = (h_0, h_1, 2·h_2).
    SMA:      token 0 sees nothing; token 1 sees ΔH[0] only: o_1 = 1·0.5;
              token 2 sees ΔH[0], ΔH[1] with scores 1·0.5·3 = 1.5 and
              1·1.0·3 = 3 and values 2·0.5 = 1 and 2·1.0 = 2.
    """
    x = np.array([1.0, 2.0, -1.0]).reshape(1, 3, 1, 1)
    dt = np.array([0.5, 0.25, 0.2]).reshape(1, 3, 1)
    A = np.array([-2.0])
    Bm = np.array([1.0, 2.0, 1.0]).reshape(1, 3, 1, 1)
    C = np.array([1.0, 1.0, 2.0]).reshape(1, 3, 1, 1)
    Q = np.ones((1, 3, 1, 1))
    E = np.array([1.0, 1.0, 3.0]).reshape(1, 3, 1, 1)
    h0 = np.full((1, 1, 1, 1), 0.5)
    r = orc.prefill(x, dt, A, Bm, C, Q, E, 0.5, 1, h0=h0)
    e = math.exp
    h_0 = e(-1.0) * 0.5 + 0.5
    h_1 = e(-0.5) * h_0 + 1.0
    h_2 = e(-0.4) * h_1 - 0.2
    y_ssd = [h_0, h_1, 2.0 * h_2]
    a0, a1 = e(1.5) / (e(1.5) + e(3.0)), e(3.0) / (e(1.5) + e(3.0))
    o = [0.0, 0.5, a0 * 1.0 + a1 * 2.0]
    _close(r["dH"].ravel(), [0.5, 1.0, -0.2], what="memories")
    _close(r["y_ssd"].ravel(), y_ssd, what="y_ssd")
    _close(r["o"].ravel(), o, what="sma")
    _close(r["y"].ravel(), [ys + 0.5 * oo for ys, oo in zip(y_ssd, o)], what="y")
    _close(r["h_final"].ravel(), [h_2], what="final state")


# ------------------------------------------------------------------ decode
def pin_decode_equals_prefill(orc):
    """Decoding token by token from the state after k completed chunks
    reproduces the prefill outputs, memories and final state (the decode
    cache is exactly the prefill's chunk memories)."""
    S, M, k0 = 3, 4, 1
    B, H, G, N, P = 2, 4, 2, 3, 5
    d = _inputs(16, B=B, L=S * M, H=H, G=G, N=N, P=P)
    g = 0.8
    r = orc.prefill(d["x"], d["dt"], d["A"], d["Bm"], d["C"], d["Q"], d["E"], g, S)
    state = {"cache": np.zeros((B, H, M, N, P)), "h": r["H_in"][:, :, k0].copy(),
             "dH_cur": np.zeros((B, H, N, P)), "n_chunks": np.full(B, k0),
             "pos": np.zeros(B, dtype=np.int64)}
    state["cache"][:, :, :k0] = r["dH"][:, :, :k0]
    for t in range(k0 * S, S * M):
        y, state = orc.decode_step(state, d["x"][:, t], d["dt"][:, t], d["A"],
                                   d["Bm"][:, t], d["C"][:, t], d["Q"][:, t],
                                   d["E"][:, t], g, S, cache_bf16=False)
        _close(y, r["y"][:, t], what=f"decode token {t}")
    _close(state["cache"], r["dH"], what="appended memories")
    _close(state["h"], r["h_final"], what="final state")
    assert list(state["n_chunks"]) == [M] * B and list(state["pos"]) == [0] * B


def pin_round_bf16(orc):
    """round_bf16 is round-to-nearest-even onto the bfloat16 grid (8
    significant bits; subnormal step 2^-133), taken once from fp64.
    Exact midpoints: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 and goes
    to the even significand 1; 1 + 3·2^-8 lies halfway between 1 + 2^-7
    (odd) and 1 + 2^-6 (even).  A value above a midpoint by less than half
    an fp32 step must round up (a conversion through fp32 first would meet
    a tie there and round down).  On fp32 values, where a single rounding
    from fp32 is the same rounding, it agrees with torch's float32 ->
    bfloat16 conversion."""
    cases = [
        (1 + 2.0 ** -8, 1.0),
        (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),
        (-(1 + 2.0 ** -8), -1.0),
        (-(1 + 3 * 2.0 ** -8), -(1 + 2.0 ** -6)),
        (1 + 2.0 ** -8 + 2.0 ** -40, 1 + 2.0 ** -7),
        (1 + 2.0 ** -8 - 2.0 ** -40, 1.0),
        (3 * 2.0 ** 20 + 2.0 ** 13, 3 * 2.0 ** 20),          # tie above 1.5·2^21 (step 2^14): even
        (3 * 2.0 ** 20 + 3 * 2.0 ** 13, 3 * 2.0 ** 20 + 2.0 ** 15),  # tie above an odd multiple
        (2.0 ** -126 * (1 + 2.0 ** -8), 2.0 ** -126),        # tie at the smallest normal
        (2.0 ** -134, 0.0),                                  # half the smallest subnormal: tie to 0
        (3 * 2.0 ** -134, 2.0 ** -132),                      # tie between 1 and 2 subnormal steps
        (0.0, 0.0),
        (2.0 ** 128 * (1 - 2.0 ** -9), np.inf),              # midpoint above the largest finite
        (2.0 ** 128 * (1 - 2.0 ** -8), 2.0 ** 128 * (1 - 2.0 ** -8)),
    ]
    for x, want in cases:
        got = float(orc.round_bf16(np.array([x]))[0])
        assert got == want, f"round_bf16({x!r}) = {got!r}, want {want!r}"
    rng = np.random.default_rng(40)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 120, 20000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref), "round_bf16 differs from torch's fp32 -> bf16 conversion"


# ------------------------------------------------------------ cache ratio
def pin_cache_ratio_golden(orc):
    """The printed figure: at S=256, N=128 the DART cache is 25% of the
    matched attention cache (75% saving), for any L multiple of S and any P."""
    with open(os.path.join(GOLDEN, "cache_ratio.json")) as f:
        gold = json.load(f)
    for L in (256, 4096, 32768):
        for P in (64, 128):
            r = orc.cache_ratio(L, gold["S"], gold["N"], P)
            assert abs(r - gold["ratio"]) < 1e-15, r
            assert abs((1 - r) - gold["saving"]) < 1e-15
    dart, attn = orc.cache_elements(128 * 256, 256, 128, 64)   # 32K context
    assert (dart, attn) == (1048576, 4194304)


def pin_sma_continue_is_suffix_of_whole(orc):
    """Continuing a sequence after its first k0 chunks reads the same as the
    whole sequence's readout of those tokens (chunked prefill changes where
    the work is split, not what is computed)."""
    d = _inputs(23, B=2, L=20, H=2, G=1, N=3, P=4)
    S, k0 = 4, 2
    dH = orc.chunk_states(d["x"], d["dt"], d["A"], d["Bm"], S)
    whole = orc.sma(d["Q"], d["E"], d["C"], dH, S)
    tail = {k: v[:, k0 * S:] for k, v in d.items() if k in ("Q", "E", "C")}
    got = orc.sma_continue(tail["Q"], tail["E"], tail["C"], dH[:, :, :k0], dH[:, :, k0:], S)
    _close(got, whole[:, k0 * S:], what="continued SMA")


def pin_sma_decayed_no_decay(orc):
    """With A = 0 nothing decays (d = 1) and the decay-included variant is
    the plain SMA."""
    d = _inputs(21, B=1, L=16, H=2, G=1, N=3, P=4, A_zero=True)
    S = 4
    dH = orc.chunk_states(d["x"], d["dt"], d["A"], d["Bm"], S)
    _close(orc.sma_decayed(d["Q"], d["E"], d["C"], dH, d["dt"], d["A"], S),
           orc.sma(d["Q"], d["E"], d["C"], dH, S), what="A=0 decayed SMA")


def pin_sma_decayed_from_recurrence(orc):
    """The decayed memory of chunk c seen from token t is, by linearity, the
    recurrent state at t when only chunk c's tokens feed the recurrence.
    Building keys, values and the softmax from those states by hand (scalar
    loops) must give the decay-included readout (Pith review, major comment
    3: the decay A_{e(c)+1:t} applied to ΔH[c])."""
    d = _inputs(22, B=1, L=12, H=2, G=1, N=3, P=4)
    d["Q"] = d["Q"] * 3.0                      # a peaked softmax
    S = 3
    B, L, H, P = d["x"].shape
    N = d["Bm"].shape[-1]
    M = L // S
    dH = orc.chunk_states(d["x"], d["dt"], d["A"], d["Bm"], S)
    got = orc.sma_decayed(d["Q"], d["E"], d["C"], dH, d["dt"], d["A"], S)
    # states[c][t]: recurrence fed by chunk c alone
    states = []
    for c in range(M):
        xc = np.zeros_like(d["x"])
        xc[:, c * S:(c + 1) * S] = d["x"][:, c * S:(c + 1) * S]
        _, _, st = orc.recurrence(xc, d["dt"], d["A"], d["Bm"], d["C"], keep_states=True)
        states.append(st)
    ref = np.zeros((B, L, H, P))
    for h in range(H):
        for t in range(S, L):
            k = t // S
            sc, vals = [], []
            for c in range(k):
                m = states[c][0, t, h]               # [N, P]
                key = [sum(m[n, p] * d["E"][0, t, h, p] for p in range(P)) for n in range(N)]
                sc.append(sum(d["Q"][0, t, 0, n] * key[n] for n in range(N)) / math.sqrt(N))
                vals.append([sum(d["C"][0, t, 0, n] * m[n, p] for n in range(N))
                             for p in range(P)])
            mx = max(sc)
            w = [math.exp(v - mx) for v in sc]
            for p in range(P):
                ref[0, t, h, p] = sum(wi * v[p] for wi, v in zip(w, vals)) / sum(w)
    _close(got, ref, tol=1e-9, what="decayed SMA vs recurrence states")



# ------------------------------------------------------------ fp8 cache
# The E4M3 format is fixed by the OCP 8-bit floating point specification;
# torch's float8_e4m3fn dtype implements it (conversion from float32 rounds
# to nearest, ties to even) and serves as the library routine.
def _torch_e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def pin_fp8_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.fp8_e4m3_decode(codes)
    ref = _torch_e4m3_values(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "fp8 NaN codes"
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and np.isnan(got).sum() == 2
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin]), "fp8 decode differs from the library"
    # format facts: 1.0, the largest finite value, the smallest subnormal and
    # normal, the largest subnormal, a negative value, negative zero
    for c, v in ((0x38, 1.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x08, 2.0 ** -6),
                 (0x07, 7 * 2.0 ** -9), (0xB8, -1.0), (0xC4, -3.0)):
        assert got[c] == v, (hex(c), got[c], v)
    assert got[0x80] == 0.0 and np.signbit(got[0x80])


def pin_fp8_encode_matches_library(orc):
    rng = np.random.default_rng(81)
    # magnitudes across every binade, the subnormals included
    v = rng.standard_normal(60000) * np.exp2(rng.uniform(-13.0, 8.7, 60000))
    # every midpoint between neighbouring finite values (ties), and the
    # values themselves
    fin = np.sort(np.unique(_torch_e4m3_values(np.arange(0x7F, dtype=np.uint8))))
    mids = 0.5 * (fin[1:] + fin[:-1])
    v = np.concatenate([v, fin, -fin, mids, -mids, [0.0, -0.0, 2.0 ** -11, -(2.0 ** -11)]])
    v = v[np.abs(v) <= 448.0].astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.fp8_e4m3_encode(v.astype(np.float64))
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"fp8 encode differs at {v[bad[:4]]}: {got[bad[:4]]} vs {ref[bad[:4]]}"
    # ties go to the even mantissa
    assert orc.fp8_e4m3_encode(np.array([1.0625, 1.1875, 1.5 * 2.0 ** -9])).tolist() == [
        0x38, 0x3A, 0x02]


def pin_fp8_memory_scale(orc):
    rng = np.random.default_rng(82)
    for mag in (1e-30, 3e-7, 0.02, 1.0, 7.5, 4e5, 1e30):
        mem = rng.standard_normal((6, 5)) * mag
        s = orc.fp8_memory_scale(mem)
        m, e = math.frexp(s)
        assert m == 0.5, "scale is not a power of two"
        top = np.max(np.abs(mem)) / s
        assert 128.0 <= top < 256.0, (mag, top)
        codes, s2 = orc.fp8_quantize_memory(mem)
        assert s2 == s and codes.shape == mem.shape and codes.dtype == np.uint8
        deq = _torch_e4m3_values(codes) * s
        # half a grid step: 1/16 of the magnitude in the normal range,
        # 2^-10 of the scale among the subnormals
        assert np.all(np.abs(deq - mem) <= np.maximum(np.abs(mem) / 16.0, s * 2.0 ** -10))
    pow2 = np.zeros((3, 3))
    pow2[1, 2] = -2.0 ** 5
    assert orc.fp8_memory_scale(pow2) * 128.0 == 2.0 ** 5
    assert orc.fp8_memory_scale(np.zeros((4, 4))) == 1.0


def pin_decode_step_fp8_reads_the_dequantised_cache(orc):
    """The fp8 decode step equals the float decode step over the memories the
    codes stand for (dequantised here with the library), and a memory it
    appends is its f64 counterpart within the rounding bound."""
    rng = np.random.default_rng(83)
    B, H, G, N, P, S, Mx = 2, 2, 1, 4, 3, 5, 4
    codes = rng.integers(0, 256, (B, H, Mx, N, P)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x30  # no NaN codes
    scales = np.exp2(rng.integers(-9, 4, (B, H, Mx))).astype(np.float64)
    cache = _torch_e4m3_values(codes) * scales[..., None, None]
    h = rng.standard_normal((B, H, N, P))
    dHc = rng.standard_normal((B, H, N, P))
    state = {"h": h, "dH_cur": dHc, "n_chunks": np.array([3, 2]), "pos": np.array([S - 1, 1])}
    x, E = rng.standard_normal((B, H, P)), rng.standard_normal((B, H, P))
    dt = np.full((B, H), 0.1)
    A = -np.ones(H)
    Bm, C, Q = (rng.standard_normal((B, G, N)) for _ in range(3))
    y8, new8 = orc.decode_step_fp8(dict(state, codes=codes, scales=scales), x, dt, A, Bm, C, Q,
                                   E, 0.7, S)
    yf, newf = orc.decode_step(dict(state, cache=cache), x, dt, A, Bm, C, Q, E, 0.7, S,
                               cache_bf16=False)
    _close(y8, yf, 1e-12, "fp8 decode y")
    _close(new8["h"], newf["h"], 1e-12, "fp8 decode h")
    assert list(new8["n_chunks"]) == [4, 2] and list(new8["pos"]) == [0, 2]
    # sequence 0 appended memory 3; everything else is untouched
    app = _torch_e4m3_values(new8["codes"][0, :, 3]) * new8["scales"][0, :, 3, None, None]
    ref = newf["cache"][0, :, 3]
    assert np.all(np.abs(app - ref) <= np.abs(ref) / 16.0 + 2.0 ** -10 * np.max(np.abs(ref)))
    for hh in range(H):
        top = np.max(np.abs(ref[hh])) / new8["scales"][0, hh, 3]
        assert 128.0 <= top < 256.0
    keep = np.ones((B, H, Mx), dtype=bool)
    keep[0, :, 3] = False
    assert np.array_equal(new8["codes"][keep], codes[keep])
    assert np.array_equal(new8["scales"][keep], scales[keep])


# ------------------------------------------------------------ backward
def _fd_grad(f, arr, eps=1e-6):
    """Central finite differences of the scalar f() with respect to every
    element of arr (modified in place and restored)."""
    g = np.zeros_like(arr)
    for idx in np.ndindex(arr.shape):
        a0 = arr[idx]
        arr[idx] = a0 + eps
        fp = f()
        arr[idx] = a0 - eps
        fm = f()
        arr[idx] = a0
        g[idx] = (fp - fm) / (2 * eps)
    return g


def pin_sma_backward_finite_differences(orc):
    """Every gradient of Σ do·o against central differences of the forward
    readout (three chunks, heads sharing a group, sharpened scores)."""
    rng = np.random.default_rng(91)
    B, L, H, G, N, P, S = 1, 12, 4, 2, 3, 2, 4
    Q = rng.standard_normal((B, L, G, N)) * 2.0
    E = rng.standard_normal((B, L, H, P))
    C = rng.standard_normal((B, L, G, N))
    dH = rng.standard_normal((B, H, L // S, N, P))
    do = rng.standard_normal((B, L, H, P))
    grads = orc.sma_backward(Q, E, C, dH, S, do)

    def loss():
        return float(np.sum(do * orc.sma(Q, E, C, dH, S)))

    for name, arr, g in zip(("dQ", "dE", "dC", "ddH"), (Q, E, C, dH), grads):
        num = _fd_grad(loss, arr)
        _close(g, num, 1e-7 * max(1.0, float(np.max(np.abs(num)))), f"sma backward {name}")


def pin_sma_backward_single_memory(orc):
    """Two chunks: the second chunk's tokens see one memory, so α = 1 and
    o_t = ΔH[0]ᵀC_t; then dQ = dE = 0, dC_t = ΔH[0]·do_t and
    dΔH[0] = Σ_t C_t do_tᵀ (first-chunk tokens contribute nothing)."""
    rng = np.random.default_rng(92)
    B, L, H, G, N, P, S = 2, 10, 1, 1, 4, 3, 5
    Q = rng.standard_normal((B, L, G, N))
    E = rng.standard_normal((B, L, H, P))
    C = rng.standard_normal((B, L, G, N))
    dH = rng.standard_normal((B, H, 2, N, P))
    do = rng.standard_normal((B, L, H, P))
    dQ, dE, dC, ddH = orc.sma_backward(Q, E, C, dH, S, do)
    _close(dQ, np.zeros_like(dQ), 1e-12, "single memory dQ")
    _close(dE, np.zeros_like(dE), 1e-12, "single memory dE")
    for b in range(B):
        for t in range(L):
            want = dH[b, 0, 0] @ do[b, t, 0] if t >= S else np.zeros(N)
            _close(dC[b, t, 0], want, 1e-12, "single memory dC")
        want = sum(np.outer(C[b, t, 0], do[b, t, 0]) for t in range(S, L))
        _close(ddH[b, 0, 0], want, 1e-12, "single memory ddH[0]")
        _close(ddH[b, 0, 1], np.zeros((N, P)), 1e-12, "last memory unread")


def pin_gated_backward(orc):
    rng = np.random.default_rng(93)
    dy, o, ys = (rng.standard_normal((2, 6, 3, 4)) for _ in range(3))
    g = np.array([0.3])
    dys, do, dg = orc.gated_backward(dy, o, g[0])
    _close(dys, dy, 0.0, "dy_ssd")
    _close(do, 0.3 * dy, 1e-15, "do")
    num = _fd_grad(lambda: float(np.sum(dy * orc.gated_output(ys, o, g[0]))), g)
    _close(np.array([dg]), num, 1e-7, "dg")


def pin_sma_logsumexp(orc):
    """One visible memory: the normaliser is the score itself; Q = 0 (all
    scores 0): it is log k for chunk k."""
    rng = np.random.default_rng(94)
    B, L, H, G, N, P, S = 1, 12, 2, 1, 3, 2, 4
    Q = rng.standard_normal((B, L, G, N))
    E = rng.standard_normal((B, L, H, P))
    C = rng.standard_normal((B, L, G, N))
    dH = rng.standard_normal((B, H, 3, N, P))
    lse = orc.sma_logsumexp(Q, E, C, dH, S)
    for h in range(H):
        for t in range(S, 2 * S):
            want = Q[0, t, 0] @ (dH[0, h, 0] @ E[0, t, h]) / math.sqrt(N)
            _close(lse[0, h, t], want, 1e-12, "one-memory normaliser")
    lse0 = orc.sma_logsumexp(np.zeros_like(Q), E, C, dH, S)
    for t in range(L):
        want = 0.0 if t < S else math.log(t // S)
        _close(lse0[0, :, t], np.full(H, want), 1e-12, "uniform normaliser")


def pin_ssd_backward_finite_differences(orc):
    """Every gradient of the scan (dx, ddt, dA, dB, dC, dh0) against central
    differences of Σ dy·y_ssd + Σ ddH·ΔH + Σ dh_final·h_final computed with
    the forward functions (two chunks, two heads sharing B/C, initial
    state)."""
    rng = np.random.default_rng(95)
    B, L, H, G, N, P, S = 1, 8, 2, 1, 3, 2, 4
    M = L // S
    x = rng.standard_normal((B, L, H, P))
    dt = rng.uniform(0.1, 0.6, (B, L, H))
    A = -rng.uniform(0.5, 2.0, H)
    Bm, C = rng.standard_normal((B, L, G, N)), rng.standard_normal((B, L, G, N))
    h0 = rng.standard_normal((B, H, N, P))
    dy = rng.standard_normal((B, L, H, P))
    ddH = rng.standard_normal((B, H, M, N, P))
    dhf = rng.standard_normal((B, H, N, P))
    g = orc.ssd_backward(x, dt, A, Bm, C, S, dy, ddH, dhf, h0)

    def loss():
        dH = orc.chunk_states(x, dt, A, Bm, S)
        H_in = orc.state_pass(dH, dt, A, S, h0)
        y = orc.chunk_output(x, dt, A, Bm, C, H_in, S)
        return float(np.sum(dy * y) + np.sum(ddH * dH) + np.sum(dhf * H_in[:, :, M]))

    for name, arr in (("dx", x), ("ddt", dt), ("dA", A), ("dB", Bm), ("dC", C), ("dh0", h0)):
        num = _fd_grad(loss, arr)
        _close(g[name], num, 1e-7 * max(1.0, float(np.max(np.abs(num)))), f"ssd backward {name}")

ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
