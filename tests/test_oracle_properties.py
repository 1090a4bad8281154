"""Property checks of the oracle over many tiny random shapes (hypothesis):
the chunked scan equals the sequential recurrence for any chunking, and the
vectorised SMA equals the scalar loops."""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle


@st.composite
def shapes(draw):
    S = draw(st.sampled_from([1, 2, 3, 4, 8]))
    M = draw(st.integers(1, 4))
    G = draw(st.integers(1, 2))
    H = G * draw(st.integers(1, 2))
    return dict(B=draw(st.integers(1, 2)), S=S, M=M, H=H, G=G,
                N=draw(st.integers(1, 4)), P=draw(st.integers(1, 4)),
                seed=draw(st.integers(0, 2**31 - 1)))


def _draw(sh):
    rng = np.random.default_rng(sh["seed"])
    B, L, H, G, N, P = sh["B"], sh["S"] * sh["M"], sh["H"], sh["G"], sh["N"], sh["P"]
    return dict(
        A=-np.exp(rng.uniform(0, np.log(16), H)),
        dt=np.exp(rng.uniform(np.log(1e-3), np.log(0.5), (B, L, H))),
        x=rng.standard_normal((B, L, H, P)), Bm=rng.standard_normal((B, L, G, N)),
        C=rng.standard_normal((B, L, G, N)), Q=3 * rng.standard_normal((B, L, G, N)),
        E=rng.standard_normal((B, L, H, P)), h0=rng.standard_normal((B, H, N, P)))


@settings(max_examples=60, deadline=None)
@given(shapes())
def test_chunked_scan_equals_recurrence(sh):
    d = _draw(sh)
    S = sh["S"]
    y_rec, h_rec, _ = oracle.recurrence(d["x"], d["dt"], d["A"], d["Bm"], d["C"], h0=d["h0"])
    dH = oracle.chunk_states(d["x"], d["dt"], d["A"], d["Bm"], S)
    H_in = oracle.state_pass(dH, d["dt"], d["A"], S, d["h0"])
    y = oracle.chunk_output(d["x"], d["dt"], d["A"], d["Bm"], d["C"], H_in, S)
    np.testing.assert_allclose(y, y_rec, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(H_in[:, :, -1], h_rec, rtol=1e-9, atol=1e-11)


@settings(max_examples=40, deadline=None)
@given(shapes())
def test_sma_vectorised_equals_loops(sh):
    d = _draw(sh)
    dH = np.random.default_rng(sh["seed"] + 1).standard_normal(
        (sh["B"], sh["H"], sh["M"], sh["N"], sh["P"]))
    np.testing.assert_allclose(
        oracle.sma(d["Q"], d["E"], d["C"], dH, sh["S"]),
        oracle.sma_bruteforce(d["Q"], d["E"], d["C"], dH, sh["S"]), rtol=1e-9, atol=1e-11)
