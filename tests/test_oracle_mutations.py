"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check
that at least one pin catches each: the pins are strong enough to trust."""
import importlib.util
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "dart_oracle.py")

# (name, original text, mutated text): each text occurs in the oracle source
MUTATIONS = [
    ("decay dropped in recurrence",
     "h = a[:, :, None, None] * h + inp\n        y[:, t]",
     "h = h + inp\n        y[:, t]"),
    ("input term without dt",
     "inp = dt[:, t, :, None, None] * Bh[:, t, :, :, None] * x[:, t, :, None, :]",
     "inp = Bh[:, t, :, :, None] * x[:, t, :, None, :]"),
    ("chunk decay includes own token",
     "dtc[:, i + 1:, :].sum(axis=1)", "dtc[:, i:, :].sum(axis=1)"),
    ("chunk weight missing dt",
     "w = np.exp(tail * A[None, None, :]) * dtc", "w = np.exp(tail * A[None, None, :])"),
    ("state pass sign",
     "* H_in[:, :, c] + dH[:, :, c]", "* H_in[:, :, c] - dH[:, :, c]"),
    ("state pass without decay",
     "H_in[:, :, c + 1] = decay[:, :, None, None] * H_in[:, :, c]",
     "H_in[:, :, c + 1] = H_in[:, :, c]"),
    ("inter-chunk decay sign",
     "np.exp(cs * A)[..., None] * inter", "np.exp(-cs * A)[..., None] * inter"),
    ("intra-chunk anti-causal",
     "causal = np.tril(np.ones((S, S), dtype=bool))",
     "causal = np.triu(np.ones((S, S), dtype=bool))"),
    ("intra-chunk weight missing dt",
     "wts = cb * decay * dtk[:, None, :, :]", "wts = cb * decay"),
    ("decayed SMA: decay starts at the chunk's last token",
     "ends = np.arange(k) * S + (S - 1)", "ends = np.arange(k) * S + (S - 2)"),
    ("decayed SMA: decay on the score only",
     "vals = d[:, :, None] * np.einsum", "vals = 1.0 * np.einsum"),
    ("decayed SMA: decay on the value only",
     "scores = d * np.einsum(\"tn,tcn->tc\"", "scores = 1.0 * np.einsum(\"tn,tcn->tc\""),
    ("score scale sqrt(P)",
     'scores = np.einsum("tn,tcn->tc", Qh[b, ts, h], keys) / math.sqrt(N)',
     'scores = np.einsum("tn,tcn->tc", Qh[b, ts, h], keys) / math.sqrt(P)'),
    ("decode score scale sqrt(P)",
     "scores = keys @ Qh[b, hh] / math.sqrt(N)", "scores = keys @ Qh[b, hh] / math.sqrt(P)"),
    ("decode value read with the query",
     'vals = np.einsum("n,cnp->cp", Ch[b, hh], mem)', 'vals = np.einsum("n,cnp->cp", Qh[b, hh], mem)'),
    ("query replaced by C",
     'scores = np.einsum("tn,tcn->tc", Qh[b, ts, h], keys)',
     'scores = np.einsum("tn,tcn->tc", Ch[b, ts, h], keys)'),
    ("own chunk visible",
     "mem = dH[b, h, :k]                                  # [k,N,P]",
     "mem = dH[b, h, :k + 1]                              # [k,N,P]"),
    ("value decoded with E instead of C",
     'vals = np.einsum("tn,cnp->tcp", Ch[b, ts, h], mem)',
     'vals = np.einsum("tn,cnp->tcp", Qh[b, ts, h], mem)'),
    ("softmax sign",
     "e = np.exp(s - m)", "e = np.exp(m - s)"),
    ("convex gate",
     "return _f64(y_ssd) + float(g) * _f64(o)",
     "return (1.0 - float(g)) * _f64(y_ssd) + float(g) * _f64(o)"),
    ("groups interleaved",
     "return np.arange(H) // (H // G)", "return np.arange(H) % G"),
    ("decode closes chunk one token late",
     "if pos[b] == S - 1:", "if pos[b] == S:"),
    ("decode skips the SSM decay of the chunk memory",
     "dHc = a[:, :, None, None] * dHc + inp", "dHc = dHc + inp"),
    ("fp8 exponent bias 8",
     "normal = (1.0 + mant / 8.0) * np.exp2(field - 7.0)",
     "normal = (1.0 + mant / 8.0) * np.exp2(field - 8.0)"),
    ("bf16 rounding truncates",
     "r = np.rint(a / step) * step", "r = np.trunc(a / step) * step"),
    ("bf16 rounding ties away from zero",
     "r = np.rint(a / step) * step", "r = np.copysign(np.floor(np.abs(a / step) + 0.5), a) * step"),
    ("bf16 grid one bit too fine",
     "step = np.ldexp(1.0, np.maximum(e - 8, -133))", "step = np.ldexp(1.0, np.maximum(e - 9, -133))"),
    ("fp8 encoding truncates",
     "r = np.round(a / step) * step", "r = np.floor(a / step) * step"),
    ("fp8 subnormal grid too fine",
     "e = np.maximum(E - 1, -6)", "e = np.maximum(E - 1, -7)"),
    ("fp8 scale one binade too high",
     "return math.ldexp(1.0, max(E - 8, -126))", "return math.ldexp(1.0, max(E - 7, -126))"),
    ("fp8 decode step ignores the scales",
     'plain["cache"] = fp8_dequantize(codes, scales)',
     'plain["cache"] = fp8_e4m3_decode(codes)'),
    ("SMA backward drops the softmax centring",
     "ds = alpha * (dalpha - np.sum(alpha * dalpha, axis=1, keepdims=True))",
     "ds = alpha * dalpha"),
    ("SMA backward key gradient without the score scale",
     "dK = ds[:, :, None] * Qt[:, None, :] * rs", "dK = ds[:, :, None] * Qt[:, None, :]"),
    ("SMA backward value gradient from the query",
     "dCh[b, ts, h] += np.einsum(\"cnp,tcp->tn\", mem, dV)",
     "dCh[b, ts, h] += np.einsum(\"cnp,tcp->tn\", mem, dV) * 0.5"),
    ("SMA backward drops the key term of the memory gradient",
     "ddH[b, h, :k] += (np.einsum(\"tcn,tp->cnp\", dK, Et)",
     "ddH[b, h, :k] += (0.0 * np.einsum(\"tcn,tp->cnp\", dK, Et)"),
    ("gate gradient scaled by g",
     "return dy.copy(), float(g) * dy, float(np.sum(dy * o))",
     "return dy.copy(), float(g) * dy, float(g) * float(np.sum(dy * o))"),
    ("scan backward: state gradient passed back without the chunk decay",
     "Gs = np.exp(u[-1]) * Gs + dHin[c]", "Gs = Gs + dHin[c]"),
    ("scan backward: intra term misses the dt factor's own gradient",
     "ddt[b, ts, h] += np.sum(dw * cb * dec, axis=0)", "ddt[b, ts, h] += 0.0"),
    ("scan backward: log-decay gradient summed over earlier tokens",
     "ddt[b, ts, h] += a * np.cumsum(du[ts][::-1])[::-1]", "ddt[b, ts, h] += a * np.cumsum(du[ts])"),
    ("scan backward: state gradient of the output without exp(u)",
     "dHin[k] += (eu[:, None] * Ck).T @ dyk", "dHin[k] += Ck.T @ dyk"),
    ("cache ratio counts keys only",
     "return (L // S) * N * P, 2 * L * P", "return (L // S) * N * P, L * P"),
]


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("dart_oracle_mutant")
    exec(compile(src.replace(old, new), "dart_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_some_pin_catches(name, old, new):
    mutant = _load_mutant(old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin catches mutation '{name}'"
