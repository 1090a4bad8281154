"""Seeded synthetic inputs for the DART hot path.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic.  Both the HIP path (through the tests and ``bench.py``)
and the CPU oracle consume what it returns.

Recipe (per prefill draw), numpy ``default_rng(seed)`` (PCG64), drawn in the
order A, dt, x, Bm, C, Q, E, each in C order:

* A  = -exp(U[0, ln 16])                      [H]          float32
* dt = exp(U[ln 1e-3, ln 1e-1])               [B, L, H]    float32
* x  ~ N(0, 1)                                [B, L, H, P] io dtype
* Bm, C ~ N(0, 1)/sqrt(N)                     [B, L, G, N] io dtype
* Q  ~ qscale·N(0, 1)/sqrt(N)                 [B, L, G, N] io dtype
* E  ~ N(0, 1)/sqrt(P)                        [B, L, H, P] io dtype

fp64 draws are cast with torch's round-to-nearest-even; the oracle receives
the cast values upcast to fp64 (``as_f64``), so parity measures computation
error only.
"""

import math

import numpy as np
import torch

_BLOCK = 1 << 24  # draw large tensors in blocks of this many values


def _cast(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype)


def _normal(rng, shape, scale, dtype):
    """N(0, scale²) values of ``shape`` drawn in C order, cast to ``dtype``."""
    total = int(np.prod(shape))
    out = torch.empty(total, dtype=dtype)
    done = 0
    while done < total:
        n = min(_BLOCK, total - done)
        out[done:done + n] = _cast(rng.standard_normal(n) * scale, dtype)
        done += n
    return out.view(*shape)


def draw_prefill(seed, batch, seqlen, nheads, ngroups, dstate, headdim,
                 io=torch.bfloat16, qscale=1.0):
    """Prefill inputs as CPU tensors: dict with A, dt, x, Bm, C, Q, E."""
    if nheads % ngroups:
        raise ValueError("nheads must be a multiple of ngroups")
    rng = np.random.default_rng(seed)
    B, L, H, G, N, P = batch, seqlen, nheads, ngroups, dstate, headdim
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=H))
    dt = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=(B, L, H)))
    out = {"A": _cast(A, torch.float32), "dt": _cast(dt, torch.float32)}
    out["x"] = _normal(rng, (B, L, H, P), 1.0, io)
    out["Bm"] = _normal(rng, (B, L, G, N), 1.0 / math.sqrt(N), io)
    out["C"] = _normal(rng, (B, L, G, N), 1.0 / math.sqrt(N), io)
    out["Q"] = _normal(rng, (B, L, G, N), qscale / math.sqrt(N), io)
    out["E"] = _normal(rng, (B, L, H, P), 1.0 / math.sqrt(P), io)
    return out


def draw_decode_token(seed, batch, nheads, ngroups, dstate, headdim,
                      io=torch.bfloat16, qscale=1.0):
    """One new token per sequence: dict with A [H], dt [B,H], x [B,H,P],
    Bm/C/Q [B,G,N], E [B,H,P] (same distributions as the prefill draw)."""
    rng = np.random.default_rng(seed)
    B, H, G, N, P = batch, nheads, ngroups, dstate, headdim
    A = -np.exp(rng.uniform(0.0, math.log(16.0), size=H))
    dt = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=(B, H)))
    out = {"A": _cast(A, torch.float32), "dt": _cast(dt, torch.float32)}
    out["x"] = _normal(rng, (B, H, P), 1.0, io)
    out["Bm"] = _normal(rng, (B, G, N), 1.0 / math.sqrt(N), io)
    out["C"] = _normal(rng, (B, G, N), 1.0 / math.sqrt(N), io)
    out["Q"] = _normal(rng, (B, G, N), qscale / math.sqrt(N), io)
    out["E"] = _normal(rng, (B, H, P), 1.0 / math.sqrt(P), io)
    return out


def draw_state(seed, shape, std, dtype, device="cpu"):
    """N(0, std²) tensor of ``shape`` (decode cache, h, ΔH_cur).  On a GPU
    device the values come from torch's device generator seeded with
    ``seed`` (a 4 GiB cache is too slow to draw on the host); on the CPU from
    numpy as above."""
    if torch.device(device).type == "cpu":
        return _normal(np.random.default_rng(seed), shape, std, dtype)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    step = 1 << 28
    for i in range(0, flat.numel(), step):
        n = min(step, flat.numel() - i)
        flat[i:i + n] = (torch.randn(n, generator=gen, device=device,
                                     dtype=torch.float32) * std).to(dtype)
    return out


def as_f64(t):
    """Exact fp64 numpy copy of a tensor's values (any device, any dtype)."""
    return t.detach().to("cpu", torch.float64).numpy()
