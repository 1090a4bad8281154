"""Plain fp64 CPU oracle for the DART hot path.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
in ``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module.  It shares no code, headers, helpers or tables with the HIP
library; the HIP path never imports it.  Every function is written for a
reader to check against the pages by eye: loops and numpy primitives (einsum,
cumsum, exp), fp64 throughout, no blocking or fusion beyond what the
definition states.

Sources (cited by page and section; the pages print no code):

* [abstract]  DART abstract (aipentium and mlsanity pages): DART keeps the
  per-chunk state contributions that the Mamba-2 chunked scan produces,
  decodes token-conditioned keys and values from them, runs state-memory
  attention (SMA) over them and adds the result to the Mamba-2 output through
  a gated residual; the cache saving is 75% at S=256, N=128.
* [pith-core]  Pith review of DART, "Core claim": values read as C_t·ΔH[c],
  keys as ΔH[c]·E_t, attention over chunk-level pairs, readout added through a
  zero-initialised scalar gate.
* [pith-carries]  Pith review, "What carries the argument": ΔH[c] is the
  N×P contribution of chunk c to the chunk-boundary state (key axis N, value
  axis P); query Q_t.
* [pith-maj3]  Pith review, referee major comment 3 (paper §3 Eq. 8): the
  readouts use the raw ΔH[c], with no inter-chunk decay applied; the referee
  asks for the variant with the decay A_{e(c)+1:t} applied as an ablation.
* [pith-eq14]  Pith review, minor comment 1 and circularity check (paper §4
  Eq. 14): per head the DART cache holds M·N·P values against 2·L·P for a
  token-level attention layer.
* [pith-axioms]  Pith review, axiom ledger: SSD writes Mamba-2 as structured
  causal attention (paper Eq. 4); the chunked scan splits the output into
  intra-chunk and inter-chunk terms and yields ΔH[c].
* [pith-ext]  Pith review, "Where Pith is reading between the lines"
  (editorial extensions): since SMA reads the scan's own ΔH, the memory cache
  could be combined with cache quantisation.

Readings where the pages are silent:
* Mamba-2 recurrence h_t = exp(dt_t·A)·h_{t-1} + dt_t·B_t x_tᵀ, y_t = C_tᵀ h_t
  (zero-order-hold discretisation; D skip, gating and norm are absent).
* A token in chunk k attends over the completed chunks c < k only; tokens of
  chunk 0 get a zero SMA readout.
* Score scale 1/sqrt(N) (N is the key dimension).
* Gate: y = y_ssd + g·o with g a raw scalar.
* B, C and Q are shared by groups of H/G consecutive heads; x, E, dt per head.
* Quantised cache [pith-ext] (the pages name no format): each memory is kept
  as OCP FP8 E4M3 codes times one power-of-two scale per memory, see
  :func:`fp8_quantize_memory`.

Layouts (row-major numpy arrays, float64):
  x, E   [B, L, H, P]      dt [B, L, H]      A [H]
  Bm, C, Q [B, L, G, N]    ΔH [B, H, M, N, P]   H_in [B, H, M+1, N, P]
"""

import math

import numpy as np

__all__ = [
    "group_of_head",
    "recurrence",
    "chunk_states",
    "state_pass",
    "chunk_output",
    "sma",
    "sma_bruteforce",
    "sma_decayed",
    "sma_continue",
    "gated_output",
    "prefill",
    "decode_step",
    "cache_elements",
    "cache_ratio",
    "round_bf16",
    "fp8_e4m3_decode",
    "fp8_e4m3_encode",
    "fp8_memory_scale",
    "fp8_quantize_memory",
    "fp8_dequantize",
    "decode_step_fp8",
    "sma_backward",
    "gated_backward",
    "sma_logsumexp",
    "ssd_backward",
]


def group_of_head(H, G):
    """Head h reads the B/C/Q group h // (H // G) (reading: heads grouped
    contiguously, as in Mamba-2's grouped B/C)."""
    if G <= 0 or H % G:
        raise ValueError(f"heads {H} not divisible by groups {G}")
    return np.arange(H) // (H // G)


def _per_head(T, H):
    """Expand a grouped [B, L, G, N] tensor to [B, L, H, N]."""
    return np.asarray(T, dtype=np.float64)[:, :, group_of_head(H, T.shape[2]), :]


def _f64(a):
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# O2 - sequential recurrence (ground truth of the SSM branch)
# --------------------------------------------------------------------------
def recurrence(x, dt, A, Bm, C, h0=None, keep_states=False):
    """Token-by-token Mamba-2 recurrence [pith-core: Mamba-2 reads values
    from its state as C_t H_t; pith-axioms].

    a_t = exp(dt_t·A_h);  h_t = a_t·h_{t-1} + dt_t·B_t x_tᵀ;  y_t = C_tᵀ h_t.
    Returns (y [B,L,H,P], h_final [B,H,N,P], states [B,L,H,N,P] or None).
    """
    x, dt, A = _f64(x), _f64(dt), _f64(A)
    Bsz, L, H, P = x.shape
    Bh, Ch = _per_head(Bm, H), _per_head(C, H)
    N = Bh.shape[-1]
    h = np.zeros((Bsz, H, N, P)) if h0 is None else _f64(h0).copy()
    y = np.empty((Bsz, L, H, P))
    states = np.empty((Bsz, L, H, N, P)) if keep_states else None
    for t in range(L):
        a = np.exp(dt[:, t, :] * A[None, :])                      # [B,H]
        inp = dt[:, t, :, None, None] * Bh[:, t, :, :, None] * x[:, t, :, None, :]
        h = a[:, :, None, None] * h + inp
        y[:, t] = np.einsum("bhn,bhnp->bhp", Ch[:, t], h)
        if keep_states:
            states[:, t] = h
    return y, h, states


# --------------------------------------------------------------------------
# O3 - chunk state contributions ΔH[c]
# --------------------------------------------------------------------------
def chunk_states(x, dt, A, Bm, S):
    """ΔH[c] = Σ_{i in c} exp(A·Σ_{j=i+1}^{end(c)} dt_j)·dt_i·B_i x_iᵀ
    [pith-carries: contribution of chunk c to the chunk-boundary state;
    abstract].  The decay from token i to the chunk end is a direct segment
    sum of the later dt's of the chunk (not a cumsum difference).
    Returns ΔH [B,H,M,N,P]."""
    x, dt, A = _f64(x), _f64(dt), _f64(A)
    Bsz, L, H, P = x.shape
    if L % S:
        raise ValueError("L must be a multiple of S")
    M = L // S
    Bh = _per_head(Bm, H)
    N = Bh.shape[-1]
    dH = np.zeros((Bsz, H, M, N, P))
    for c in range(M):
        sl = slice(c * S, (c + 1) * S)
        dtc = dt[:, sl, :]                                          # [B,S,H]
        tail = np.zeros_like(dtc)
        for i in range(S):
            tail[:, i, :] = dtc[:, i + 1:, :].sum(axis=1)
        w = np.exp(tail * A[None, None, :]) * dtc                   # [B,S,H]
        dH[:, :, c] = np.einsum("bsh,bshn,bshp->bhnp", w, Bh[:, sl], x[:, sl])
    return dH


# --------------------------------------------------------------------------
# O4 - inter-chunk state passing
# --------------------------------------------------------------------------
def state_pass(dH, dt, A, S, h0=None):
    """H_in[0] = h0 (zero by default); H_in[c+1] = exp(A·Σ_{j in c} dt_j)·H_in[c]
    + ΔH[c]  [pith-axioms: inter-chunk term of the chunked scan].
    Returns H_in [B,H,M+1,N,P]; H_in[:, :, M] is the final state."""
    dH, dt, A = _f64(dH), _f64(dt), _f64(A)
    Bsz, H, M, N, P = dH.shape
    H_in = np.zeros((Bsz, H, M + 1, N, P))
    if h0 is not None:
        H_in[:, :, 0] = _f64(h0)
    for c in range(M):
        total = dt[:, c * S:(c + 1) * S, :].sum(axis=1)             # [B,H]
        decay = np.exp(total * A[None, :])
        H_in[:, :, c + 1] = decay[:, :, None, None] * H_in[:, :, c] + dH[:, :, c]
    return H_in


# --------------------------------------------------------------------------
# O5 - native chunk output (quadratic SSD form)
# --------------------------------------------------------------------------
def chunk_output(x, dt, A, Bm, C, H_in, S):
    """y_t = Σ_{j in k, j<=t} (C_t·B_j)·exp(A·Σ_{l=j+1}^{t} dt_l)·dt_j·x_j
           + exp(A·Σ_{l=kS}^{t} dt_l)·C_tᵀ H_in[k]
    for token t of chunk k  [pith-axioms: SSD as structured causal attention
    (paper Eq. 4), split into intra- and inter-chunk terms].
    Returns y_ssd [B,L,H,P]."""
    x, dt, A = _f64(x), _f64(dt), _f64(A)
    Bsz, L, H, P = x.shape
    M = L // S
    Bh, Ch = _per_head(Bm, H), _per_head(C, H)
    y = np.empty((Bsz, L, H, P))
    causal = np.tril(np.ones((S, S), dtype=bool))                   # j <= t
    for k in range(M):
        sl = slice(k * S, (k + 1) * S)
        dtk = dt[:, sl, :]                                          # [B,S,H]
        cs = np.cumsum(dtk, axis=1)                                 # Σ_{l=kS}^{t}
        seg = cs[:, :, None, :] - cs[:, None, :, :]                 # [B,t,j,H] = Σ_{l=j+1}^{t}
        seg = np.where(causal[None, :, :, None], seg, 0.0)
        decay = np.where(causal[None, :, :, None], np.exp(seg * A), 0.0)
        cb = np.einsum("bthn,bjhn->btjh", Ch[:, sl], Bh[:, sl])
        wts = cb * decay * dtk[:, None, :, :]
        intra = np.einsum("btjh,bjhp->bthp", wts, x[:, sl])
        inter = np.einsum("bthn,bhnp->bthp", Ch[:, sl], H_in[:, :, k])
        y[:, sl] = intra + np.exp(cs * A)[..., None] * inter
    return y


def ssd_backward(x, dt, A, Bm, C, S, dy, ddH=None, dh_final=None, h0=None):
    """Gradients through the chunked scan (reverse of :func:`chunk_states`,
    :func:`state_pass` and :func:`chunk_output`) [pith-axioms;
    pith-carries].  Upstream gradients: dy of y_ssd [B,L,H,P], ddH of the
    chunk memories [B,H,M,N,P] (e.g. from SMA) and dh_final of the final
    state [B,H,N,P]; the last two default to zero.

    With u_t = A·Σ_{l=kS}^{t} dt_l (the log-decay from the start of token
    t's chunk k to t) and U_c = u at the last token of chunk c:
      intra  y_t += Σ_{j<=t} (C_t·B_j)·exp(u_t − u_j)·dt_j·x_j
      inter  y_t += exp(u_t)·C_tᵀH_in[k]
      state  H_in[c+1] = exp(U_c)·H_in[c] + ΔH[c]
      memory ΔH[c] = Σ_i exp(U_c − u_i)·dt_i·B_i x_iᵀ
    each term is differentiated in turn, the state recursion last chunk
    first, and the log-decays u pass their gradient to dt and A at the end.
    B and C are shared by the heads of a group, so dB and dC are summed over
    them.  Returns a dict with dx [B,L,H,P], ddt [B,L,H], dA [H],
    dB [B,L,G,N], dC [B,L,G,N] and dh0 [B,H,N,P]."""
    x, dt, A, dy = _f64(x), _f64(dt), _f64(A), _f64(dy)
    Bsz, L, H, P = x.shape
    M = L // S
    G = np.shape(Bm)[2]
    Bh, Ch = _per_head(Bm, H), _per_head(C, H)
    N = Bh.shape[-1]
    H_in = state_pass(chunk_states(x, dt, A, Bm, S), dt, A, S, h0)
    dx, ddt, dA = np.zeros_like(x), np.zeros_like(dt), np.zeros(H)
    dBh, dCh = np.zeros((Bsz, L, H, N)), np.zeros((Bsz, L, H, N))
    dh0 = np.zeros((Bsz, H, N, P))
    lower = np.tril(np.ones((S, S), dtype=bool))        # pairs j <= t of a chunk
    for b in range(Bsz):
        for h in range(H):
            a = A[h]
            du = np.zeros(L)                    # ∂loss/∂u_t
            dHin = np.zeros((M + 1, N, P))      # ∂loss/∂H_in[c] through the outputs
            if dh_final is not None:
                dHin[M] = _f64(dh_final)[b, h]
            chunks = []
            for k in range(M):
                ts = np.arange(k * S, (k + 1) * S)
                xk, Bk, Ck = x[b, ts, h], Bh[b, ts, h], Ch[b, ts, h]
                dyk, dtk = dy[b, ts, h], dt[b, ts, h]
                u = a * np.cumsum(dtk)
                chunks.append((ts, xk, Bk, dtk, u))
                # intra-chunk term
                dec = np.where(lower, np.exp(np.where(lower, u[:, None] - u[None, :], 0.0)), 0.0)
                cb = Ck @ Bk.T                                      # [t,j]
                dx[b, ts, h] += (cb * dec * dtk[None, :]).T @ dyk
                dw = np.where(lower, dyk @ xk.T, 0.0)              # ∂/∂ of each product term
                dcb = dw * dec * dtk[None, :]
                dCh[b, ts, h] += dcb @ Bk
                dBh[b, ts, h] += dcb.T @ Ck
                ddt[b, ts, h] += np.sum(dw * cb * dec, axis=0)
                g = dw * cb * dtk[None, :] * dec                    # ∂/∂(u_t − u_j)
                du[ts] += g.sum(axis=1) - g.sum(axis=0)
                # inter-chunk term
                eu = np.exp(u)
                dCh[b, ts, h] += eu[:, None] * (dyk @ H_in[b, h, k].T)
                dHin[k] += (eu[:, None] * Ck).T @ dyk
                du[ts] += eu * np.sum(dyk * (Ck @ H_in[b, h, k]), axis=1)
            # state passing, last chunk first
            dmem = np.zeros((M, N, P))
            Gs = dHin[M].copy()
            for c in range(M - 1, -1, -1):
                ts, _, _, _, u = chunks[c]
                dmem[c] = Gs + (0.0 if ddH is None else _f64(ddH)[b, h, c])
                du[ts[-1]] += np.sum(Gs * np.exp(u[-1]) * H_in[b, h, c])
                Gs = np.exp(u[-1]) * Gs + dHin[c]
            dh0[b, h] = Gs
            # chunk memories
            for c in range(M):
                ts, xk, Bk, dtk, u = chunks[c]
                wd = np.exp(u[-1] - u)
                dx[b, ts, h] += (wd * dtk)[:, None] * (Bk @ dmem[c])
                dBh[b, ts, h] += (wd * dtk)[:, None] * (xk @ dmem[c].T)
                dwi = np.einsum("in,np,ip->i", Bk, dmem[c], xk)
                ddt[b, ts, h] += wd * dwi
                gw = dwi * wd * dtk                                 # ∂/∂(U_c − u_i)
                du[ts[-1]] += gw.sum()
                du[ts] -= gw
            # u_t = a·Σ_{l=kS}^{t} dt_l
            for ts, _, _, dtk, _ in chunks:
                ddt[b, ts, h] += a * np.cumsum(du[ts][::-1])[::-1]
                dA[h] += np.sum(du[ts] * np.cumsum(dtk))
    gmap = group_of_head(H, G)
    dB, dC = np.zeros((Bsz, L, G, N)), np.zeros((Bsz, L, G, N))
    for h in range(H):
        dB[:, :, gmap[h]] += dBh[:, :, h]
        dC[:, :, gmap[h]] += dCh[:, :, h]
    return {"dx": dx, "ddt": ddt, "dA": dA, "dB": dB, "dC": dC, "dh0": dh0}


# --------------------------------------------------------------------------
# O6 - state-memory attention
# --------------------------------------------------------------------------
def _softmax(s):
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def sma(Q, E, C, dH, S, tokens=None):
    """SMA readout o_t for every token (or for the listed token indices)
    [pith-core; pith-carries; pith-maj3; abstract]:

    for token t of chunk k >= 1 and every completed chunk c < k
        key    K_{t,c} = ΔH[c]·E_t          (in R^N, value axis contracted)
        value  V_{t,c} = C_tᵀ·ΔH[c]         (in R^P, same C_t as the SSM)
        score  s_{t,c} = Q_t·K_{t,c} / sqrt(N)
        o_t = Σ_c softmax_c(s_{t,c})·V_{t,c};  o_t = 0 for chunk 0.
    Returns o [B,L,H,P] (rows not listed in ``tokens`` stay zero)."""
    E, dH = _f64(E), _f64(dH)
    Bsz, L, H, P = E.shape
    Qh, Ch = _per_head(Q, H), _per_head(C, H)
    N = Qh.shape[-1]
    o = np.zeros((Bsz, L, H, P))
    t_all = np.arange(L) if tokens is None else np.asarray(tokens)
    for b in range(Bsz):
        for h in range(H):
            for k in range(1, L // S):
                ts = t_all[(t_all >= k * S) & (t_all < (k + 1) * S)]
                if ts.size == 0:
                    continue
                mem = dH[b, h, :k]                                  # [k,N,P]
                keys = np.einsum("cnp,tp->tcn", mem, E[b, ts, h])
                scores = np.einsum("tn,tcn->tc", Qh[b, ts, h], keys) / math.sqrt(N)
                vals = np.einsum("tn,cnp->tcp", Ch[b, ts, h], mem)
                o[b, ts, h] = np.einsum("tc,tcp->tp", _softmax(scores), vals)
    return o


def sma_backward(Q, E, C, dH, S, do):
    """Gradients of a loss through the SMA readout, given do = ∂loss/∂o
    [B,L,H,P] (reverse-mode chain rule through the steps of :func:`sma`).
    For token t of chunk k, memory c < k, with K, V, s as in :func:`sma` and
    α the softmax weights over c:

        dV_{t,c} = α_{t,c}·do_t
        dα_{t,c} = do_t·V_{t,c}
        ds_{t,c} = α_{t,c}·(dα_{t,c} − Σ_c' α_{t,c'}·dα_{t,c'})
        dK_{t,c} = ds_{t,c}·Q_t / sqrt(N)
        dQ_t  += Σ_c ds_{t,c}·K_{t,c} / sqrt(N)
        dE_t  += Σ_c ΔH[c]ᵀ·dK_{t,c}
        dC_t  += Σ_c ΔH[c]·dV_{t,c}
        dΔH[c] += Σ_t dK_{t,c}·E_tᵀ + C_t·dV_{t,c}ᵀ

    Q and C are shared by the heads of a group, so their gradients are
    summed over those heads.  Returns (dQ [B,L,G,N], dE [B,L,H,P],
    dC [B,L,G,N], ddH [B,H,M,N,P])."""
    E, dH, do = _f64(E), _f64(dH), _f64(do)
    Bsz, L, H, P = E.shape
    G = np.shape(Q)[2]
    Qh, Ch = _per_head(Q, H), _per_head(C, H)
    N = Qh.shape[-1]
    dQh = np.zeros((Bsz, L, H, N))
    dCh = np.zeros((Bsz, L, H, N))
    dE = np.zeros((Bsz, L, H, P))
    ddH = np.zeros_like(dH)
    rs = 1.0 / math.sqrt(N)
    for b in range(Bsz):
        for h in range(H):
            for k in range(1, L // S):
                ts = np.arange(k * S, (k + 1) * S)
                mem = dH[b, h, :k]  # the memories token ts read, [k,N,P]
                Qt, Ct, Et, dot = Qh[b, ts, h], Ch[b, ts, h], E[b, ts, h], do[b, ts, h]
                K = np.einsum("cnp,tp->tcn", mem, Et)               # [t,c,N]
                V = np.einsum("tn,cnp->tcp", Ct, mem)               # [t,c,P]
                alpha = _softmax(np.einsum("tn,tcn->tc", Qt, K) * rs)
                dV = alpha[:, :, None] * dot[:, None, :]
                dalpha = np.einsum("tp,tcp->tc", dot, V)
                ds = alpha * (dalpha - np.sum(alpha * dalpha, axis=1, keepdims=True))
                dK = ds[:, :, None] * Qt[:, None, :] * rs           # [t,c,N]
                dQh[b, ts, h] += np.einsum("tc,tcn->tn", ds, K) * rs
                dE[b, ts, h] += np.einsum("cnp,tcn->tp", mem, dK)
                dCh[b, ts, h] += np.einsum("cnp,tcp->tn", mem, dV)
                ddH[b, h, :k] += (np.einsum("tcn,tp->cnp", dK, Et)
                                  + np.einsum("tn,tcp->cnp", Ct, dV))
    gmap = group_of_head(H, G)
    dQ = np.zeros((Bsz, L, G, N))
    dC = np.zeros((Bsz, L, G, N))
    for h in range(H):
        dQ[:, :, gmap[h]] += dQh[:, :, h]
        dC[:, :, gmap[h]] += dCh[:, :, h]
    return dQ, dE, dC, ddH


def sma_logsumexp(Q, E, C, dH, S):
    """log Σ_{c<k} exp(s_{t,c}) per token (natural log; the softmax
    normaliser of :func:`sma`), [B,H,L]; 0 for chunk-0 tokens."""
    E, dH = _f64(E), _f64(dH)
    Bsz, L, H, P = E.shape
    Qh = _per_head(Q, H)
    N = Qh.shape[-1]
    out = np.zeros((Bsz, H, L))
    for b in range(Bsz):
        for h in range(H):
            for k in range(1, L // S):
                ts = np.arange(k * S, (k + 1) * S)
                keys = np.einsum("cnp,tp->tcn", dH[b, h, :k], E[b, ts, h])
                sc = np.einsum("tn,tcn->tc", Qh[b, ts, h], keys) / math.sqrt(N)
                m = np.max(sc, axis=1)
                out[b, h, ts] = m + np.log(np.sum(np.exp(sc - m[:, None]), axis=1))
    return out


def gated_backward(dy, o, g):
    """Backward of y = y_ssd + g·o [pith-core]: returns (dy_ssd, do, dg) =
    (dy, g·dy, Σ dy·o) for an upstream gradient dy."""
    dy, o = _f64(dy), _f64(o)
    return dy.copy(), float(g) * dy, float(np.sum(dy * o))


def sma_bruteforce(Q, E, C, dH, S):
    """The same readout as :func:`sma`, one token and one chunk at a time with
    scalar loops (tiny inputs only)."""
    E, dH = _f64(E), _f64(dH)
    Bsz, L, H, P = E.shape
    Qh, Ch = _per_head(Q, H), _per_head(C, H)
    N = Qh.shape[-1]
    o = np.zeros((Bsz, L, H, P))
    for b in range(Bsz):
        for h in range(H):
            for t in range(L):
                k = t // S
                if k == 0:
                    continue
                scores, vals = [], []
                for c in range(k):
                    s = 0.0
                    for n in range(N):
                        key_n = 0.0
                        for p in range(P):
                            key_n += dH[b, h, c, n, p] * E[b, t, h, p]
                        s += Qh[b, t, h, n] * key_n
                    scores.append(s / math.sqrt(N))
                    v = [sum(Ch[b, t, h, n] * dH[b, h, c, n, p] for n in range(N))
                         for p in range(P)]
                    vals.append(v)
                mx = max(scores)
                wts = [math.exp(s - mx) for s in scores]
                tot = sum(wts)
                for p in range(P):
                    o[b, t, h, p] = sum(w * v[p] for w, v in zip(wts, vals)) / tot
    return o


def sma_continue(Q, E, C, dH_prior, dH, S):
    """SMA readout of tokens that continue sequences already holding
    k0 = dH_prior.shape[2] completed chunks (chunked prefill): token t of
    local chunk j is token k0·S + t of the whole sequence and attends to the
    k0 prior memories and the first j new ones, with the formulas of
    :func:`sma`.  Returns o [B,L,H,P] for the new tokens."""
    E = _f64(E)
    Bsz, L, H, P = E.shape
    Qh, Ch = _per_head(Q, H), _per_head(C, H)
    N = Qh.shape[-1]
    mem_all = np.concatenate([_f64(dH_prior), _f64(dH)], axis=2)
    k0 = dH_prior.shape[2]
    o = np.zeros((Bsz, L, H, P))
    for b in range(Bsz):
        for h in range(H):
            for j in range(L // S):
                if k0 + j == 0:
                    continue
                ts = np.arange(j * S, (j + 1) * S)
                seen = mem_all[b, h, :k0 + j]                       # [k0+j,N,P]
                key = np.einsum("cnp,tp->tcn", seen, E[b, ts, h])
                sc = np.einsum("tn,tcn->tc", Qh[b, ts, h], key) / math.sqrt(N)
                val = np.einsum("tn,cnp->tcp", Ch[b, ts, h], seen)
                o[b, ts, h] = np.einsum("tc,tcp->tp", _softmax(sc), val)
    return o


def sma_decayed(Q, E, C, dH, dt, A, S, tokens=None):
    """The decay-included SMA variant that the review asks to ablate
    [pith-maj3]: memory c enters the readout of token t (chunk k > c) scaled
    by the decay the SSM applies to chunk c's contribution between the chunk
    boundary e(c) = (c+1)·S − 1 and t,

        d_{t,c} = exp(A_h · Σ_{j=e(c)+1}^{t} dt_j),
        key   d_{t,c}·ΔH[c]·E_t,   value   d_{t,c}·C_tᵀ·ΔH[c],
        score d_{t,c}·Q_t·(ΔH[c]·E_t) / sqrt(N),   o_t = Σ_c softmax_c·value.

    The segment sum of dt is a difference of an inclusive fp64 cumsum.
    Returns o [B,L,H,P] (rows not listed in ``tokens`` stay zero)."""
    E, dH, dt, A = _f64(E), _f64(dH), _f64(dt), _f64(A)
    Bsz, L, H, P = E.shape
    Qh, Ch = _per_head(Q, H), _per_head(C, H)
    N = Qh.shape[-1]
    o = np.zeros((Bsz, L, H, P))
    t_all = np.arange(L) if tokens is None else np.asarray(tokens)
    for b in range(Bsz):
        for h in range(H):
            cs = np.cumsum(dt[b, :, h])                             # inclusive
            for k in range(1, L // S):
                ts = t_all[(t_all >= k * S) & (t_all < (k + 1) * S)]
                if ts.size == 0:
                    continue
                ends = np.arange(k) * S + (S - 1)                   # e(c)
                d = np.exp(A[h] * (cs[ts][:, None] - cs[ends][None, :]))  # [t,c]
                mem = dH[b, h, :k]  # undecayed memories, [k,N,P]
                keys = np.einsum("cnp,tp->tcn", mem, E[b, ts, h])
                scores = d * np.einsum("tn,tcn->tc", Qh[b, ts, h], keys) / math.sqrt(N)
                vals = d[:, :, None] * np.einsum("tn,cnp->tcp", Ch[b, ts, h], mem)
                o[b, ts, h] = np.einsum("tc,tcp->tp", _softmax(scores), vals)
    return o


# --------------------------------------------------------------------------
# O7 - gated residual
# --------------------------------------------------------------------------
def gated_output(y_ssd, o, g):
    """y = y_ssd + g·o  [pith-core: readout added through a zero-initialised
    scalar gate; abstract: gated residual]."""
    return _f64(y_ssd) + float(g) * _f64(o)


def prefill(x, dt, A, Bm, C, Q, E, g, S, h0=None, decayed=False):
    """The whole prefill path O3 -> O4 -> O5 -> O6 -> O7 (O6 in the
    decay-included variant when ``decayed``).
    Returns a dict with dH, H_in, y_ssd, o, y, h_final."""
    dH = chunk_states(x, dt, A, Bm, S)
    H_in = state_pass(dH, dt, A, S, h0)
    y_ssd = chunk_output(x, dt, A, Bm, C, H_in, S)
    o = sma_decayed(Q, E, C, dH, dt, A, S) if decayed else sma(Q, E, C, dH, S)
    return {"dH": dH, "H_in": H_in, "y_ssd": y_ssd, "o": o,
            "y": gated_output(y_ssd, o, g), "h_final": H_in[:, :, -1]}


# --------------------------------------------------------------------------
# O8 - single-token decode over the chunk-memory cache
# --------------------------------------------------------------------------
def round_bf16(a):
    """Round fp64 values to the nearest bfloat16 (ties to even), returned as
    fp64.  Used where the cache is kept in bfloat16.

    bfloat16 is binary32 with the significand cut to 8 bits (1 implicit + 7
    stored), so a finite x = m·2^e (0.5 <= |m| < 1, numpy frexp) lies on the
    grid 2^(e-8); below the smallest normal 2^-126 the grid stays at the
    subnormal step 2^-133.  x is rounded once, straight from fp64, to the
    nearest grid point, an exact tie going to the even multiple (numpy rint);
    magnitudes that round to 2^128 or beyond overflow to infinity."""
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(a / step) * step
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, a), r)


def decode_step(state, x, dt, A, Bm, C, Q, E, g, S, cache_bf16=True):
    """One new token per sequence [abstract: the length-dependent cache is
    the set of chunk memories; pith-eq14].

    state: dict with cache [B,H,Mmax,N,P], h [B,H,N,P], dH_cur [B,H,N,P],
    n_chunks [B] and pos [B] (pos = index of the new token in its chunk).
    Token inputs: x [B,H,P], dt [B,H], A [H], Bm/C/Q [B,G,N], E [B,H,P].

    1. a = exp(dt·A); h <- a·h + dt·B xᵀ; ΔH_cur <- a·ΔH_cur + dt·B xᵀ;
       y_ssd = Cᵀ h.
    2. o = SMA over cache[0 .. n_chunks-1] (same formulas as :func:`sma`).
    3. y = y_ssd + g·o.
    4. If the token closes its chunk (pos = S-1): cache[n_chunks] <- ΔH_cur
       (rounded to bfloat16 when the cache is bfloat16), ΔH_cur <- 0,
       n_chunks += 1, pos <- 0; otherwise pos += 1.
    Returns (y [B,H,P], new_state)."""
    x, dt, A, E = _f64(x), _f64(dt), _f64(A), _f64(E)
    Bsz, H, P = x.shape
    gmap = group_of_head(H, Bm.shape[1])
    Bh, Ch, Qh = _f64(Bm)[:, gmap], _f64(C)[:, gmap], _f64(Q)[:, gmap]
    N = Bh.shape[-1]
    cache = _f64(state["cache"]).copy()
    h = _f64(state["h"]).copy()
    dHc = _f64(state["dH_cur"]).copy()
    n_chunks = np.asarray(state["n_chunks"]).astype(np.int64).copy()
    pos = np.asarray(state["pos"]).astype(np.int64).copy()

    a = np.exp(dt * A[None, :])                                     # [B,H]
    inp = dt[:, :, None, None] * Bh[:, :, :, None] * x[:, :, None, :]
    h = a[:, :, None, None] * h + inp
    dHc = a[:, :, None, None] * dHc + inp
    y_ssd = np.einsum("bhn,bhnp->bhp", Ch, h)

    o = np.zeros((Bsz, H, P))
    for b in range(Bsz):
        k = int(n_chunks[b])
        if k == 0:
            continue
        for hh in range(H):
            mem = cache[b, hh, :k]                                  # [k,N,P]
            keys = np.einsum("cnp,p->cn", mem, E[b, hh])
            scores = keys @ Qh[b, hh] / math.sqrt(N)
            vals = np.einsum("n,cnp->cp", Ch[b, hh], mem)
            o[b, hh] = _softmax(scores) @ vals
    y = y_ssd + float(g) * o

    for b in range(Bsz):
        if pos[b] == S - 1:
            k = int(n_chunks[b])
            cache[b, :, k] = round_bf16(dHc[b]) if cache_bf16 else dHc[b]
            dHc[b] = 0.0
            n_chunks[b] = k + 1
            pos[b] = 0
        else:
            pos[b] += 1
    new_state = {"cache": cache, "h": h, "dH_cur": dHc,
                 "n_chunks": n_chunks, "pos": pos}
    return y, new_state


# --------------------------------------------------------------------------
# O9 - cache accounting
# --------------------------------------------------------------------------
def cache_elements(L, S, N, P):
    """Per head: DART keeps one N×P memory per completed chunk, a token-level
    attention layer keeps a key and a value of size P per token
    [pith-eq14].  Returns (dart_elements, attention_elements)."""
    return (L // S) * N * P, 2 * L * P


def cache_ratio(L, S, N, P):
    """DART cache / attention cache, per head [pith-eq14]."""
    dart, attn = cache_elements(L, S, N, P)
    return dart / attn


# --------------------------------------------------------------------------
# O10 - fp8 chunk-memory cache [pith-ext]
# --------------------------------------------------------------------------
# OCP 8-bit floating point, E4M3 variant: sign bit, 4 exponent bits with bias
# 7, 3 mantissa bits; exponent field 0 holds the subnormals m·2^-9; there are
# no infinities, the codes 0x7F and 0xFF are NaN, the largest finite value is
# 1.75·2^8 = 448.
E4M3_MAX = 448.0


def fp8_e4m3_decode(codes):
    """Value of each E4M3 code (uint8 array) as fp64; NaN codes give NaN."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c >= 128, -1.0, 1.0)
    field = (c >> 3) & 15
    mant = c & 7
    normal = (1.0 + mant / 8.0) * np.exp2(field - 7.0)
    sub = mant * 2.0 ** -9
    v = sign * np.where(field == 0, sub, normal)
    return np.where((field == 15) & (mant == 7), np.nan, v)


def fp8_e4m3_encode(v):
    """E4M3 code (uint8) of each value, rounded to the nearest representable
    value with ties to the even mantissa.  The values must round to at most
    448 in magnitude (ValueError otherwise): the scaled cache never gets
    near that bound.  A value that rounds to zero keeps its sign (0x80 is
    negative zero)."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("fp8_e4m3_encode: non-finite value")
    neg = np.signbit(v)
    a = np.abs(v)
    # binade 2^e of |v| (frexp: a = f·2^E, 0.5 <= f < 1, so e = E - 1);
    # the grid spacing is 2^(e-3), and 2^-9 throughout the subnormal range
    _, E = np.frexp(a)
    e = np.maximum(E - 1, -6)
    step = np.exp2(e - 3.0)
    r = np.round(a / step) * step  # numpy rounds halves to even
    if np.any(r > E4M3_MAX):
        raise ValueError("fp8_e4m3_encode: value beyond the E4M3 range")
    # fields of the rounded magnitude (rounding may carry into the next binade)
    _, Er = np.frexp(r)
    er = Er - 1
    is_sub = (r < 2.0 ** -6)
    field = np.where(is_sub, 0, er + 7)
    mant = np.where(is_sub, r / 2.0 ** -9,
                    (r / np.exp2(np.where(is_sub, 0, er).astype(np.float64)) - 1.0) * 8.0)
    mant = np.rint(mant).astype(np.int64)
    code = np.where(neg, 128, 0) + field.astype(np.int64) * 8 + mant
    return code.astype(np.uint8)


def fp8_memory_scale(mem):
    """Scale of one memory: 2^e with e = max(E - 8, -126), where the largest
    magnitude of the memory is f·2^E, 0.5 <= f < 1; 1 for an all-zero memory.
    The scaled memory then has its largest magnitude in [128, 256), inside
    the E4M3 range with one binade to spare."""
    amax = float(np.max(np.abs(np.asarray(mem, dtype=np.float64))))
    if amax == 0.0:
        return 1.0
    _, E = math.frexp(amax)
    return math.ldexp(1.0, max(E - 8, -126))


def fp8_quantize_memory(mem):
    """(codes uint8 of mem's shape, scale): codes = E4M3(mem / scale).  The
    division by a power of two is exact, so the codes are the rounding of
    the memory itself on a grid scaled by the scale."""
    mem = np.asarray(mem, dtype=np.float64)
    s = fp8_memory_scale(mem)
    return fp8_e4m3_encode(mem / s), s


def fp8_dequantize(codes, scale):
    """Memories from codes [..., N, P] and scales [...]: decode(code)·scale."""
    return fp8_e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None, None]


def decode_step_fp8(state, x, dt, A, Bm, C, Q, E, g, S):
    """:func:`decode_step` over an fp8 cache.

    state: as for decode_step, with the cache held as codes [B,H,Mmax,N,P]
    (uint8) and scales [B,H,Mmax] instead of "cache".  The SMA reads the
    dequantised memories decode(code)·scale; a memory appended by this step
    is quantised with :func:`fp8_quantize_memory` (one scale per head)."""
    codes = np.asarray(state["codes"]).copy()
    scales = np.asarray(state["scales"], dtype=np.float64).copy()
    plain = dict(state)
    plain["cache"] = fp8_dequantize(codes, scales)
    del plain["codes"], plain["scales"]
    y, new = decode_step(plain, x, dt, A, Bm, C, Q, E, g, S, cache_bf16=False)
    n_old = np.asarray(state["n_chunks"]).astype(np.int64)
    for b in range(codes.shape[0]):
        k = int(n_old[b])
        if new["n_chunks"][b] == k + 1:  # this token closed chunk k
            for h in range(codes.shape[1]):
                codes[b, h, k], scales[b, h, k] = fp8_quantize_memory(new["cache"][b, h, k])
    del new["cache"]
    new["codes"], new["scales"] = codes, scales
    return y, new
