"""Thin Python binding of the DART C ABI (include/dart.h).

Functions named like the C entry points take torch tensors that already
live on the GPU, check their dtype, shape, device and contiguity, and pass
raw pointers plus torch's current HIP stream.  Every step of the hot path
runs inside libdart's HIP kernels; torch only provides device memory and
the stream.  ``prefill`` and ``decode_step`` allocate the outputs with torch
and chain the entry points.
"""

import torch

from ._lib import DART_BF16, DART_F32, DartDecodeDims, DartDims, check, lib

_IO = {torch.float32: DART_F32, torch.bfloat16: DART_BF16}


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _ptr(t, name, dtype=None, shape=None, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _io_code(dtype):
    if dtype not in _IO:
        raise TypeError(f"element type must be float32 or bfloat16 (got {dtype})")
    return _IO[dtype]


def prefill_dims(x, Bm, chunk):
    """dart_dims from x [B, L, H, P] and Bm [B, L, G, N]."""
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    return DartDims(B, L, H, G, N, P, int(chunk), _io_code(x.dtype))


def dart_chunk_state(x, dt, A, Bm, acum, dH, dH_f32, chunk):
    """Chunk state memories: acum [B,H,M,S] f32, dH [B,H,M,P,N] io and
    dH_f32 [B,H,M,P,N] f32 from x, dt, A, Bm."""
    d = prefill_dims(x, Bm, chunk)
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    M, io, dev = L // chunk, x.dtype, x.device
    args = [_ptr(x, "x", io, (B, L, H, P), dev), _ptr(dt, "dt", torch.float32, (B, L, H), dev),
            _ptr(A, "A", torch.float32, (H,), dev), _ptr(Bm, "Bm", io, (B, L, G, N), dev),
            _ptr(acum, "acum", torch.float32, (B, H, M, chunk), dev),
            _ptr(dH, "dH", io, (B, H, M, P, N), dev),
            _ptr(dH_f32, "dH_f32", torch.float32, (B, H, M, P, N), dev)]
    check(lib().dart_chunk_state(d, *args, _stream()), "dart_chunk_state")


def dart_state_pass(x, dt, Bm, C, acum, dH_f32, h0, H_in, h_final, y_ssd, chunk):
    """State passing: H_in [B,H,M,P,N] io (state entering each chunk),
    h_final [B,H,P,N] f32 and the native output y_ssd [B,L,H,P] io;
    h0 [B,H,P,N] f32 or None (zero)."""
    d = prefill_dims(x, Bm, chunk)
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    M, io, dev = L // chunk, x.dtype, x.device
    args = [_ptr(x, "x", io, (B, L, H, P), dev), _ptr(dt, "dt", torch.float32, (B, L, H), dev),
            _ptr(Bm, "Bm", io, (B, L, G, N), dev), _ptr(C, "C", io, (B, L, G, N), dev),
            _ptr(acum, "acum", torch.float32, (B, H, M, chunk), dev),
            _ptr(dH_f32, "dH_f32", torch.float32, (B, H, M, P, N), dev),
            _ptr(h0, "h0", torch.float32, (B, H, P, N), dev),
            _ptr(H_in, "H_in", io, (B, H, M, P, N), dev),
            _ptr(h_final, "h_final", torch.float32, (B, H, P, N), dev),
            _ptr(y_ssd, "y_ssd", io, (B, L, H, P), dev)]
    check(lib().dart_state_pass(d, *args, _stream()), "dart_state_pass")


def dart_chunk_scan_workspace(dims):
    """Bytes of device workspace dart_chunk_scan needs for these dims."""
    return int(lib().dart_chunk_scan_workspace(dims))


def dart_chunk_scan(x, dt, A, Bm, h0, acum, dH, dH_f32, H_in, h_final, workspace, chunk):
    """Chunk memories and the state recurrence in one pass: acum, dH (io),
    dH_f32 (f32, or None to skip), H_in (io) and h_final (f32), the outputs
    of dart_chunk_state and of dart_state_pass's recurrence; h0 [B,H,P,N]
    f32 or None (zero); workspace a uint8 device tensor of at least
    dart_chunk_scan_workspace bytes."""
    d = prefill_dims(x, Bm, chunk)
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    M, io, dev = L // chunk, x.dtype, x.device
    args = [_ptr(x, "x", io, (B, L, H, P), dev), _ptr(dt, "dt", torch.float32, (B, L, H), dev),
            _ptr(A, "A", torch.float32, (H,), dev), _ptr(Bm, "Bm", io, (B, L, G, N), dev),
            _ptr(h0, "h0", torch.float32, (B, H, P, N), dev),
            _ptr(acum, "acum", torch.float32, (B, H, M, chunk), dev),
            _ptr(dH, "dH", io, (B, H, M, P, N), dev),
            _ptr(dH_f32, "dH_f32", torch.float32, (B, H, M, P, N), dev),
            _ptr(H_in, "H_in", io, (B, H, M, P, N), dev),
            _ptr(h_final, "h_final", torch.float32, (B, H, P, N), dev)]
    wsp = _ptr(workspace, "workspace", torch.uint8, None, dev)
    check(lib().dart_chunk_scan(d, *args, wsp, workspace.numel(), _stream()), "dart_chunk_scan")


def dart_chunk_out(x, dt, Bm, C, acum, H_in, y_ssd, chunk):
    """Native chunk output y_ssd [B,L,H,P] io from H_in [B,H,M,P,N] io."""
    d = prefill_dims(x, Bm, chunk)
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    M, io, dev = L // chunk, x.dtype, x.device
    args = [_ptr(x, "x", io, (B, L, H, P), dev), _ptr(dt, "dt", torch.float32, (B, L, H), dev),
            _ptr(Bm, "Bm", io, (B, L, G, N), dev), _ptr(C, "C", io, (B, L, G, N), dev),
            _ptr(acum, "acum", torch.float32, (B, H, M, chunk), dev),
            _ptr(H_in, "H_in", io, (B, H, M, P, N), dev),
            _ptr(y_ssd, "y_ssd", io, (B, L, H, P), dev)]
    check(lib().dart_chunk_out(d, *args, _stream()), "dart_chunk_out")


def _scan(out, x, dt, A, Bm, C, chunk, h0, one_pass):
    """The chunked scan into the tensors of ``out``: dart_chunk_state +
    dart_state_pass (also filling out["dH_f32"]), or with one_pass
    dart_chunk_scan + dart_chunk_out (no f32 memories)."""
    if not one_pass:
        dart_chunk_state(x, dt, A, Bm, out["acum"], out["dH"], out["dH_f32"], chunk)
        dart_state_pass(x, dt, Bm, C, out["acum"], out["dH_f32"], h0, out["H_in"],
                        out["h_final"], out["y_ssd"], chunk)
        return
    ws = torch.empty(dart_chunk_scan_workspace(prefill_dims(x, Bm, chunk)), dtype=torch.uint8,
                     device=x.device)
    dart_chunk_scan(x, dt, A, Bm, h0, out["acum"], out["dH"], None, out["H_in"], out["h_final"],
                    ws, chunk)
    dart_chunk_out(x, dt, Bm, C, out["acum"], out["H_in"], out["y_ssd"], chunk)


def dart_sma_fwd(Q, E, C, dH, y_ssd, gate, y, chunk):
    """State-memory attention + gated add: y [B,L,H,P] io."""
    B, L, H, P = E.shape
    G, N = Q.shape[2], Q.shape[3]
    d = DartDims(B, L, H, G, N, P, int(chunk), _io_code(E.dtype))
    M, io, dev = L // chunk, E.dtype, E.device
    args = [_ptr(Q, "Q", io, (B, L, G, N), dev), _ptr(E, "E", io, (B, L, H, P), dev),
            _ptr(C, "C", io, (B, L, G, N), dev), _ptr(dH, "dH", io, (B, H, M, P, N), dev),
            _ptr(y_ssd, "y_ssd", io, (B, L, H, P), dev)]
    yp = _ptr(y, "y", io, (B, L, H, P), dev)
    check(lib().dart_sma_fwd(d, *args, float(gate), yp, _stream()), "dart_sma_fwd")


def dart_sma_fwd_cont(Q, E, C, cache, prior_chunks, dH, y_ssd, gate, y, chunk):
    """SMA + gated add for tokens that continue sequences holding
    ``prior_chunks`` memories in ``cache`` [B,H,max_chunks,P,N] io (see
    include/dart.h); dH [B,H,M,P,N] are the new tokens' memories."""
    B, L, H, P = E.shape
    G, N = Q.shape[2], Q.shape[3]
    d = DartDims(B, L, H, G, N, P, int(chunk), _io_code(E.dtype))
    M, io, dev = L // chunk, E.dtype, E.device
    cache_chunks = cache.shape[2]
    args = [_ptr(Q, "Q", io, (B, L, G, N), dev), _ptr(E, "E", io, (B, L, H, P), dev),
            _ptr(C, "C", io, (B, L, G, N), dev),
            _ptr(cache, "cache", io, (B, H, cache_chunks, P, N), dev),
            _ptr(dH, "dH", io, (B, H, M, P, N), dev),
            _ptr(y_ssd, "y_ssd", io, (B, L, H, P), dev)]
    yp = _ptr(y, "y", io, (B, L, H, P), dev)
    check(lib().dart_sma_fwd_cont(d, int(prior_chunks), int(cache_chunks), *args, float(gate),
                                  yp, _stream()), "dart_sma_fwd_cont")


def dart_sma_fwd_cont_fp8(Q, E, C, cache8, scale, prior_chunks, dH, y_ssd, gate, y, chunk):
    """dart_sma_fwd_cont with the prior memories in the fp8 cache: codes
    cache8 [B,H,max_chunks,P,N] uint8 and scales [B,H,max_chunks] f32 (see
    include/dart.h); bfloat16 io only."""
    B, L, H, P = E.shape
    G, N = Q.shape[2], Q.shape[3]
    d = DartDims(B, L, H, G, N, P, int(chunk), _io_code(E.dtype))
    M, io, dev = L // chunk, E.dtype, E.device
    cache_chunks = cache8.shape[2]
    args = [_ptr(Q, "Q", io, (B, L, G, N), dev), _ptr(E, "E", io, (B, L, H, P), dev),
            _ptr(C, "C", io, (B, L, G, N), dev),
            _ptr(cache8, "cache8", torch.uint8, (B, H, cache_chunks, P, N), dev),
            _ptr(scale, "scale", torch.float32, (B, H, cache_chunks), dev),
            _ptr(dH, "dH", io, (B, H, M, P, N), dev),
            _ptr(y_ssd, "y_ssd", io, (B, L, H, P), dev)]
    yp = _ptr(y, "y", io, (B, L, H, P), dev)
    check(lib().dart_sma_fwd_cont_fp8(d, int(prior_chunks), int(cache_chunks), *args,
                                      float(gate), yp, _stream()), "dart_sma_fwd_cont_fp8")


def dart_sma_fwd_decayed(Q, E, C, dH, acum, y_ssd, gate, y, chunk):
    """Decay-included SMA + gated add (see include/dart.h): acum [B,H,M,S]
    f32 from dart_chunk_state; y [B,L,H,P] io."""
    B, L, H, P = E.shape
    G, N = Q.shape[2], Q.shape[3]
    d = DartDims(B, L, H, G, N, P, int(chunk), _io_code(E.dtype))
    M, io, dev = L // chunk, E.dtype, E.device
    args = [_ptr(Q, "Q", io, (B, L, G, N), dev), _ptr(E, "E", io, (B, L, H, P), dev),
            _ptr(C, "C", io, (B, L, G, N), dev), _ptr(dH, "dH", io, (B, H, M, P, N), dev),
            _ptr(acum, "acum", torch.float32, (B, H, M, chunk), dev),
            _ptr(y_ssd, "y_ssd", io, (B, L, H, P), dev)]
    yp = _ptr(y, "y", io, (B, L, H, P), dev)
    check(lib().dart_sma_fwd_decayed(d, *args, float(gate), yp, _stream()),
          "dart_sma_fwd_decayed")


def dart_sma_fwd_train(Q, E, C, dH, y_ssd, gate, y, o, lse, chunk):
    """SMA + gated add that also writes o [B,L,H,P] f32 and lse [B,H,L] f32
    for the backward (see include/dart.h)."""
    B, L, H, P = E.shape
    G, N = Q.shape[2], Q.shape[3]
    d = DartDims(B, L, H, G, N, P, int(chunk), _io_code(E.dtype))
    M, io, dev = L // chunk, E.dtype, E.device
    args = [_ptr(Q, "Q", io, (B, L, G, N), dev), _ptr(E, "E", io, (B, L, H, P), dev),
            _ptr(C, "C", io, (B, L, G, N), dev), _ptr(dH, "dH", io, (B, H, M, P, N), dev),
            _ptr(y_ssd, "y_ssd", io, (B, L, H, P), dev)]
    outs = [_ptr(y, "y", io, (B, L, H, P), dev), _ptr(o, "o", torch.float32, (B, L, H, P), dev),
            _ptr(lse, "lse", torch.float32, (B, H, L), dev)]
    check(lib().dart_sma_fwd_train(d, *args, float(gate), *outs, _stream()),
          "dart_sma_fwd_train")


def dart_sma_bwd_workspace(dims):
    """Workspace bytes for dart_sma_bwd (0 for unsupported dims)."""
    return int(lib().dart_sma_bwd_workspace(dims))


def dart_sma_bwd(Q, E, C, dH, o, lse, dy, gate, chunk, out=None):
    """Backward of SMA + gated add (see include/dart.h).  Returns a dict of
    f32 device tensors dQ, dC [B,L,G,N], dE [B,L,H,P], ddH [B,H,M,P,N] and
    dgate [1]; ``out`` may hold preallocated ones plus "workspace"."""
    B, L, H, P = E.shape
    G, N = Q.shape[2], Q.shape[3]
    d = DartDims(B, L, H, G, N, P, int(chunk), _io_code(E.dtype))
    M, io, dev = L // chunk, E.dtype, E.device
    ws = dart_sma_bwd_workspace(d)
    if ws == 0:
        raise ValueError("dart_sma_bwd: unsupported dimensions")
    f32 = dict(dtype=torch.float32, device=dev)
    if out is None:
        out = {"dQ": torch.empty(B, L, G, N, **f32), "dC": torch.empty(B, L, G, N, **f32),
               "dE": torch.empty(B, L, H, P, **f32), "ddH": torch.empty(B, H, M, P, N, **f32),
               "dgate": torch.empty(1, **f32),
               "workspace": torch.empty(ws, dtype=torch.uint8, device=dev)}
    args = [_ptr(Q, "Q", io, (B, L, G, N), dev), _ptr(E, "E", io, (B, L, H, P), dev),
            _ptr(C, "C", io, (B, L, G, N), dev), _ptr(dH, "dH", io, (B, H, M, P, N), dev),
            _ptr(o, "o", torch.float32, (B, L, H, P), dev),
            _ptr(lse, "lse", torch.float32, (B, H, L), dev),
            _ptr(dy, "dy", io, (B, L, H, P), dev)]
    outs = [_ptr(out["dQ"], "dQ", torch.float32, (B, L, G, N), dev),
            _ptr(out["dE"], "dE", torch.float32, (B, L, H, P), dev),
            _ptr(out["dC"], "dC", torch.float32, (B, L, G, N), dev),
            _ptr(out["ddH"], "ddH", torch.float32, (B, H, M, P, N), dev),
            _ptr(out["dgate"], "dgate", torch.float32, (1,), dev)]
    wsp = _ptr(out["workspace"], "workspace", torch.uint8, None, dev)
    check(lib().dart_sma_bwd(d, *args, float(gate), *outs, wsp, out["workspace"].numel(),
                             _stream()), "dart_sma_bwd")
    return out


def dart_scan_bwd(x, dt, A, Bm, C, acum, H_in, dy, chunk, ddH=None, dh_final=None,
                  dC_sma=None, out=None):
    """Backward of the chunked scan (see include/dart.h).  Returns a dict of
    f32 device tensors dx [B,L,H,P], ddt [B,L,H], dA [H], dB, dC [B,L,G,N]
    (dC includes dC_sma when given) and dh0 [B,H,P,N]; ``out`` may hold
    preallocated ones plus "workspace"."""
    B, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    d = DartDims(B, L, H, G, N, P, int(chunk), _io_code(x.dtype))
    M, io, dev = L // chunk, x.dtype, x.device
    ws = int(lib().dart_scan_bwd_workspace(d))
    if ws == 0:
        raise ValueError("dart_scan_bwd: unsupported dimensions")
    f32 = dict(dtype=torch.float32, device=dev)
    if out is None:
        out = {"dx": torch.empty(B, L, H, P, **f32), "ddt": torch.empty(B, L, H, **f32),
               "dA": torch.empty(H, **f32), "dB": torch.empty(B, L, G, N, **f32),
               "dC": torch.empty(B, L, G, N, **f32), "dh0": torch.empty(B, H, P, N, **f32),
               "workspace": torch.empty(ws, dtype=torch.uint8, device=dev)}
    args = [_ptr(x, "x", io, (B, L, H, P), dev), _ptr(dt, "dt", torch.float32, (B, L, H), dev),
            _ptr(A, "A", torch.float32, (H,), dev), _ptr(Bm, "Bm", io, (B, L, G, N), dev),
            _ptr(C, "C", io, (B, L, G, N), dev),
            _ptr(acum, "acum", torch.float32, (B, H, M, chunk), dev),
            _ptr(H_in, "H_in", io, (B, H, M, P, N), dev), _ptr(dy, "dy", io, (B, L, H, P), dev),
            _ptr(ddH, "ddH", torch.float32, (B, H, M, P, N), dev),
            _ptr(dh_final, "dh_final", torch.float32, (B, H, P, N), dev),
            _ptr(dC_sma, "dC_sma", torch.float32, (B, L, G, N), dev)]
    outs = [_ptr(out["dx"], "dx", torch.float32, (B, L, H, P), dev),
            _ptr(out["ddt"], "ddt", torch.float32, (B, L, H), dev),
            _ptr(out["dA"], "dA", torch.float32, (H,), dev),
            _ptr(out["dB"], "dB", torch.float32, (B, L, G, N), dev),
            _ptr(out["dC"], "dC", torch.float32, (B, L, G, N), dev),
            _ptr(out["dh0"], "dh0", torch.float32, (B, H, P, N), dev)]
    wsp = _ptr(out["workspace"], "workspace", torch.uint8, None, dev)
    check(lib().dart_scan_bwd(d, *args, *outs, wsp, out["workspace"].numel(), _stream()),
          "dart_scan_bwd")
    return out


def decode_dims(batch, nheads, ngroups, dstate, headdim, chunk, max_chunks, dtype):
    return DartDecodeDims(batch, nheads, ngroups, dstate, headdim, int(chunk), int(max_chunks),
                          _io_code(dtype))


def dart_sma_decode_workspace(dims):
    """Workspace bytes for dart_sma_decode (0 for invalid dims)."""
    return int(lib().dart_sma_decode_workspace(dims))


def dart_sma_decode(x, dt, A, Bm, C, Q, E, gate, cache, h, dH_cur, n_chunks, pos, y,
                    workspace, chunk):
    """One decode step (see include/dart.h).  cache [B,H,max_chunks,P,N] io,
    h / dH_cur [B,H,P,N] f32, n_chunks / pos [B] int32 are updated in place;
    y [B,H,P] io is written; workspace is a uint8 device tensor."""
    B, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    max_chunks = cache.shape[2]
    io, dev = x.dtype, x.device
    d = decode_dims(B, H, G, N, P, chunk, max_chunks, io)
    args = [_ptr(x, "x", io, (B, H, P), dev), _ptr(dt, "dt", torch.float32, (B, H), dev),
            _ptr(A, "A", torch.float32, (H,), dev), _ptr(Bm, "Bm", io, (B, G, N), dev),
            _ptr(C, "C", io, (B, G, N), dev), _ptr(Q, "Q", io, (B, G, N), dev),
            _ptr(E, "E", io, (B, H, P), dev)]
    state = [_ptr(cache, "cache", io, (B, H, max_chunks, P, N), dev),
             _ptr(h, "h", torch.float32, (B, H, P, N), dev),
             _ptr(dH_cur, "dH_cur", torch.float32, (B, H, P, N), dev),
             _ptr(n_chunks, "n_chunks", torch.int32, (B,), dev),
             _ptr(pos, "pos", torch.int32, (B,), dev), _ptr(y, "y", io, (B, H, P), dev)]
    wsp = _ptr(workspace, "workspace", torch.uint8, None, dev)
    check(lib().dart_sma_decode(d, *args, float(gate), *state, wsp, workspace.numel(),
                                _stream()), "dart_sma_decode")


def dart_sma_decode_noalloc(x, dt, A, Bm, C, Q, E, gate, cache, h, dH_cur, n_chunks, pos, y,
                            chunk, cache_full=None):
    """dart_sma_decode without a workspace (see include/dart.h): the library
    keeps the step's partials in its static per-GPU scratch and allocates
    nothing.  cache_full: an int32 device tensor of one element set to 1
    when a chunk could not be appended (None: not reported).  Calls that may
    overlap on one GPU race on the scratch."""
    B, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    max_chunks = cache.shape[2]
    io, dev = x.dtype, x.device
    d = decode_dims(B, H, G, N, P, chunk, max_chunks, io)
    args = [_ptr(x, "x", io, (B, H, P), dev), _ptr(dt, "dt", torch.float32, (B, H), dev),
            _ptr(A, "A", torch.float32, (H,), dev), _ptr(Bm, "Bm", io, (B, G, N), dev),
            _ptr(C, "C", io, (B, G, N), dev), _ptr(Q, "Q", io, (B, G, N), dev),
            _ptr(E, "E", io, (B, H, P), dev)]
    state = [_ptr(cache, "cache", io, (B, H, max_chunks, P, N), dev),
             _ptr(h, "h", torch.float32, (B, H, P, N), dev),
             _ptr(dH_cur, "dH_cur", torch.float32, (B, H, P, N), dev),
             _ptr(n_chunks, "n_chunks", torch.int32, (B,), dev),
             _ptr(pos, "pos", torch.int32, (B,), dev), _ptr(y, "y", io, (B, H, P), dev)]
    flag = _ptr(cache_full, "cache_full", torch.int32, (1,), dev)
    check(lib().dart_sma_decode_noalloc(d, *args, float(gate), *state, flag, _stream()),
          "dart_sma_decode_noalloc")


def dart_sma_decode_fp8(x, dt, A, Bm, C, Q, E, gate, cache8, scale, h, dH_cur, n_chunks, pos,
                        y, workspace, chunk):
    """dart_sma_decode over the fp8 cache: cache8 [B,H,max_chunks,P,N] uint8
    E4M3 codes and scale [B,H,max_chunks] f32 (see include/dart.h)."""
    B, H, P = x.shape
    G, N = Bm.shape[1], Bm.shape[2]
    max_chunks = cache8.shape[2]
    io, dev = x.dtype, x.device
    d = decode_dims(B, H, G, N, P, chunk, max_chunks, io)
    args = [_ptr(x, "x", io, (B, H, P), dev), _ptr(dt, "dt", torch.float32, (B, H), dev),
            _ptr(A, "A", torch.float32, (H,), dev), _ptr(Bm, "Bm", io, (B, G, N), dev),
            _ptr(C, "C", io, (B, G, N), dev), _ptr(Q, "Q", io, (B, G, N), dev),
            _ptr(E, "E", io, (B, H, P), dev)]
    state = [_ptr(cache8, "cache8", torch.uint8, (B, H, max_chunks, P, N), dev),
             _ptr(scale, "scale", torch.float32, (B, H, max_chunks), dev),
             _ptr(h, "h", torch.float32, (B, H, P, N), dev),
             _ptr(dH_cur, "dH_cur", torch.float32, (B, H, P, N), dev),
             _ptr(n_chunks, "n_chunks", torch.int32, (B,), dev),
             _ptr(pos, "pos", torch.int32, (B,), dev), _ptr(y, "y", io, (B, H, P), dev)]
    wsp = _ptr(workspace, "workspace", torch.uint8, None, dev)
    check(lib().dart_sma_decode_fp8(d, *args, float(gate), *state, wsp, workspace.numel(),
                                    _stream()), "dart_sma_decode_fp8")


def dart_cache_fp8_store(dH_f32, first, cache8, scale, ngroups, chunk, io):
    """Encode dH_f32 [B,H,n_mem,P,N] f32 into fp8 cache slots first ..
    first + n_mem - 1 of cache8 [B,H,max_chunks,P,N] uint8 and scale
    [B,H,max_chunks] f32.  ngroups, chunk and io are the decode dims the
    cache serves (validated only)."""
    B, H, n_mem, P, N = dH_f32.shape
    max_chunks, dev = cache8.shape[2], dH_f32.device
    d = decode_dims(B, H, ngroups, N, P, chunk, max_chunks, io)
    args = [_ptr(dH_f32, "dH_f32", torch.float32, (B, H, n_mem, P, N), dev), int(n_mem),
            int(first), _ptr(cache8, "cache8", torch.uint8, (B, H, max_chunks, P, N), dev),
            _ptr(scale, "scale", torch.float32, (B, H, max_chunks), dev)]
    check(lib().dart_cache_fp8_store(d, *args, _stream()), "dart_cache_fp8_store")


# ----------------------------------------------------------------- helpers
def prefill(x, dt, A, Bm, C, Q, E, gate, chunk, h0=None, decayed=False, one_pass=False):
    """Whole prefill path; returns a dict of device tensors: y, y_ssd, dH
    ([B,H,M,P,N] io), H_in ([B,H,M,P,N] io, the state entering each chunk),
    h_final ([B,H,P,N] f32, the state after the last chunk), acum and dH_f32
    (the unrounded memories).  one_pass runs the scan as dart_chunk_scan +
    dart_chunk_out: the same outputs bit for bit, without dH_f32 (an 8 MB
    workspace instead of the f32 memories; about 1% slower per step at the
    ~370M layer shape)."""
    B, L, H, P = x.shape
    N = Bm.shape[3]
    M, dev = L // chunk, x.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = {
        "acum": torch.empty(B, H, M, chunk, **f32),
        "dH": torch.empty(B, H, M, P, N, dtype=x.dtype, device=dev),
        "H_in": torch.empty(B, H, M, P, N, dtype=x.dtype, device=dev),
        "h_final": torch.empty(B, H, P, N, **f32),
        "y_ssd": torch.empty(B, L, H, P, dtype=x.dtype, device=x.device),
        "y": torch.empty(B, L, H, P, dtype=x.dtype, device=dev),
    }
    if not one_pass:
        out["dH_f32"] = torch.empty(B, H, M, P, N, **f32)
    _scan(out, x, dt, A, Bm, C, chunk, h0, one_pass)
    if decayed:
        dart_sma_fwd_decayed(Q, E, C, out["dH"], out["acum"], out["y_ssd"], gate, out["y"], chunk)
    else:
        dart_sma_fwd(Q, E, C, out["dH"], out["y_ssd"], gate, out["y"], chunk)
    return out


def prefill_train(x, dt, A, Bm, C, Q, E, gate, chunk, h0=None, one_pass=False):
    """:func:`prefill` that also keeps what the backward reads: o [B,L,H,P]
    f32 and lse [B,H,L] f32 (dart_sma_fwd_train)."""
    B, L, H, P = x.shape
    N = Bm.shape[3]
    M, dev = L // chunk, x.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = {
        "acum": torch.empty(B, H, M, chunk, **f32),
        "dH": torch.empty(B, H, M, P, N, dtype=x.dtype, device=dev),
        "H_in": torch.empty(B, H, M, P, N, dtype=x.dtype, device=dev),
        "h_final": torch.empty(B, H, P, N, **f32),
        "y_ssd": torch.empty(B, L, H, P, dtype=x.dtype, device=dev),
        "y": torch.empty(B, L, H, P, dtype=x.dtype, device=dev),
        "o": torch.empty(B, L, H, P, **f32),
        "lse": torch.empty(B, H, L, **f32),
    }
    if not one_pass:
        out["dH_f32"] = torch.empty(B, H, M, P, N, **f32)
    _scan(out, x, dt, A, Bm, C, chunk, h0, one_pass)
    dart_sma_fwd_train(Q, E, C, out["dH"], out["y_ssd"], gate, out["y"], out["o"], out["lse"],
                       chunk)
    return out


def prefill_backward(fwd, x, dt, A, Bm, C, Q, E, gate, chunk, dy, dh_final=None):
    """Gradients of the whole prefill (SMA, gated add and the chunked scan)
    for an upstream gradient dy [B,L,H,P] of y (and optionally dh_final of
    the final state), from the tensors :func:`prefill_train` returned.
    Returns f32 tensors dx, ddt, dA, dB, dC, dQ, dE, dgate and dh0."""
    sm = dart_sma_bwd(Q, E, C, fwd["dH"], fwd["o"], fwd["lse"], dy, gate, chunk)
    sc = dart_scan_bwd(x, dt, A, Bm, C, fwd["acum"], fwd["H_in"], dy, chunk, ddH=sm["ddH"],
                       dh_final=dh_final, dC_sma=sm["dC"])
    return {"dx": sc["dx"], "ddt": sc["ddt"], "dA": sc["dA"], "dB": sc["dB"], "dC": sc["dC"],
            "dQ": sm["dQ"], "dE": sm["dE"], "dgate": sm["dgate"], "dh0": sc["dh0"]}


def prefill_continue(x, dt, A, Bm, C, Q, E, gate, chunk, cache, prior_chunks, h0, scale=None):
    """Chunked prefill: the tokens are chunks prior_chunks, prior_chunks+1, ...
    of sequences whose first prior_chunks memories are in ``cache``
    [B,H,max_chunks,P,N] (the decode cache: io-typed, or uint8 fp8 codes with
    their ``scale`` [B,H,max_chunks]) and whose state after them is ``h0``
    [B,H,P,N] f32.  Returns the dict of :func:`prefill` for the new tokens;
    the new memories (out["dH"]) are not written into the cache."""
    if (cache.dtype == torch.uint8) != (scale is not None):
        raise ValueError("an fp8 cache (uint8) needs its scale, and only it takes one")
    B, L, H, P = x.shape
    N = Bm.shape[3]
    M, dev = L // chunk, x.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = {
        "acum": torch.empty(B, H, M, chunk, **f32),
        "dH": torch.empty(B, H, M, P, N, dtype=x.dtype, device=dev),
        "dH_f32": torch.empty(B, H, M, P, N, **f32),
        "H_in": torch.empty(B, H, M, P, N, dtype=x.dtype, device=dev),
        "h_final": torch.empty(B, H, P, N, **f32),
        "y_ssd": torch.empty(B, L, H, P, dtype=x.dtype, device=dev),
        "y": torch.empty(B, L, H, P, dtype=x.dtype, device=dev),
    }
    dart_chunk_state(x, dt, A, Bm, out["acum"], out["dH"], out["dH_f32"], chunk)
    dart_state_pass(x, dt, Bm, C, out["acum"], out["dH_f32"], h0, out["H_in"], out["h_final"],
                    out["y_ssd"], chunk)
    if scale is not None:
        dart_sma_fwd_cont_fp8(Q, E, C, cache, scale, prior_chunks, out["dH"], out["y_ssd"], gate,
                              out["y"], chunk)
    else:
        dart_sma_fwd_cont(Q, E, C, cache, prior_chunks, out["dH"], out["y_ssd"], gate, out["y"],
                          chunk)
    return out


def new_decode_state(batch, nheads, ngroups, dstate, headdim, chunk, max_chunks, dtype, device,
                     fp8_cache=False):
    """Zeroed decode state: the cache ("cache" in the io type, or with
    fp8_cache "cache8" codes and "scale"), h, dH_cur, n_chunks, pos and
    workspace."""
    dims = decode_dims(batch, nheads, ngroups, dstate, headdim, chunk, max_chunks, dtype)
    ws = dart_sma_decode_workspace(dims)
    if ws == 0:
        raise ValueError("unsupported decode dimensions")
    f32 = dict(dtype=torch.float32, device=device)
    shape = (batch, nheads, max_chunks, headdim, dstate)
    if fp8_cache:
        cache = {"cache8": torch.zeros(shape, dtype=torch.uint8, device=device),
                 "scale": torch.ones(batch, nheads, max_chunks, **f32)}
    else:
        cache = {"cache": torch.zeros(shape, dtype=dtype, device=device)}
    return {
        "chunk": int(chunk),
        "ngroups": int(ngroups),
        "io": dtype,
        **cache,
        "h": torch.zeros(batch, nheads, headdim, dstate, **f32),
        "dH_cur": torch.zeros(batch, nheads, headdim, dstate, **f32),
        "n_chunks": torch.zeros(batch, dtype=torch.int32, device=device),
        "pos": torch.zeros(batch, dtype=torch.int32, device=device),
        "workspace": torch.zeros(ws, dtype=torch.uint8, device=device),
    }


def cache_overflowed(state):
    """True once a decode step on ``state`` closed a chunk while its sequence's
    cache was full: that chunk's memory was dropped (n_chunks stays at
    max_chunks), so later tokens of the sequence attend an incomplete set of
    memories.  Reads the flag the library keeps in the first int32 of the
    workspace, which is a device-to-host copy and synchronises the stream."""
    return bool(state["workspace"][:4].view(torch.int32).item())


def decode_step(state, x, dt, A, Bm, C, Q, E, gate, y=None, check_overflow=False):
    """Advance ``state`` (from new_decode_state) by one token per sequence;
    returns y [B,H,P].  A full cache does not stop the step (see
    :func:`cache_overflowed`); with ``check_overflow`` the step raises
    RuntimeError once that has happened, at the price of a synchronisation
    per call.  Without it, callers poll cache_overflowed themselves."""
    if y is None:
        y = torch.empty(x.shape, dtype=x.dtype, device=x.device)
    if "cache8" in state:
        dart_sma_decode_fp8(x, dt, A, Bm, C, Q, E, gate, state["cache8"], state["scale"],
                            state["h"], state["dH_cur"], state["n_chunks"], state["pos"], y,
                            state["workspace"], state["chunk"])
    else:
        dart_sma_decode(x, dt, A, Bm, C, Q, E, gate, state["cache"], state["h"],
                        state["dH_cur"], state["n_chunks"], state["pos"], y, state["workspace"],
                        state["chunk"])
    if check_overflow and cache_overflowed(state):
        raise RuntimeError("decode cache full: a finished chunk's memory could not be appended "
                           "(allocate the state with a larger max_chunks)")
    return y


def store_memories(state, dH_f32, dH=None, first=0):
    """Put memories into the decode cache at slots first, first + 1, ...:
    the f32 memories dH_f32 [B,H,n,P,N] are encoded into an fp8 cache; an
    io cache takes dH [B,H,n,P,N] (the io-typed memories of the prefill)."""
    n = dH_f32.shape[2]
    if "cache8" in state:
        dart_cache_fp8_store(dH_f32, first, state["cache8"], state["scale"], state["ngroups"],
                             state["chunk"], state["io"])
    else:
        state["cache"][:, :, first:first + n].copy_(dH)
