"""C-ABI checks that need no GPU: the library loads, exports every function
include/dart.h declares, and rejects bad arguments on the host before any
HIP call (error paths only; no compute call is made here)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch

import ssm_state_attention_amd as dart
from ssm_state_attention_amd import _lib, api
from ssm_state_attention_amd._lib import DartDecodeDims, DartDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dart.h")

OK, NULLP, BAD, UNSUP, DTYPE, WS, HIP, ALIGN, SCRATCH = range(9)
F32, BF16 = 0, 1


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\*\s]+?)\b(dart_\w+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("dart_chunk_state", "dart_state_pass", "dart_sma_fwd", "dart_sma_decode"):
        assert n in names


def test_library_exports_every_declared_function():
    lib = dart.lib()
    for name in declared_functions():
        assert hasattr(lib, name), f"libdart.so does not export {name}"
    if shutil.which("nm"):
        out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                             capture_output=True, text=True, check=True).stdout
        exported = set(re.findall(r"\bT (dart_\w+)", out))
        assert set(declared_functions()) <= exported


def test_status_strings():
    lib = dart.lib()
    for code in range(9):
        s = lib.dart_status_str(code).decode()
        assert s.startswith("DART_") and s == s.strip()
    assert lib.dart_status_str(99).decode() == "DART_ERR_UNKNOWN"


def dims(B=1, L=1024, H=1, G=1, N=16, P=16, S=64, io=F32):
    return DartDims(B, L, H, G, N, P, S, io)


@pytest.mark.parametrize("d", [
    dims(),                                         # tiny fp32 layer
    dims(1, 4096, 8, 8, 128, 64, 256, BF16),        # L=4K bf16 prefill
    dims(4, 8192, 32, 4, 128, 64, 256, BF16),       # ~370M layer shape
    dims(1, 65536, 32, 32, 128, 64, 256, BF16),     # long context
    dims(2, 96, 3, 3, 32, 32, 96, F32),
    dims(1, 512, 2, 2, 128, 128, 256, BF16),
])
def test_validate_accepts(d):
    assert dart.lib().dart_validate_dims(d) == OK


@pytest.mark.parametrize("d,code", [
    (dims(B=0), BAD), (dims(L=-64), BAD), (dims(H=0), BAD), (dims(S=0), BAD),
    (dims(L=1000), BAD),                            # L % S != 0
    (dims(H=3, G=2), BAD),                          # H % G != 0
    (dims(N=16, P=32), UNSUP),                      # shape not compiled
    (dims(N=16, P=16, io=BF16), UNSUP),             # bf16 needs N >= 32
    (dims(S=48, L=960), UNSUP),                     # S % 32 != 0
    (dims(S=512, L=1024), UNSUP),                   # S > 256
    (dims(io=7), DTYPE),
    (dims(B=70000, L=64, S=64), BAD),               # grid limit
])
def test_validate_rejects(d, code):
    assert dart.lib().dart_validate_dims(d) == code


def test_validate_null():
    assert dart.lib().dart_validate_dims(None) == NULLP
    assert dart.lib().dart_validate_decode_dims(None) == NULLP


def ddims(B=64, H=32, G=32, N=128, P=64, S=256, mx=128, io=BF16):
    return DartDecodeDims(B, H, G, N, P, S, mx, io)


def test_decode_workspace():
    lib = dart.lib()
    for d in (ddims(), ddims(2, 4, 4, 128, 64, 256, 8), ddims(1, 1, 1, 16, 16, 64, 3, F32)):
        assert lib.dart_validate_decode_dims(d) == OK
        ws = api.dart_sma_decode_workspace(d)
        assert ws > 0 and ws % 256 == 0
    assert api.dart_sma_decode_workspace(ddims(mx=0)) == 0
    assert lib.dart_validate_decode_dims(ddims(H=6, G=4)) == BAD
    assert lib.dart_validate_decode_dims(ddims(N=96)) == UNSUP


# Fake device addresses: never dereferenced, because every call below fails
# host-side validation before any HIP call.
A16 = 0x10000
MIS = 0x10004


def test_entry_points_reject_null_pointers():
    lib = dart.lib()
    d = dims()
    p = [A16] * 7
    for i in range(7):
        q = list(p)
        q[i] = None
        assert lib.dart_chunk_state(d, *q, None) == NULLP
    # x, dt, Bm, C, acum, dH_f32, h0 (may be NULL), H_in, h_final, y_ssd
    for i in (0, 1, 2, 3, 4, 5, 7, 8, 9):
        q = [A16] * 10
        q[6] = None
        q[i] = None
        assert lib.dart_state_pass(d, *q, None) == NULLP
    assert lib.dart_sma_fwd(d, A16, A16, None, A16, A16, 0.5, A16, None) == NULLP


def test_entry_points_reject_misaligned_pointers():
    lib = dart.lib()
    d = dims()
    assert lib.dart_chunk_state(d, A16, A16, A16, MIS, A16, A16, A16, None) == ALIGN
    assert lib.dart_state_pass(d, A16, A16, A16, A16, A16, A16, MIS, A16, A16, A16,
                               None) == ALIGN
    assert lib.dart_sma_fwd(d, A16, A16, A16, A16, A16, 0.5, MIS, None) == ALIGN


def test_entry_points_reject_bad_dims_before_pointers():
    lib = dart.lib()
    assert lib.dart_sma_fwd(dims(L=1000), None, None, None, None, None, 0.5, None,
                            None) == BAD
    assert lib.dart_chunk_state(dims(N=16, P=32), *([A16] * 7), None) == UNSUP


def test_decode_rejects_small_workspace():
    lib = dart.lib()
    d = ddims(2, 4, 4, 128, 64, 256, 8)
    need = api.dart_sma_decode_workspace(d)
    args = [A16] * 7
    state = [A16] * 6
    assert lib.dart_sma_decode(d, *args, 0.5, *state, A16, need - 256, None) == WS
    assert lib.dart_sma_decode(d, *args, 0.5, *state, None, need, None) == WS
    assert lib.dart_sma_decode(d, *args, 0.5, *state, MIS, need, None) == ALIGN


def test_fp8_cache_entry_points_validate_on_host():
    lib = dart.lib()
    d = ddims(2, 4, 4, 128, 64, 256, 8)
    need = api.dart_sma_decode_workspace(d)
    args = [A16] * 7
    # cache8, scale, h, dH_cur, n_chunks, pos, y
    for i in range(7):
        state = [A16] * 7
        state[i] = None
        assert lib.dart_sma_decode_fp8(d, *args, 0.5, *state, A16, need, None) == NULLP
    state = [A16] * 7
    assert lib.dart_sma_decode_fp8(d, *args, 0.5, *state, A16, need - 256, None) == WS
    state[1] = MIS
    assert lib.dart_sma_decode_fp8(d, *args, 0.5, *state, A16, need, None) == ALIGN
    assert lib.dart_sma_decode_fp8(ddims(N=96), *args, 0.5, *([A16] * 7), A16, need,
                                   None) == UNSUP
    # store: 0 <= n_mem, 0 <= first <= max_chunks - n_mem
    st = lib.dart_cache_fp8_store
    assert st(d, A16, -1, 0, A16, A16, None) == BAD
    assert st(d, A16, 2, -1, A16, A16, None) == BAD
    assert st(d, A16, 9, 0, A16, A16, None) == BAD
    assert st(d, A16, 4, 5, A16, A16, None) == BAD
    assert st(d, None, 8, 0, A16, A16, None) == NULLP
    assert st(d, A16, 8, 0, A16, None, None) == NULLP
    assert st(d, A16, 8, 0, MIS, A16, None) == ALIGN
    assert st(ddims(mx=0), A16, 0, 0, A16, A16, None) == BAD


def test_fp8_continuation_validates_on_host():
    lib = dart.lib()
    cont = lib.dart_sma_fwd_cont_fp8
    d = dims(2, 512, 4, 2, 128, 64, 128, BF16)
    # Q, E, C, cache8, scale, dH, y_ssd, gate, y
    for i in range(8):
        p = [A16] * 8
        p[i] = None
        assert cont(d, 3, 5, *p[:7], 0.5, p[7], None) == NULLP
    p = [A16] * 8
    p[3] = p[4] = MIS
    assert cont(d, 3, 5, *p[:7], 0.5, p[7], None) == ALIGN
    # (a NULL cache with prior_chunks = 0 passes validation and would launch:
    # not called here)
    assert cont(d, 6, 5, *([A16] * 7), 0.5, A16, None) == BAD
    assert cont(d, -1, 5, *([A16] * 7), 0.5, A16, None) == BAD
    assert cont(dims(2, 512, 4, 2, 32, 32, 128, F32), 1, 5, *([A16] * 7), 0.5, A16,
                None) == UNSUP
    assert cont(dims(2, 512, 4, 2, 96, 64, 128, BF16), 1, 5, *([A16] * 7), 0.5, A16,
                None) == UNSUP


def test_backward_entry_points_validate_on_host():
    lib = dart.lib()
    d = dims(2, 512, 4, 2, 128, 64, 128, BF16)
    ws_sma, ws_scan = lib.dart_sma_bwd_workspace(d), lib.dart_scan_bwd_workspace(d)
    assert ws_sma > 0 and ws_sma % 256 == 0 and ws_scan > 0
    # f32 io: the plain f32 kernels' workspaces (dgate partials and the
    # factor pairs; du, the two state-gradient arrays and the dA partials)
    f = dims(1, 1024, 1, 1, 16, 16, 64, F32)
    M = 16
    assert lib.dart_sma_bwd_workspace(f) == 256 + 1 * 64 * M * (M - 1) // 2 * 8
    assert lib.dart_scan_bwd_workspace(f) == 4096 + 2 * (M * 256 * 4) + 256
    # unsupported: P = 128, 32-token chunks (bf16)
    for bad in (dims(1, 512, 2, 2, 128, 128, 256, BF16), dims(1, 1024, 2, 2, 128, 64, 32, BF16)):
        assert lib.dart_sma_bwd_workspace(bad) == 0 and lib.dart_scan_bwd_workspace(bad) == 0
        assert lib.dart_sma_bwd(bad, *([A16] * 7), 0.5, *([A16] * 5), A16, 1 << 30,
                                None) == UNSUP
        assert lib.dart_scan_bwd(bad, *([A16] * 8), None, None, None, *([A16] * 6), A16,
                                 1 << 30, None) == UNSUP
    # Q, E, C, dH, o, lse, dy, then dQ, dE, dC, ddH, dgate
    for i in range(12):
        p = [A16] * 12
        p[i] = None
        assert lib.dart_sma_bwd(d, *p[:7], 0.5, *p[7:], A16, ws_sma, None) == NULLP
    assert lib.dart_sma_bwd(d, *([A16] * 7), 0.5, *([A16] * 5), A16, ws_sma - 256, None) == WS
    assert lib.dart_sma_bwd(d, *([A16] * 7), 0.5, *([A16] * 5), MIS, ws_sma, None) == ALIGN
    # x, dt, A, Bm, C, acum, H_in, dy, (ddH, dh_final, dC_sma optional), dx .. dh0
    for i in range(14):
        p = [A16] * 14
        p[i] = None
        assert lib.dart_scan_bwd(d, *p[:8], None, None, None, *p[8:], A16, ws_scan,
                                 None) == NULLP
    assert lib.dart_scan_bwd(d, *([A16] * 8), MIS, None, None, *([A16] * 6), A16, ws_scan,
                             None) == ALIGN
    assert lib.dart_scan_bwd(d, *([A16] * 8), None, None, None, *([A16] * 6), A16,
                             ws_scan - 256, None) == WS


def test_binding_checks_tensors_before_calling():
    x = torch.zeros(1, 64, 1, 16)
    with pytest.raises(ValueError, match="GPU"):
        api.dart_chunk_state(x, torch.zeros(1, 64, 1), torch.zeros(1), torch.zeros(1, 64, 1, 16),
                             torch.zeros(1, 1, 1, 64), torch.zeros(1, 1, 1, 16, 16),
                             torch.zeros(1, 1, 1, 16, 16), 64)
    with pytest.raises(TypeError):
        api.prefill_dims(torch.zeros(1, 64, 1, 16, dtype=torch.float16),
                         torch.zeros(1, 64, 1, 16), 64)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libdart.so"))
    with pytest.raises(RuntimeError, match="must be built"):
        _lib.lib()


VALIDATE_DRIVER = r"""
#include <stdio.h>
#include "dart.h"
int main(void) {
  dart_dims d = {4, 8192, 32, 4, 128, 64, 256, DART_BF16};
  int bad = 0;
  bad |= dart_validate_dims(&d) != DART_OK;
  d.seqlen = 8000; bad |= dart_validate_dims(&d) != DART_ERR_BAD_DIMS;
  d.seqlen = 8192; d.dstate = 100; bad |= dart_validate_dims(&d) != DART_ERR_UNSUPPORTED;
  dart_decode_dims dd = {64, 32, 32, 128, 64, 256, 128, DART_BF16};
  bad |= dart_sma_decode_workspace(&dd) == 0;
  for (int s = -1; s < 10; ++s) bad |= dart_status_str((dart_status)s) == 0;
  printf("%s\n", bad ? "FAIL" : "OK");
  return bad;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_validators_under_host_sanitizers(tmp_path):
    """The host validation code, built without HIP under ASan/UBSan."""
    drv = tmp_path / "drv.c"
    drv.write_text(VALIDATE_DRIVER)
    exe = tmp_path / "drv"
    csrc = os.path.join(ROOT, "ssm_state_attention_amd", "csrc")
    subprocess.run(["g++", "-x", "c++", str(drv), "-x", "c++",
                    os.path.join(csrc, "dart_validate.cpp"), "-I", os.path.join(ROOT, "include"),
                    "-I", csrc, "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-g", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "OK", out.stdout + out.stderr


def test_decode_noalloc_validates_on_host():
    """The allocation-free decode entry point rejects bad arguments, and dims
    whose scratch need exceeds DART_DECODE_SCRATCH_BYTES, before any HIP
    call (so before its first look-up of the device scratch)."""
    lib = dart.lib()
    fn = lib.dart_sma_decode_noalloc
    d = ddims()
    # x, dt, A, Bm, C, Q, E, gate, cache, h, dH_cur, n_chunks, pos, y, cache_full
    for i in range(13):
        p = [A16] * 13
        p[i] = None
        assert fn(d, *p[:7], 0.5, *p[7:], None, None) == NULLP
    p = [A16] * 13
    p[8] = MIS
    assert fn(d, *p[:7], 0.5, *p[7:], None, None) == ALIGN
    assert fn(d, *p[:7], 0.5, *([A16] * 6), A16 + 2, None) == ALIGN   # cache_full not 4-aligned
    assert fn(ddims(H=6, G=4), *([A16] * 7), 0.5, *([A16] * 6), None, None) == BAD
    assert fn(ddims(N=96), *([A16] * 7), 0.5, *([A16] * 6), None, None) == UNSUP
    # the scratch bound: the largest batch that fits is accepted by the size
    # rule, one more sequence is rejected
    cap = _lib.DECODE_SCRATCH_BYTES
    fits = [B for B in range(200, 300) if api.dart_sma_decode_workspace(ddims(B=B)) <= cap]
    big = max(fits) + 1
    assert api.dart_sma_decode_workspace(ddims(B=big)) > cap
    assert fn(ddims(B=big), *([A16] * 7), 0.5, *([A16] * 6), None, None) == SCRATCH
    assert "DART_ERR_SCRATCH" in lib.dart_status_str(SCRATCH).decode()


def test_chunk_scan_workspace_sizes():
    """16-bit io: 256 bytes of failure words, an 8-byte flag per (batch, head)
    rounded to 256 bytes, two f32 state slots per (batch, head); f32 io: the
    f32 memories of every chunk."""
    B, L, H, G, N, P, S = 4, 8192, 32, 4, 128, 64, 256
    got = api.dart_chunk_scan_workspace(dims(B, L, H, G, N, P, S, BF16))
    assert got == 256 + 1024 + B * H * 2 * N * P * 4
    got = api.dart_chunk_scan_workspace(dims(1, 1024, 2, 1, 16, 16, 64, F32))
    assert got == 2 * 16 * 16 * 16 * 4
    assert api.dart_chunk_scan_workspace(dims(L=1000)) == 0


def test_chunk_scan_and_chunk_out_reject_bad_arguments():
    lib = dart.lib()
    d = dims(1, 1024, 2, 1, 128, 64, 256, BF16)
    need = api.dart_chunk_scan_workspace(d)
    # x, dt, A, Bm, h0 (may be NULL), acum, dH, dH_f32 (may be NULL), H_in, h_final
    for i in (0, 1, 2, 3, 5, 6, 8, 9):
        q = [A16] * 10
        q[4] = q[7] = None
        q[i] = None
        assert lib.dart_chunk_scan(d, *q, A16, need, None) == NULLP
    q = [A16] * 10
    assert lib.dart_chunk_scan(d, *q, None, need, None) == WS
    assert lib.dart_chunk_scan(d, *q, A16, need - 256, None) == WS
    assert lib.dart_chunk_scan(d, *q, MIS, need, None) == ALIGN
    q[4] = MIS
    assert lib.dart_chunk_scan(d, *q, A16, need, None) == ALIGN
    q[4], q[7] = A16, MIS
    assert lib.dart_chunk_scan(d, *q, A16, need, None) == ALIGN
    assert lib.dart_chunk_scan(dims(N=16, P=32), *([A16] * 10), A16, need, None) == UNSUP
    for i in range(7):
        q = [A16] * 7
        q[i] = None
        assert lib.dart_chunk_out(d, *q, None) == NULLP
    q = [A16] * 7
    q[5] = MIS
    assert lib.dart_chunk_out(d, *q, None) == ALIGN
