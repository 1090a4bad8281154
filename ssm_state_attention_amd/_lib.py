"""ctypes view of libdart.so (the C ABI declared in include/dart.h)."""

import ctypes
import os

from ._build import LIB_PATH

DART_F32, DART_BF16 = 0, 1

STATUS_NAMES = {
    0: "DART_OK", 1: "DART_ERR_NULL_PTR", 2: "DART_ERR_BAD_DIMS", 3: "DART_ERR_UNSUPPORTED",
    4: "DART_ERR_DTYPE", 5: "DART_ERR_WORKSPACE", 6: "DART_ERR_HIP", 7: "DART_ERR_ALIGN",
    8: "DART_ERR_SCRATCH",
}

# DART_DECODE_SCRATCH_BYTES of include/dart.h: the static scratch behind
# dart_sma_decode_noalloc
DECODE_SCRATCH_BYTES = 4 << 20


class DartDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("io", ctypes.c_int32)]


class DartDecodeDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("chunk", ctypes.c_int64),
                ("max_chunks", ctypes.c_int64), ("io", ctypes.c_int32)]


class DartError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}")


_VP = ctypes.c_void_p
_F = ctypes.c_float
_SIG = {
    "dart_chunk_state": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "dart_state_pass": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                        _VP, _VP],
    "dart_chunk_scan_workspace": [ctypes.POINTER(DartDims)],
    "dart_chunk_scan": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                        _VP, _VP, ctypes.c_size_t, _VP],
    "dart_chunk_out": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "dart_sma_fwd": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _F, _VP, _VP],
    "dart_sma_fwd_decayed": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _VP, _F, _VP,
                             _VP],
    "dart_sma_fwd_cont": [ctypes.POINTER(DartDims), ctypes.c_int64, ctypes.c_int64, _VP, _VP,
                          _VP, _VP, _VP, _VP, _F, _VP, _VP],
    "dart_sma_fwd_cont_fp8": [ctypes.POINTER(DartDims), ctypes.c_int64, ctypes.c_int64, _VP,
                              _VP, _VP, _VP, _VP, _VP, _VP, _F, _VP, _VP],
    "dart_sma_decode_workspace": [ctypes.POINTER(DartDecodeDims)],
    "dart_sma_decode": [ctypes.POINTER(DartDecodeDims), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F,
                        _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "dart_sma_decode_noalloc": [ctypes.POINTER(DartDecodeDims), _VP, _VP, _VP, _VP, _VP, _VP,
                                _VP, _F, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "dart_sma_decode_fp8": [ctypes.POINTER(DartDecodeDims), _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                            _F, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "dart_cache_fp8_store": [ctypes.POINTER(DartDecodeDims), _VP, ctypes.c_int64, ctypes.c_int64,
                             _VP, _VP, _VP],
    "dart_sma_fwd_train": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _F, _VP, _VP, _VP,
                           _VP],
    "dart_sma_bwd_workspace": [ctypes.POINTER(DartDims)],
    "dart_sma_bwd": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _F, _VP, _VP,
                     _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "dart_scan_bwd_workspace": [ctypes.POINTER(DartDims)],
    "dart_scan_bwd": [ctypes.POINTER(DartDims), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                      _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "dart_validate_dims": [ctypes.POINTER(DartDims)],
    "dart_validate_decode_dims": [ctypes.POINTER(DartDecodeDims)],
    "dart_status_str": [ctypes.c_int],
}
_RES = {"dart_sma_decode_workspace": ctypes.c_size_t, "dart_chunk_scan_workspace": ctypes.c_size_t, "dart_sma_bwd_workspace": ctypes.c_size_t,
        "dart_scan_bwd_workspace": ctypes.c_size_t,
        "dart_status_str": ctypes.c_char_p}

_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: the HIP extension must be built "
                "(ssm_state_attention_amd._build.build_library())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIG.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = _RES.get(name, ctypes.c_int)
        _lib = handle
    return _lib


def check(status, where):
    if status != 0:
        raise DartError(status, where)
