"""DART hot path on AMD Instinct MI355X (gfx950): chunked scan, chunk state
memories, state-memory attention and decode, as HIP kernels behind the C ABI
in include/dart.h.  The shared library is loaded on first use and a missing
build raises; there is no fallback path."""

from .api import (  # noqa: F401
    dart_chunk_state,
    dart_sma_decode,
    dart_sma_decode_workspace,
    dart_sma_fwd,
    cache_overflowed,
    dart_state_pass,
    decode_dims,
    decode_step,
    new_decode_state,
    prefill,
    prefill_dims,
)
from ._lib import DartError, lib  # noqa: F401
