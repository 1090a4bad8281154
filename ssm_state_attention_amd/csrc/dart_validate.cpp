// Host-side validation of the DART C ABI.  Pure C++ with no HIP call, so it
// runs (and is tested) on machines without a GPU.
#include "dart.h"
#include "dart_shapes.hpp"

extern "C" const char* dart_status_str(dart_status s) {
  switch (s) {
    case DART_OK: return "DART_OK";
    case DART_ERR_NULL_PTR: return "DART_ERR_NULL_PTR: a required pointer is NULL";
    case DART_ERR_BAD_DIMS: return "DART_ERR_BAD_DIMS: inconsistent or non-positive dimensions";
    case DART_ERR_UNSUPPORTED: return "DART_ERR_UNSUPPORTED: (dtype, N, P, S) not in the compiled set";
    case DART_ERR_DTYPE: return "DART_ERR_DTYPE: unknown element type";
    case DART_ERR_WORKSPACE: return "DART_ERR_WORKSPACE: decode workspace missing or too small";
    case DART_ERR_HIP: return "DART_ERR_HIP: a HIP launch failed";
    case DART_ERR_ALIGN: return "DART_ERR_ALIGN: a pointer is not 16-byte aligned";
    case DART_ERR_SCRATCH:
      return "DART_ERR_SCRATCH: the dims need more decode scratch than the allocation-free "
             "entry point's static maximum (DART_DECODE_SCRATCH_BYTES)";
  }
  return "DART_ERR_UNKNOWN";
}

namespace dart {

bool shape_supported(int io, int64_t N, int64_t P) {
  if (io == DART_F32) return (N == 16 && P == 16) || (N == 32 && P == 32);
  if (io == DART_BF16)
    return (N == 32 && P == 32) || (N == 64 && P == 64) || (N == 128 && P == 64) ||
           (N == 128 && P == 128);
  return false;
}

bool chunk_supported(int64_t S) { return S >= kMinChunk && S <= kMaxChunk && S % 32 == 0; }

int decode_splits(const dart_decode_dims& d) {
  const int64_t pairs = d.batch * d.nheads;
  if (pairs >= kDecodeTargetBlocks) return 1;
  int64_t s = (kDecodeTargetBlocks + pairs - 1) / pairs;
  const int64_t cap = (d.max_chunks + 3) / 4;  // at least ~4 chunks per split
  if (s > cap) s = cap;
  return s < 1 ? 1 : static_cast<int>(s);
}

size_t decode_workspace_bytes(const dart_decode_dims& d) {
  const int splits = decode_splits(d);
  const size_t pairs = static_cast<size_t>(d.batch * d.nheads);
  size_t bytes = 256;                                                   // status flag
  bytes += ((static_cast<size_t>(d.batch) * sizeof(int32_t) + 255) / 256) * 256;  // n_chunks copy
  bytes += ((pairs * d.headdim * sizeof(float) + 255) / 256) * 256;     // y_ssd
  bytes += ((pairs * splits * (d.headdim + 2) * sizeof(float) + 255) / 256) * 256;
  return bytes;
}

}  // namespace dart

extern "C" dart_status dart_validate_dims(const dart_dims* d) {
  if (!d) return DART_ERR_NULL_PTR;
  if (d->io != DART_F32 && d->io != DART_BF16) return DART_ERR_DTYPE;
  if (d->batch <= 0 || d->seqlen <= 0 || d->nheads <= 0 || d->ngroups <= 0 ||
      d->dstate <= 0 || d->headdim <= 0 || d->chunk <= 0)
    return DART_ERR_BAD_DIMS;
  if (d->nheads % d->ngroups != 0 || d->seqlen % d->chunk != 0) return DART_ERR_BAD_DIMS;
  // index arithmetic inside the kernels is 32-bit per (batch, head) pair and
  // 64-bit across pairs; keep every per-pair extent well inside int32
  if (d->seqlen > (int64_t(1) << 24) || d->batch * d->nheads > (int64_t(1) << 24) ||
      d->batch > 65535 || d->nheads > 65535)  // grid y/z limits
    return DART_ERR_BAD_DIMS;
  if (!dart::shape_supported(d->io, d->dstate, d->headdim) || !dart::chunk_supported(d->chunk))
    return DART_ERR_UNSUPPORTED;
  return DART_OK;
}

extern "C" dart_status dart_validate_decode_dims(const dart_decode_dims* d) {
  if (!d) return DART_ERR_NULL_PTR;
  if (d->io != DART_F32 && d->io != DART_BF16) return DART_ERR_DTYPE;
  if (d->batch <= 0 || d->nheads <= 0 || d->ngroups <= 0 || d->dstate <= 0 ||
      d->headdim <= 0 || d->chunk <= 0 || d->max_chunks <= 0)
    return DART_ERR_BAD_DIMS;
  if (d->nheads % d->ngroups != 0) return DART_ERR_BAD_DIMS;
  if (d->batch * d->nheads > (int64_t(1) << 24) || d->max_chunks > (int64_t(1) << 20) ||
      d->batch > 65535 || d->nheads > 65535)  // grid y/z limits
    return DART_ERR_BAD_DIMS;
  if (!dart::shape_supported(d->io, d->dstate, d->headdim) || !dart::chunk_supported(d->chunk))
    return DART_ERR_UNSUPPORTED;
  return DART_OK;
}

extern "C" size_t dart_sma_decode_workspace(const dart_decode_dims* d) {
  if (dart_validate_decode_dims(d) != DART_OK) return 0;
  return dart::decode_workspace_bytes(*d);
}
