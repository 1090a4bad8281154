// Shape rules shared by the host validation and the launch code (no HIP).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "dart.h"

namespace dart {

constexpr int64_t kMinChunk = 32;
constexpr int64_t kMaxChunk = 256;
// decode launches at least this many workgroups, splitting each (sequence,
// head) over chunk ranges when there are fewer pairs than that
constexpr int64_t kDecodeTargetBlocks = 1024;

bool shape_supported(int io, int64_t N, int64_t P);
bool chunk_supported(int64_t S);
int decode_splits(const dart_decode_dims& d);
size_t decode_workspace_bytes(const dart_decode_dims& d);

}  // namespace dart
