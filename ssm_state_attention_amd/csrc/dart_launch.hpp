// Internal launch interface between the C ABI (dart_api.hip) and the kernel
// files.  Every launcher enqueues on `stream` and returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>

#include "dart_device.hpp"

namespace dart {

struct PrefillShape {
  int B, L, H, G, S;  // batch, length, heads, groups, chunk
};

struct DecodeShape {
  int B, H, G, S, max_chunks, splits;
};

template <typename T, int N, int P>
hipError_t launch_chunk_state(const PrefillShape& s, const T* x, const float* dt, const float* A,
                              const T* Bm, float* acum, T* dH, float* dH_f32, hipStream_t st);

template <typename T, int N, int P>
hipError_t launch_state_pass(const PrefillShape& s, const T* x, const float* dt, const T* Bm,
                             const T* C, const float* acum, const float* dH_f32,
                             const float* h0, T* H_in, float* h_final, T* y_ssd,
                             hipStream_t st);

// Native chunk output y_ssd from H_in (the second half of launch_state_pass).
template <typename T, int N, int P>
hipError_t launch_chunk_out(const PrefillShape& s, const T* x, const float* dt, const T* Bm,
                            const T* C, const float* acum, const T* H_in, T* y_ssd,
                            hipStream_t st);

// Chunk memories and the state recurrence in one pass (16-bit io: one
// kernel handing the f32 state from chunk to chunk through the workspace;
// f32 io: launch_chunk_state and the recurrence kernel, the f32 memories in
// dH_f32 or, when that is null, in the workspace).  tag must differ from
// the tags of earlier calls that used the same workspace.
template <typename T, int N, int P>
hipError_t launch_chunk_scan(const PrefillShape& s, const T* x, const float* dt, const float* A,
                             const T* Bm, const float* h0, float* acum, T* dH, float* dH_f32,
                             T* H_in, float* h_final, void* workspace, unsigned tag,
                             hipStream_t st);
size_t chunk_scan_workspace_bytes(int io, int64_t B, int64_t L, int64_t H, int64_t N, int64_t P,
                                  int64_t S);

// acum == nullptr: the SMA of the pages; otherwise the decay-included variant.
// k0 > 0: the tokens continue sequences whose first k0 memories are in prior
// (pstride memories per (batch, head)), or, with prior8 != nullptr, in the fp8
// cache prior8 with one scale per memory in pscale (bf16 only; acum must be
// nullptr).  o != nullptr: also write the readout o [B,L,H,P] (f32) and the
// base-2 log-normaliser lse [B,H,L] for the backward.
template <typename T, int N, int P>
hipError_t launch_sma_fwd(const PrefillShape& s, const T* Q, const T* E, const T* C,
                          const T* dH, const T* y_ssd, const float* acum, float gate, T* y,
                          const T* prior, int k0, int pstride, float* o, float* lse,
                          const uint8_t* prior8, const float* pscale, hipStream_t st);

// cache8 == nullptr: the cache is `cache` in the io type; otherwise it is
// the fp8 code array cache8 with one scale per memory in cscale.  flag !=
// nullptr: the cache-full flag goes there instead of the workspace's first
// int32.
template <typename T, int N, int P>
hipError_t launch_sma_decode(const DecodeShape& s, const T* x, const float* dt, const float* A,
                             const T* Bm, const T* C, const T* Q, const T* E, float gate,
                             T* cache, uint8_t* cache8, float* cscale, float* h, float* dH_cur,
                             int* n_chunks, int* pos, T* y, void* workspace, int* flag,
                             hipStream_t st);

// Device address of this GPU's static decode scratch (DART_DECODE_SCRATCH_BYTES),
// looked up on the first call made with the device current.
hipError_t decode_scratch(void** ptr);

// fp8 codes and scales of n_mem f32 memories per (batch, head), written to
// cache slots first .. first + n_mem - 1 (T only selects the instantiation).
template <typename T, int N, int P>
hipError_t launch_fp8_store(int B, int H, int n_mem, int first, int max_chunks, const float* src,
                            uint8_t* cache8, float* cscale, hipStream_t st);

// SMA backward (16-bit io, P <= 64): dQ, dC [B,L,G,N], dE [B,L,H,P], ddH
// [B,H,M,P,N] and dgate (all f32) from the training forward's o and lse and
// the upstream gradient dy; workspace of sma_bwd_workspace_bytes().
template <typename T, int N, int P>
hipError_t launch_sma_bwd(const PrefillShape& s, const T* Q, const T* E, const T* C,
                          const T* dH, const float* o, const float* lse, const T* dy, float gate,
                          float* dQ, float* dE, float* dC, float* ddH, float* dgate,
                          void* workspace, hipStream_t st);
size_t sma_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t S);

// Backward for f32 io (N = P = 16 or 32), plain f32 kernels: the same
// arguments and results as launch_sma_bwd / launch_scan_bwd, with their own
// workspaces.
template <int N, int P>
hipError_t launch_sma_bwd_f32(const PrefillShape& s, const float* Q, const float* E,
                              const float* C, const float* dH, const float* o, const float* lse,
                              const float* dy, float gate, float* dQ, float* dE, float* dC,
                              float* ddH, float* dgate, void* workspace, hipStream_t st);
template <int N, int P>
hipError_t launch_scan_bwd_f32(const PrefillShape& s, const float* x, const float* dt,
                               const float* A, const float* Bm, const float* C,
                               const float* acum, const float* H_in, const float* dy,
                               const float* ddH, const float* dh_final, const float* dC_sma,
                               float* dx, float* ddt, float* dA, float* dB, float* dC,
                               float* dh0, void* workspace, hipStream_t st);
size_t sma_bwd_f32_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t G, int64_t S);
size_t scan_bwd_f32_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t N, int64_t P,
                                    int64_t S);

// Scan backward (16-bit io, P <= 64, S a multiple of 64): dx, ddt, dA, dB,
// dC (+ dC_sma), dh0 (all f32) from dy, ddH and dh_final (both may be null).
template <typename T, int N, int P>
hipError_t launch_scan_bwd(const PrefillShape& s, const T* x, const float* dt, const float* A,
                           const T* Bm, const T* C, const float* acum, const T* H_in, const T* dy,
                           const float* ddH, const float* dh_final, const float* dC_sma,
                           float* dx, float* ddt, float* dA, float* dB, float* dC, float* dh0,
                           void* workspace, hipStream_t st);
size_t scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t N, int64_t P,
                                int64_t S);

}  // namespace dart

// (T, N, P) combinations compiled into the library; must match
// dart::shape_supported().
#define DART_FOR_EACH_SHAPE(X) \
  X(float, 16, 16)             \
  X(float, 32, 32)             \
  X(dart::bf16, 32, 32)        \
  X(dart::bf16, 64, 64)        \
  X(dart::bf16, 128, 64)       \
  X(dart::bf16, 128, 128)
