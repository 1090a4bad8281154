// extern "C" entry points of libdart: host validation, then dispatch on the
// element type and (N, P) to the compiled kernel set.
#include <stdint.h>

#include <atomic>
#include <chrono>

#include "dart.h"
#include "dart_launch.hpp"
#include "dart_shapes.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename... Ps>
dart_status check_ptrs(Ps... ps) {
  const void* arr[] = {static_cast<const void*>(ps)...};
  for (const void* p : arr)
    if (!p) return DART_ERR_NULL_PTR;
  for (const void* p : arr)
    if (!aligned16(p)) return DART_ERR_ALIGN;
  return DART_OK;
}

dart::PrefillShape prefill_shape(const dart_dims* d) {
  return {static_cast<int>(d->batch), static_cast<int>(d->seqlen), static_cast<int>(d->nheads),
          static_cast<int>(d->ngroups), static_cast<int>(d->chunk)};
}

dart_status hip_status(hipError_t e) { return e == hipSuccess ? DART_OK : DART_ERR_HIP; }

// Calls fn.template run<T, N, P>() for the compiled combination matching
// (io, N, P); the caller has validated that one exists.
template <typename Fn>
dart_status dispatch(int io, int64_t N, int64_t P, Fn&& fn) {
#define DART_DISPATCH_CASE(T, NN, PP)                                             \
  if (io == (std::is_same<T, float>::value ? DART_F32 : DART_BF16) && N == NN && \
      P == PP)                                                                    \
    return hip_status(fn.template run<T, NN, PP>());
  DART_FOR_EACH_SHAPE(DART_DISPATCH_CASE)
#undef DART_DISPATCH_CASE
  return DART_ERR_UNSUPPORTED;
}

struct ChunkStateFn {
  dart::PrefillShape sh;
  const void *x, *Bm;
  const float *dt, *A;
  float* acum;
  void* dH;
  float* dHf;
  hipStream_t st;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_chunk_state<T, N, P>(sh, static_cast<const T*>(x), dt, A,
                                             static_cast<const T*>(Bm), acum, static_cast<T*>(dH),
                                             dHf, st);
  }
};

struct StatePassFn {
  dart::PrefillShape sh;
  const void *x, *Bm, *C;
  const float *dt, *acum, *dHf, *h0;
  void* H_in;
  float* h_final;
  void* y_ssd;
  hipStream_t st;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_state_pass<T, N, P>(sh, static_cast<const T*>(x), dt,
                                            static_cast<const T*>(Bm), static_cast<const T*>(C),
                                            acum, dHf, h0, static_cast<T*>(H_in), h_final,
                                            static_cast<T*>(y_ssd), st);
  }
};

struct ChunkScanFn {
  dart::PrefillShape sh;
  const void *x, *Bm;
  const float *dt, *A, *h0;
  float* acum;
  void* dH;
  float* dHf;
  void* H_in;
  float* h_final;
  void* ws;
  unsigned tag;
  hipStream_t st;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_chunk_scan<T, N, P>(sh, static_cast<const T*>(x), dt, A,
                                            static_cast<const T*>(Bm), h0, acum,
                                            static_cast<T*>(dH), dHf, static_cast<T*>(H_in),
                                            h_final, ws, tag, st);
  }
};

struct ChunkOutFn {
  dart::PrefillShape sh;
  const void *x, *Bm, *C;
  const float *dt, *acum;
  const void* H_in;
  void* y_ssd;
  hipStream_t st;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_chunk_out<T, N, P>(sh, static_cast<const T*>(x), dt,
                                           static_cast<const T*>(Bm), static_cast<const T*>(C),
                                           acum, static_cast<const T*>(H_in),
                                           static_cast<T*>(y_ssd), st);
  }
};

// Tags of dart_chunk_scan calls: distinct per call within the process, and
// started from the clock so that a flag value left in reused device memory
// by an earlier process is unlikely to match.
unsigned next_scan_tag() {
  static std::atomic<unsigned> counter{static_cast<unsigned>(
      std::chrono::steady_clock::now().time_since_epoch().count() * 2654435761ull)};
  unsigned t;
  do t = counter.fetch_add(1, std::memory_order_relaxed);
  while (t == 0);
  return t;
}

struct SmaFwdFn {
  dart::PrefillShape sh;
  const void *Q, *E, *C, *dH, *y_ssd;
  const float* acum;
  float gate;
  void* y;
  const void* prior;
  int k0, pstride;
  hipStream_t st;
  void* o = nullptr;
  float* lse = nullptr;
  const uint8_t* prior8 = nullptr;
  const float* pscale = nullptr;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_sma_fwd<T, N, P>(sh, static_cast<const T*>(Q), static_cast<const T*>(E),
                                         static_cast<const T*>(C), static_cast<const T*>(dH),
                                         static_cast<const T*>(y_ssd), acum, gate,
                                         static_cast<T*>(y), static_cast<const T*>(prior), k0,
                                         pstride, static_cast<float*>(o), lse, prior8, pscale,
                                         st);
  }
};

struct SmaDecodeFn {
  dart::DecodeShape sh;
  const void *x, *Bm, *C, *Q, *E;
  const float *dt, *A;
  float gate;
  void* cache;
  uint8_t* cache8;
  float* cscale;
  float *h, *dHc;
  int *nc, *pos;
  void *y, *ws;
  hipStream_t st;
  int* flag = nullptr;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_sma_decode<T, N, P>(
        sh, static_cast<const T*>(x), dt, A, static_cast<const T*>(Bm), static_cast<const T*>(C),
        static_cast<const T*>(Q), static_cast<const T*>(E), gate, static_cast<T*>(cache), cache8,
        cscale, h, dHc, nc, pos, static_cast<T*>(y), ws, flag, st);
  }
};

struct Fp8StoreFn {
  int B, H, n_mem, first, max_chunks;
  const float* src;
  uint8_t* cache8;
  float* cscale;
  hipStream_t st;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_fp8_store<T, N, P>(B, H, n_mem, first, max_chunks, src, cache8, cscale,
                                           st);
  }
};

struct SmaBwdFn {
  dart::PrefillShape sh;
  const void *Q, *E, *C, *dH, *o;
  const float* lse;
  const void* dy;
  float gate;
  float *dQ, *dE, *dC, *ddH, *dgate;
  void* ws;
  hipStream_t st;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_sma_bwd<T, N, P>(
        sh, static_cast<const T*>(Q), static_cast<const T*>(E), static_cast<const T*>(C),
        static_cast<const T*>(dH), static_cast<const float*>(o), lse, static_cast<const T*>(dy), gate,
        dQ, dE, dC, ddH, dgate, ws, st);
  }
};

struct ScanBwdFn {
  dart::PrefillShape sh;
  const void *x, *Bm, *C, *H_in, *dy;
  const float *dt, *A, *acum, *ddH, *dhf, *dC_sma;
  float *dx, *ddt, *dA, *dB, *dC, *dh0;
  void* ws;
  hipStream_t st;
  template <typename T, int N, int P>
  hipError_t run() {
    return dart::launch_scan_bwd<T, N, P>(
        sh, static_cast<const T*>(x), dt, A, static_cast<const T*>(Bm), static_cast<const T*>(C),
        acum, static_cast<const T*>(H_in), static_cast<const T*>(dy), ddH, dhf, dC_sma, dx, ddt,
        dA, dB, dC, dh0, ws, st);
  }
};

// The backward is compiled for 16-bit io with P <= 64 and chunks of whole
// 64-token tiles.
bool bwd_supported(const dart_dims* d) {
  // f32 io: the plain f32 kernels, every compiled shape and chunk size
  if (d->io == DART_F32) return true;
  // the dy·o pass launches one workgroup per four (batch, token) rows
  return d->io == DART_BF16 && d->headdim <= 64 && d->chunk % 64 == 0 &&
         d->batch * d->seqlen / 4 < (int64_t(1) << 31);
}

dart::DecodeShape decode_shape(const dart_decode_dims* d) {
  return {static_cast<int>(d->batch),      static_cast<int>(d->nheads),
          static_cast<int>(d->ngroups),    static_cast<int>(d->chunk),
          static_cast<int>(d->max_chunks), dart::decode_splits(*d)};
}

}  // namespace

extern "C" dart_status dart_chunk_state(const dart_dims* dims, const void* x, const float* dt,
                                        const float* A, const void* Bm, float* acum, void* dH,
                                        float* dH_f32, void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(x, dt, A, Bm, acum, dH, dH_f32)) != DART_OK) return s;
  ChunkStateFn fn{prefill_shape(dims), x, Bm, dt, A, acum, dH, dH_f32, static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_state_pass(const dart_dims* dims, const void* x, const float* dt,
                                       const void* Bm, const void* C, const float* acum,
                                       const float* dH_f32, const float* h0, void* H_in,
                                       float* h_final, void* y_ssd, void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(x, dt, Bm, C, acum, dH_f32, H_in, h_final, y_ssd)) != DART_OK) return s;
  if (h0 && !aligned16(h0)) return DART_ERR_ALIGN;
  StatePassFn fn{prefill_shape(dims), x, Bm, C, dt, acum, dH_f32, h0, H_in, h_final, y_ssd,
       static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" size_t dart_chunk_scan_workspace(const dart_dims* dims) {
  if (dart_validate_dims(dims) != DART_OK) return 0;
  return (dart::chunk_scan_workspace_bytes(dims->io, dims->batch, dims->seqlen, dims->nheads,
                                           dims->dstate, dims->headdim, dims->chunk) +
          255) / 256 * 256;
}

extern "C" dart_status dart_chunk_scan(const dart_dims* dims, const void* x, const float* dt,
                                       const float* A, const void* Bm, const float* h0,
                                       float* acum, void* dH, float* dH_f32, void* H_in,
                                       float* h_final, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(x, dt, A, Bm, acum, dH, H_in, h_final)) != DART_OK) return s;
  if ((h0 && !aligned16(h0)) || (dH_f32 && !aligned16(dH_f32))) return DART_ERR_ALIGN;
  if (!workspace || workspace_bytes < dart_chunk_scan_workspace(dims)) return DART_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DART_ERR_ALIGN;
  ChunkScanFn fn{prefill_shape(dims), x, Bm, dt, A, h0, acum, dH, dH_f32, H_in, h_final,
                 workspace, next_scan_tag(), static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_chunk_out(const dart_dims* dims, const void* x, const float* dt,
                                      const void* Bm, const void* C, const float* acum,
                                      const void* H_in, void* y_ssd, void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(x, dt, Bm, C, acum, H_in, y_ssd)) != DART_OK) return s;
  ChunkOutFn fn{prefill_shape(dims), x, Bm, C, dt, acum, H_in, y_ssd,
                static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_sma_fwd(const dart_dims* dims, const void* Q, const void* E,
                                    const void* C, const void* dH, const void* y_ssd,
                                    float gate, void* y, void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(Q, E, C, dH, y_ssd, y)) != DART_OK) return s;
  SmaFwdFn fn{prefill_shape(dims), Q, E, C, dH, y_ssd, nullptr, gate, y, nullptr, 0, 0,
              static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_sma_fwd_train(const dart_dims* dims, const void* Q, const void* E,
                                          const void* C, const void* dH, const void* y_ssd,
                                          float gate, void* y, void* o, float* lse,
                                          void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(Q, E, C, dH, y_ssd, y, o, lse)) != DART_OK) return s;
  SmaFwdFn fn{prefill_shape(dims), Q, E, C, dH, y_ssd, nullptr, gate, y, nullptr, 0, 0,
              static_cast<hipStream_t>(stream), o, lse};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_sma_fwd_cont(const dart_dims* dims, int64_t prior_chunks,
                                         int64_t cache_chunks, const void* Q, const void* E,
                                         const void* C, const void* cache, const void* dH,
                                         const void* y_ssd, float gate, void* y, void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if (prior_chunks < 0 || cache_chunks < prior_chunks || prior_chunks > INT32_MAX ||
      cache_chunks > INT32_MAX || prior_chunks + dims->seqlen / dims->chunk > INT32_MAX)
    return DART_ERR_BAD_DIMS;
  if ((s = check_ptrs(Q, E, C, dH, y_ssd, y)) != DART_OK) return s;
  if (prior_chunks > 0 && (s = check_ptrs(cache)) != DART_OK) return s;
  SmaFwdFn fn{prefill_shape(dims), Q, E, C, dH, y_ssd, nullptr, gate, y,
              prior_chunks > 0 ? cache : nullptr, static_cast<int>(prior_chunks),
              static_cast<int>(cache_chunks), static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_sma_fwd_cont_fp8(const dart_dims* dims, int64_t prior_chunks,
                                             int64_t cache_chunks, const void* Q, const void* E,
                                             const void* C, const uint8_t* cache8,
                                             const float* scale, const void* dH,
                                             const void* y_ssd, float gate, void* y,
                                             void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if (dims->io != DART_BF16) return DART_ERR_UNSUPPORTED;
  if (prior_chunks < 0 || cache_chunks < prior_chunks || prior_chunks > INT32_MAX ||
      cache_chunks > INT32_MAX || prior_chunks + dims->seqlen / dims->chunk > INT32_MAX)
    return DART_ERR_BAD_DIMS;
  if ((s = check_ptrs(Q, E, C, dH, y_ssd, y)) != DART_OK) return s;
  if (prior_chunks > 0 && (s = check_ptrs(cache8, scale)) != DART_OK) return s;
  SmaFwdFn fn{prefill_shape(dims), Q, E, C, dH, y_ssd, nullptr, gate, y, nullptr,
              static_cast<int>(prior_chunks), static_cast<int>(cache_chunks),
              static_cast<hipStream_t>(stream)};
  if (prior_chunks > 0) {
    fn.prior8 = cache8;
    fn.pscale = scale;
  } else {
    fn.k0 = 0;
  }
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_sma_fwd_decayed(const dart_dims* dims, const void* Q, const void* E,
                                            const void* C, const void* dH, const float* acum,
                                            const void* y_ssd, float gate, void* y,
                                            void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(Q, E, C, dH, acum, y_ssd, y)) != DART_OK) return s;
  SmaFwdFn fn{prefill_shape(dims), Q, E, C, dH, y_ssd, acum, gate, y, nullptr, 0, 0,
              static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_sma_decode(const dart_decode_dims* dims, const void* x,
                                       const float* dt, const float* A, const void* Bm,
                                       const void* C, const void* Q, const void* E, float gate,
                                       void* cache, float* h, float* dH_cur, int32_t* n_chunks,
                                       int32_t* pos, void* y, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  dart_status s = dart_validate_decode_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(x, dt, A, Bm, C, Q, E, cache, h, dH_cur, n_chunks, pos, y)) != DART_OK)
    return s;
  if (!workspace || workspace_bytes < dart::decode_workspace_bytes(*dims))
    return DART_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DART_ERR_ALIGN;
  SmaDecodeFn fn{decode_shape(dims), x, Bm, C, Q, E, dt, A, gate, cache, nullptr, nullptr, h,
                 dH_cur, n_chunks, pos, y, workspace, static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_sma_decode_noalloc(const dart_decode_dims* dims, const void* x,
                                               const float* dt, const float* A, const void* Bm,
                                               const void* C, const void* Q, const void* E,
                                               float gate, void* cache, float* h, float* dH_cur,
                                               int32_t* n_chunks, int32_t* pos, void* y,
                                               int32_t* cache_full, void* stream) {
  dart_status s = dart_validate_decode_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(x, dt, A, Bm, C, Q, E, cache, h, dH_cur, n_chunks, pos, y)) != DART_OK)
    return s;
  if (cache_full && (reinterpret_cast<uintptr_t>(cache_full) & 3u) != 0) return DART_ERR_ALIGN;
  if (dart::decode_workspace_bytes(*dims) > DART_DECODE_SCRATCH_BYTES) return DART_ERR_SCRATCH;
  void* ws = nullptr;
  if (dart::decode_scratch(&ws) != hipSuccess) return DART_ERR_HIP;
  SmaDecodeFn fn{decode_shape(dims), x, Bm, C, Q, E, dt, A, gate, cache, nullptr, nullptr, h,
                 dH_cur, n_chunks, pos, y, ws, static_cast<hipStream_t>(stream), cache_full};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_sma_decode_fp8(const dart_decode_dims* dims, const void* x,
                                           const float* dt, const float* A, const void* Bm,
                                           const void* C, const void* Q, const void* E,
                                           float gate, uint8_t* cache8, float* scale, float* h,
                                           float* dH_cur, int32_t* n_chunks, int32_t* pos,
                                           void* y, void* workspace, size_t workspace_bytes,
                                           void* stream) {
  dart_status s = dart_validate_decode_dims(dims);
  if (s != DART_OK) return s;
  if ((s = check_ptrs(x, dt, A, Bm, C, Q, E, cache8, scale, h, dH_cur, n_chunks, pos, y)) !=
      DART_OK)
    return s;
  if (!workspace || workspace_bytes < dart::decode_workspace_bytes(*dims))
    return DART_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DART_ERR_ALIGN;
  SmaDecodeFn fn{decode_shape(dims), x, Bm, C, Q, E, dt, A, gate, nullptr, cache8, scale, h,
                 dH_cur, n_chunks, pos, y, workspace, static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" dart_status dart_cache_fp8_store(const dart_decode_dims* dims, const float* dH_f32,
                                            int64_t n_mem, int64_t first, uint8_t* cache8,
                                            float* scale, void* stream) {
  dart_status s = dart_validate_decode_dims(dims);
  if (s != DART_OK) return s;
  if (n_mem < 0 || first < 0 || first > dims->max_chunks - n_mem) return DART_ERR_BAD_DIMS;
  if ((s = check_ptrs(dH_f32, cache8, scale)) != DART_OK) return s;
  Fp8StoreFn fn{static_cast<int>(dims->batch), static_cast<int>(dims->nheads),
                static_cast<int>(n_mem), static_cast<int>(first),
                static_cast<int>(dims->max_chunks), dH_f32, cache8, scale,
                static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" size_t dart_sma_bwd_workspace(const dart_dims* dims) {
  if (dart_validate_dims(dims) != DART_OK || !bwd_supported(dims)) return 0;
  if (dims->io == DART_F32)
    return (dart::sma_bwd_f32_workspace_bytes(dims->batch, dims->seqlen, dims->nheads,
                                              dims->ngroups, dims->chunk) + 255) / 256 * 256;
  return (dart::sma_bwd_workspace_bytes(dims->batch, dims->seqlen, dims->nheads,
                                        dims->chunk) + 255) / 256 *
         256;
}

extern "C" dart_status dart_sma_bwd(const dart_dims* dims, const void* Q, const void* E,
                                    const void* C, const void* dH, const void* o,
                                    const float* lse, const void* dy, float gate, float* dQ,
                                    float* dE, float* dC, float* ddH, float* dgate,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if (!bwd_supported(dims)) return DART_ERR_UNSUPPORTED;
  if ((s = check_ptrs(Q, E, C, dH, o, lse, dy, dQ, dE, dC, ddH, dgate)) != DART_OK) return s;
  if (!workspace || workspace_bytes < dart_sma_bwd_workspace(dims)) return DART_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DART_ERR_ALIGN;
  SmaBwdFn fn{prefill_shape(dims), Q, E, C, dH, o, lse, dy, gate, dQ, dE, dC, ddH, dgate,
              workspace, static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}

extern "C" size_t dart_scan_bwd_workspace(const dart_dims* dims) {
  if (dart_validate_dims(dims) != DART_OK || !bwd_supported(dims)) return 0;
  if (dims->io == DART_F32)
    return dart::scan_bwd_f32_workspace_bytes(dims->batch, dims->seqlen, dims->nheads,
                                              dims->dstate, dims->headdim, dims->chunk);
  return dart::scan_bwd_workspace_bytes(dims->batch, dims->seqlen, dims->nheads, dims->dstate,
                                        dims->headdim, dims->chunk);
}

extern "C" dart_status dart_scan_bwd(const dart_dims* dims, const void* x, const float* dt,
                                     const float* A, const void* Bm, const void* C,
                                     const float* acum, const void* H_in, const void* dy,
                                     const float* ddH, const float* dh_final,
                                     const float* dC_sma, float* dx, float* ddt, float* dA,
                                     float* dB, float* dC, float* dh0, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  dart_status s = dart_validate_dims(dims);
  if (s != DART_OK) return s;
  if (!bwd_supported(dims)) return DART_ERR_UNSUPPORTED;
  if ((s = check_ptrs(x, dt, A, Bm, C, acum, H_in, dy, dx, ddt, dA, dB, dC, dh0)) != DART_OK)
    return s;
  for (const void* p : {static_cast<const void*>(ddH), static_cast<const void*>(dh_final),
                        static_cast<const void*>(dC_sma)})
    if (p && !aligned16(p)) return DART_ERR_ALIGN;
  if (!workspace || workspace_bytes < dart_scan_bwd_workspace(dims)) return DART_ERR_WORKSPACE;
  if (!aligned16(workspace)) return DART_ERR_ALIGN;
  ScanBwdFn fn{prefill_shape(dims), x, Bm, C, H_in, dy, dt, A, acum, ddH, dh_final, dC_sma,
               dx, ddt, dA, dB, dC, dh0, workspace, static_cast<hipStream_t>(stream)};
  return dispatch(dims->io, dims->dstate, dims->headdim, fn);
}
