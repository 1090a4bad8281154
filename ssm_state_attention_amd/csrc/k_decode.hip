// Single-token decode over the chunk-memory cache on gfx950, with the cache
// held either in the io element type or as 8-bit floating point codes.
//
// Definitions (DART abstract: the length-dependent inference cache is the set
// of chunk memories; Pith review of DART, "Core claim", minor comment 1 and
// paper §4 Eq. 14): for the new token t of chunk k of a sequence
//   h <- exp(dt·A)·h + dt·B_t x_tᵀ,  y_ssd = C_tᵀ·h    (the Mamba-2 recurrence)
//   o_t = Σ_{c<k} softmax_c(Q_tᵀ·dH[c]·E_t / sqrt(N))·C_tᵀ·dH[c]
//   y_t = y_ssd + gate·o_t
// and the memory of chunk k, accumulated token by token in dH_cur, joins the
// cache when its last token has been processed.
//
// The fp8 cache (Pith review, "Where Pith is reading between the lines":
// SMA's reuse of the scan's dH invites cache quantisation) keeps memory c as
// OCP FP8 E4M3 codes plus one power-of-two scale 2^e: the codes are the
// round-to-nearest-even encodings of dH[c]·2^-e, with e = max(E - 8, -126)
// for the memory's largest magnitude f·2^E (0.5 <= f < 1), so every scaled
// magnitude is below 256 and no code saturates.
#include <mutex>

#include "dart.h"
#include "dart_launch.hpp"
#include "dart_shapes.hpp"

namespace dart {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx2 __attribute__((ext_vector_type(2)));

// Exponent e of the scale 2^e of a memory whose largest magnitude is amax:
// with amax = f·2^E (0.5 <= f < 1), e = max(E - 8, -126); e = 0 when amax is 0.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  const int field = static_cast<int>((__float_as_uint(amax) >> 23) & 0xFFu);
  return max(field - 134, -126);  // normal amax: E = field - 126
}
// 2^e for e in [-126, 127]
__device__ __forceinline__ float pow2i(int e) {
  return __uint_as_float(static_cast<unsigned>(e + 127) << 23);
}
// E4M3 codes of four values (round to nearest even), value i in byte i
__device__ __forceinline__ unsigned pack_fp8x4(floatx4 v) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
  return static_cast<unsigned>(__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], lo, true));
}

// Largest value of m over a 256-thread workgroup (sh: 4 floats of LDS).
__device__ __forceinline__ float block_max256(float m, float* sh) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = m;
  __syncthreads();
  return fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
}

// The state step of one (batch, head), run by a 256-thread workgroup: advances
// the SSM state, forms y_ssd = C·h into sh_y and, when the token closes its
// chunk, appends the finished memory to the cache (at index kc = n_chunks[b],
// which the streaming loops never read): rounded to the io type, or (F8)
// encoded with the scale taken from the memory's largest magnitude, which the
// workgroup finds from the registers it already holds.  sh_c, sh_b, sh_x
// (C, B, x of the token) must be in LDS; sh_y is complete on return.
template <typename T, int N, int P, bool F8>
__device__ __forceinline__ void state_step(float dtv, float Ah, T* __restrict__ cache,
                                           uint8_t* __restrict__ cache8,
                                           float* __restrict__ cscale, float* __restrict__ hst,
                                           float* __restrict__ dHc, long pair, int kc, int ps,
                                           int S, int max_chunks, int* ws_flag,
                                           const float* sh_c, const float* sh_b,
                                           const float* sh_x, float* sh_y, float* sh_m) {
  constexpr int Q4 = N / 4;
  static_assert((P * N / 4) % 64 == 0 && 64 % Q4 == 0, "decode state mapping");
  const int tid = threadIdx.x;
  {
    const float a = exp_neg(dtv * Ah);
    const bool close = ps == S - 1;
    const bool append = close && kc < max_chunks;  // uniform over the workgroup
    floatx4* hp = reinterpret_cast<floatx4*>(hst + pair * (P * N));
    floatx4* dp = reinterpret_cast<floatx4*>(dHc + pair * (P * N));
    const long slot = pair * max_chunks + kc;
    // all of this thread's state loads first, then the updates
    // (P·N/4 is a multiple of 64, so the guard is uniform over each wave)
    constexpr int SQ = P * N / 4, SV = (SQ + 255) / 256;
    static_assert(SQ % 64 == 0 && (Q4 == 4 || Q4 == 8 || Q4 == 16 || Q4 == 32),
                  "decode state split");
    floatx4 hv[SV], dv[SV];
#pragma unroll
    for (int v = 0; v < SV; ++v) {
      const int i = tid + v * 256;
      if (SQ % 256 == 0 || i < SQ) {
        hv[v] = hp[i];
        dv[v] = dp[i];
      }
    }
#pragma unroll
    for (int v = 0; v < SV; ++v) {
      const int i = tid + v * 256;
      if (SQ % 256 != 0 && i >= SQ) break;
      const int p = i / Q4, n = (i % Q4) * 4;
      const float xd = dtv * sh_x[p];
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float u = xd * sh_b[n + e];
        hv[v][e] = a * hv[v][e] + u;
        dv[v][e] = a * dv[v][e] + u;
        part += sh_c[n + e] * hv[v][e];
      }
      hp[i] = hv[v];
      if constexpr (!F8) {
        if (append) store4(cache + slot * (P * N) + (long)i * 4, dv[v]);
      }
      dp[i] = close ? floatx4{0.f, 0.f, 0.f, 0.f} : dv[v];
      // sum over the Q4 lanes that share row p (the row rotations span 16
      // lanes, so a group of 8 takes its last step by a lane exchange)
      part += dpp_mov<0xB1>(part);
      part += dpp_mov<0x4E>(part);
      if (Q4 == 8) part += __shfl_xor(part, 4);
      if (Q4 >= 16) {
        part += dpp_mov<0x124>(part);
        part += dpp_mov<0x128>(part);
      }
      if (Q4 >= 32) {
        const unsigned u = __float_as_uint(part);
        const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
        part = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
      }
      if ((i % Q4) == 0) sh_y[p] = part;
    }
    if constexpr (F8) {
      if (append) {
        float m = 0.f;
#pragma unroll
        for (int v = 0; v < SV; ++v) {
          if (SQ % 256 != 0 && tid + v * 256 >= SQ) break;
          m = fmaxf(m, fmaxf(fmaxf(fabsf(dv[v][0]), fabsf(dv[v][1])),
                             fmaxf(fabsf(dv[v][2]), fabsf(dv[v][3]))));
        }
        const int e = fp8_scale_exp(block_max256(m, sh_m));
        const float inv = pow2i(-e);
        unsigned* dst = reinterpret_cast<unsigned*>(cache8 + slot * (P * N));
#pragma unroll
        for (int v = 0; v < SV; ++v) {
          const int i = tid + v * 256;
          if (SQ % 256 != 0 && i >= SQ) break;
          dst[i] = pack_fp8x4(dv[v] * inv);
        }
        if (tid == 0) cscale[slot] = pow2i(e);
      }
    }
    if (close && !append && tid == 0) atomicOr(ws_flag, 1);
    __syncthreads();
  }
}

// Decode, step 1: one workgroup per (head, batch) runs the state step and
// leaves y_ssd and the cache length n_chunks[b] in the workspace.  A launch of its own: run by the streaming
// workgroups (before or after their stream), its 128 KB of state reads and
// writes per head interleave with the cache stream and cost more HBM time
// than a separate launch does.
template <typename T, int N, int P, bool F8>
__global__ __launch_bounds__(256) void k_decode_state(
    const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ C, T* __restrict__ cache,
    uint8_t* __restrict__ cache8, float* __restrict__ cscale, float* __restrict__ hst,
    float* __restrict__ dHc, const int* __restrict__ n_chunks, const int* __restrict__ pos,
    int* __restrict__ ws_flag, int* __restrict__ ws_kc, float* __restrict__ ws_yssd, int H,
    int G, int S, int max_chunks) {
  __shared__ float sh_c[N], sh_b[N], sh_x[P], sh_y[P], sh_m[4];
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const long pair = (long)b * H + h;
  const int tid = threadIdx.x;
  int kc = n_chunks[b];
  kc = kc < 0 ? 0 : (kc > max_chunks ? max_chunks : kc);
  const int ps = pos[b];
  // the streaming kernel reads this copy, so that its workgroups may advance
  // n_chunks and pos while others still stream
  if (h == 0 && tid == 0) ws_kc[b] = kc;
  for (int i = tid; i < N; i += 256) {
    const long o = ((long)b * G + g) * N + i;
    sh_c[i] = to_f32(C[o]);
    sh_b[i] = to_f32(Bm[o]);
  }
  for (int i = tid; i < P; i += 256) sh_x[i] = to_f32(x[pair * P + i]);
  __syncthreads();
  state_step<T, N, P, F8>(dt[pair], A[h], cache, cache8, cscale, hst, dHc, pair, kc, ps, S,
                          max_chunks, ws_flag, sh_c, sh_b, sh_x, sh_y, sh_m);
  for (int p = tid; p < P; p += 256) ws_yssd[pair * P + p] = sh_y[p];
}

// Arguments of one decode call, as the streaming kernels see them.  From the
// workspace: kc (n_chunks[b] at the start of the call, clamped), yssd (the
// state kernel's y_ssd rows) and part (per-split partials).
template <typename T>
struct DecodeArgs {
  const T *x, *Bm, *C, *Q, *E;
  const float *dt, *A;
  T* cache;
  uint8_t* cache8;
  float* cscale;
  float *h, *dHc;
  int *n_chunks, *pos;
  int* kc;
  float *yssd, *part;
  T* y;
  float gate, scale_log2;
  int B, H, G, S, max_chunks, splits, cps;
};

// Merge of the per-wave online-softmax states of one workgroup: emit(p, num,
// m, den) receives, for each row p, the (max, denominator, numerator) of the
// workgroup's memories.  acc: this lane's value sums for rows it·RP + pr,
// already reduced over the lanes of a row.
template <int P, int NW, int NPASS, int RP, typename Emit>
__device__ __forceinline__ void merge_waves(const float (&acc)[NPASS], float mx, float ls,
                                            bool row_lead, int pr, Emit emit) {
  __shared__ float sh_wm[NW], sh_wl[NW];
  __shared__ float sh_wacc[NW][P];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (row_lead) {
#pragma unroll
    for (int it = 0; it < NPASS; ++it) sh_wacc[w][it * RP + pr] = acc[it];
  }
  if (lane == 0) {
    sh_wm[w] = mx;
    sh_wl[w] = ls;
  }
  __syncthreads();
  float mall = -INFINITY;
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) mall = fmaxf(mall, sh_wm[ww]);
  for (int p = tid; p < P; p += 64 * NW) {
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      if (sh_wm[ww] > -INFINITY) {
        const float f = exp2_fast(sh_wm[ww] - mall);
        num += f * sh_wacc[ww][p];
        den += f * sh_wl[ww];
      }
    }
    emit(p, num, mall, den);
  }
}

// Token operands the streaming workgroup of (b, h) stages in LDS: Q and C of
// the group and E of the head.
template <typename T, int N, int P>
__device__ __forceinline__ void stage_token(const DecodeArgs<T>& a, int b, int g, long pair,
                                            float* sh_q, float* sh_c, float* sh_e) {
  const int tid = threadIdx.x;
  for (int i = tid; i < N; i += 256) {
    const long o = ((long)b * a.G + g) * N + i;
    sh_q[i] = to_f32(a.Q[o]);
    sh_c[i] = to_f32(a.C[o]);
  }
  for (int i = tid; i < P; i += 256) sh_e[i] = to_f32(a.E[pair * P + i]);
  __syncthreads();
}

// Advance sequence b's position after its token: n_chunks (clamped value kc
// from the start of the call) grows by one when the token closed a chunk.
__device__ __forceinline__ void advance_position(int* n_chunks, int* pos, int b, int kc, int S,
                                                 int max_chunks) {
  if (pos[b] == S - 1) {
    n_chunks[b] = kc < max_chunks ? kc + 1 : max_chunks;
    pos[b] = 0;
  } else {
    pos[b] += 1;
  }
}

// End of a streaming workgroup.  Several splits per (b, h): the split's
// (max, denominator, numerator[P]) partial goes to the workspace for
// k_decode_combine.  One split (SINGLE): the workgroup holds all of the
// head's memories, so it writes y = y_ssd + gate·o itself (y_ssd from the
// state kernel, which ran before), and the workgroup of head 0 advances its
// sequence's position (no other workgroup of the launch reads it).
template <typename T, int P, bool SINGLE, int NW, int NPASS, int RP>
__device__ __forceinline__ void stream_tail(const float (&acc)[NPASS], float mx, float ls,
                                            bool row_lead, int pr, const DecodeArgs<T>& a,
                                            long pair, int b, int h, int kc, int split) {
  if constexpr (!SINGLE) {
    float* part = a.part + (pair * a.splits + split) * (P + 2);
    merge_waves<P, NW, NPASS, RP>(acc, mx, ls, row_lead, pr,
                                  [&](int p, float num, float m, float den) {
                                    part[2 + p] = num;
                                    if (p == 0) {
                                      part[0] = m;
                                      part[1] = den;
                                    }
                                  });
  } else {
    const float* ys = a.yssd + pair * P;
    T* yp = a.y + pair * P;
    merge_waves<P, NW, NPASS, RP>(acc, mx, ls, row_lead, pr,
                                  [&](int p, float num, float m, float den) {
                                    const float o = den > 0.f ? num / den : 0.f;
                                    yp[p] = from_f32<T>(ys[p] + a.gate * o);
                                  });
    if (h == 0 && threadIdx.x == 0) advance_position(a.n_chunks, a.pos, b, kc, a.S, a.max_chunks);
  }
}

// The memory loop of a streaming wave: memories c0, c0 + step, ... < c_end
// (c0 uniform over the wave).  PIPE: the loads of the next memory are issued
// into a second register set before the current one is consumed, so every
// wave keeps a memory in flight while it computes (used where the two sets
// leave enough registers: 64 per set for the 16-bit cache, 32 for fp8, whose
// decoding needs more temporaries).
template <bool PIPE, typename Raw, typename Load, typename Consume>
__device__ __forceinline__ void stream_memories(Load load, Consume consume, int c0, int c_end,
                                                int step) {
  Raw ra, rb;
  if constexpr (PIPE) {
    int c = c0;
    if (c < c_end) load(ra, c);
    while (c < c_end) {
      if (c + step < c_end) load(rb, c + step);
      consume(ra);
      c += step;
      if (c >= c_end) break;
      if (c + step < c_end) load(ra, c + step);
      consume(rb);
      c += step;
    }
  } else {
    (void)rb;
    for (int c = c0; c < c_end; c += step) {
      load(ra, c);
      consume(ra);
    }
  }
}

// Decode, step 2: one workgroup (4 waves) per (split, head, batch) streams
// the cached memories of its split once from HBM.  Each wave takes whole
// memories c = first + wave, first + wave + 4, ... (non-temporal 16-byte
// loads): lane (nv, pr) holds key entries n in [nv·VE, nv·VE + VE) of rows
// p = it·RP + pr, forms partial Q·dH[c] and C·dH[c] over its n-range,
// reduces the score across the wave and keeps an online softmax whose value
// accumulator stays partial over n until the end (stream_tail).
template <typename T, int N, int P, bool SINGLE>
__global__ __launch_bounds__(256) void k_sma_decode(const DecodeArgs<T> a) {
  constexpr int VE = Vec16<T>::n;
  constexpr int NV = N / VE;   // 16-byte vectors per memory row
  constexpr int RP = 64 / NV;  // rows per wave pass
  constexpr int NPASS = P / RP;
  constexpr int NW = 4;
  static_assert(64 % NV == 0 && P % RP == 0, "decode lane mapping");
  typedef typename Vec16<T>::vec vec_t;
  __shared__ float sh_q[N], sh_c[N], sh_e[P];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.H / a.G);
  const long pair = (long)b * a.H + h;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kc = a.kc[b];
  stage_token<T, N, P>(a, b, g, pair, sh_q, sh_c, sh_e);

  const int c_begin = split * a.cps;
  const int c_end = min(kc, c_begin + a.cps);
  const int nv = lane % NV, pr = lane / NV;
  constexpr bool kDot2 = std::is_same<T, bf16>::value;
  float qv[VE], cv[VE], ev[NPASS], acc[NPASS];
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    qv[e] = sh_q[nv * VE + e];
    cv[e] = sh_c[nv * VE + e];
  }
  // 16-bit io: Q and C stay packed (the widened values are exact copies)
  // and each pair of key entries is one dot2 with fp32 accumulation
  bf16x2 q2[VE / 2], c2[VE / 2];
  if constexpr (kDot2) {
#pragma unroll
    for (int e = 0; e < VE / 2; ++e) {
      q2[e] = bf16x2{from_f32<bf16>(qv[2 * e]), from_f32<bf16>(qv[2 * e + 1])};
      c2[e] = bf16x2{from_f32<bf16>(cv[2 * e]), from_f32<bf16>(cv[2 * e + 1])};
    }
  }
#pragma unroll
  for (int it = 0; it < NPASS; ++it) {
    ev[it] = sh_e[it * RP + pr];
    acc[it] = 0.f;
  }
  float mx = -INFINITY, ls = 0.f;
  const T* base = a.cache + pair * (long)a.max_chunks * (P * N);
  // the wave's memories c_begin + w, + NW, ... (stream_memories)
  auto load = [&](vec_t (&raw)[NPASS], int c) __attribute__((always_inline)) {
    const T* src = base + (long)c * (P * N);
#pragma unroll
    for (int it = 0; it < NPASS; ++it) raw[it] = load16_nt(src + ((it * RP + pr) * NV + nv) * VE);
  };
  auto consume = [&](const vec_t (&raw)[NPASS]) __attribute__((always_inline)) {
    float s = 0.f, zc[NPASS];
#pragma unroll
    for (int it = 0; it < NPASS; ++it) {
      float zq = 0.f, z2 = 0.f;
      if constexpr (kDot2) {
#pragma unroll
        for (int e = 0; e < VE / 2; ++e) {
          const bf16x2 v2 = bf16x2{raw[it][2 * e], raw[it][2 * e + 1]};
          zq = __builtin_amdgcn_fdot2_f32_bf16(q2[e], v2, zq, false);
          z2 = __builtin_amdgcn_fdot2_f32_bf16(c2[e], v2, z2, false);
        }
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          const float v = to_f32(raw[it][e]);
          zq += qv[e] * v;
          z2 += cv[e] * v;
        }
      }
      zc[it] = z2;
      s += ev[it] * zq;
    }
    s = wave_sum_dpp(s) * a.scale_log2;
    // lazy rescale, as in the prefill kernel (s is uniform over the wave)
    if (s > mx + kLazyLog2) {
      const float al = exp2_fast(mx - s);  // 0 for the first memory
      ls *= al;
#pragma unroll
      for (int it = 0; it < NPASS; ++it) acc[it] *= al;
      mx = s;
    }
    const float pw = exp2_fast(s - mx);
    ls += pw;
#pragma unroll
    for (int it = 0; it < NPASS; ++it) acc[it] += pw * zc[it];
  };
  stream_memories<NPASS * sizeof(vec_t) <= 256, vec_t[NPASS]>(load, consume, c_begin + w, c_end,
                                                              NW);
#pragma unroll
  for (int it = 0; it < NPASS; ++it)
#pragma unroll
    for (int off = 1; off < NV; off <<= 1) acc[it] += __shfl_xor(acc[it], off);
  stream_tail<T, P, SINGLE, NW, NPASS, RP>(acc, mx, ls, nv == 0, pr, a, pair, b, h, kc,
                                           split);
}

// Bytes of one fp8 cache row that a lane loads at a time: the widest of 16,
// 8 and 4 for which whole rows tile the 64 lanes of a wave and the P rows
// tile whole passes.
template <int N, int P>
struct F8Load {
  static constexpr bool fits(int lb) {
    return N % lb == 0 && 64 % (N / lb) == 0 && P % (64 / (N / lb)) == 0;
  }
  static constexpr int LB = fits(16) ? 16 : (fits(8) ? 8 : 4);
  static constexpr int W = LB / 4;  // 32-bit words per load
};
template <int W>
struct Words {
  typedef unsigned v __attribute__((ext_vector_type(W)));
};
template <>
struct Words<1> {
  typedef unsigned v;
};
template <int W>
__device__ __forceinline__ unsigned word(typename Words<W>::v r, int j) {
  if constexpr (W == 1)
    return r;
  else
    return r[j];
}

// Decode, step 2 over the fp8 cache: the streaming kernel above with LB-byte
// code loads.  16-bit io decodes each pair of codes into a bf16 pair (exact:
// every E4M3 value is a bfloat16 value) and contracts it with dot2; fp32 io
// decodes into fp32.  The products are those of the codes, so the memory's
// scale multiplies the reduced score and the softmax weight of its value.
template <typename T, int N, int P, bool SINGLE>
__global__ __launch_bounds__(256) void k_sma_decode_f8(const DecodeArgs<T> a) {
  constexpr int LB = F8Load<N, P>::LB, W = F8Load<N, P>::W;
  constexpr int NV = N / LB;   // loads per memory row
  constexpr int RP = 64 / NV;  // rows per wave pass
  constexpr int NPASS = P / RP;
  constexpr int NW = 4;
  static_assert(64 % NV == 0 && P % RP == 0, "fp8 decode lane mapping");
  typedef typename Words<W>::v load_t;
  __shared__ float sh_q[N], sh_c[N], sh_e[P];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (a.H / a.G);
  const long pair = (long)b * a.H + h;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kc = a.kc[b];
  stage_token<T, N, P>(a, b, g, pair, sh_q, sh_c, sh_e);

  const int c_begin = split * a.cps;
  const int c_end = min(kc, c_begin + a.cps);
  const int nv = lane % NV, pr = lane / NV;
  constexpr bool kDot2 = std::is_same<T, bf16>::value;
  float qv[LB], cv[LB], ev[NPASS], acc[NPASS];
#pragma unroll
  for (int e = 0; e < LB; ++e) {
    qv[e] = sh_q[nv * LB + e];
    cv[e] = sh_c[nv * LB + e];
  }
  bf16x2 q2[LB / 2], c2[LB / 2];
  if constexpr (kDot2) {
#pragma unroll
    for (int e = 0; e < LB / 2; ++e) {
      q2[e] = bf16x2{from_f32<bf16>(qv[2 * e]), from_f32<bf16>(qv[2 * e + 1])};
      c2[e] = bf16x2{from_f32<bf16>(cv[2 * e]), from_f32<bf16>(cv[2 * e + 1])};
    }
  }
#pragma unroll
  for (int it = 0; it < NPASS; ++it) {
    ev[it] = sh_e[it * RP + pr];
    acc[it] = 0.f;
  }
  float mx = -INFINITY, ls = 0.f;
  const uint8_t* base = a.cache8 + pair * (long)a.max_chunks * (P * N);
  const float* sbase = a.cscale + pair * (long)a.max_chunks;
  // codes and scale of memory c, consumed after the next memory's are issued
  struct Mem {
    load_t raw[NPASS];
    float sc;
  };
  auto load = [&](Mem& m, int c) __attribute__((always_inline)) {
    const uint8_t* src = base + (long)c * (P * N);
#pragma unroll
    for (int it = 0; it < NPASS; ++it)
      m.raw[it] = __builtin_nontemporal_load(
          reinterpret_cast<const load_t*>(src + (it * RP + pr) * N + nv * LB));
    m.sc = sbase[c];
  };
  auto consume = [&](const Mem& m) __attribute__((always_inline)) {
    float s = 0.f, zc[NPASS];
#pragma unroll
    for (int it = 0; it < NPASS; ++it) {
      float zq = 0.f, z2 = 0.f;
#pragma unroll
      for (int j = 0; j < W; ++j) {
        const unsigned wd = word<W>(m.raw[it], j);
        if constexpr (kDot2) {
          const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd, 1.0f, false);
          const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd, 1.0f, true);
          zq = __builtin_amdgcn_fdot2_f32_bf16(q2[2 * j], lo, zq, false);
          zq = __builtin_amdgcn_fdot2_f32_bf16(q2[2 * j + 1], hi, zq, false);
          z2 = __builtin_amdgcn_fdot2_f32_bf16(c2[2 * j], lo, z2, false);
          z2 = __builtin_amdgcn_fdot2_f32_bf16(c2[2 * j + 1], hi, z2, false);
        } else {
          const floatx2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(wd, false);
          const floatx2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(wd, true);
          zq += qv[4 * j] * lo[0] + qv[4 * j + 1] * lo[1] + qv[4 * j + 2] * hi[0] +
                qv[4 * j + 3] * hi[1];
          z2 += cv[4 * j] * lo[0] + cv[4 * j + 1] * lo[1] + cv[4 * j + 2] * hi[0] +
                cv[4 * j + 3] * hi[1];
        }
      }
      zc[it] = z2;
      s += ev[it] * zq;
    }
    s = wave_sum_dpp(s) * (m.sc * a.scale_log2);
    if (s > mx + kLazyLog2) {
      const float al = exp2_fast(mx - s);  // 0 for the first memory
      ls *= al;
#pragma unroll
      for (int it = 0; it < NPASS; ++it) acc[it] *= al;
      mx = s;
    }
    const float pw = exp2_fast(s - mx);
    ls += pw;
    const float pv = pw * m.sc;
#pragma unroll
    for (int it = 0; it < NPASS; ++it) acc[it] += pv * zc[it];
  };
  stream_memories<NPASS * sizeof(load_t) <= 128, Mem>(load, consume, c_begin + w, c_end, NW);
#pragma unroll
  for (int it = 0; it < NPASS; ++it)
#pragma unroll
    for (int off = 1; off < NV; off <<= 1) acc[it] += __shfl_xor(acc[it], off);
  stream_tail<T, P, SINGLE, NW, NPASS, RP>(acc, mx, ls, nv == 0, pr, a, pair, b, h, kc,
                                           split);
}

// Merge the per-split (max, denominator, numerator[P]) partials of one
// (batch, head) and apply the gate; the workgroup of head 0 advances its
// sequence's position (the launch reads no other position).
template <typename T>
__global__ __launch_bounds__(128) void k_decode_combine(const float* __restrict__ ws_yssd,
                                                        const float* __restrict__ ws_part,
                                                        const int* __restrict__ ws_kc,
                                                        float gate, T* __restrict__ y,
                                                        int* __restrict__ n_chunks,
                                                        int* __restrict__ pos, int H, int P,
                                                        int splits, int S, int max_chunks) {
  const long pair = blockIdx.x;
  const float* part = ws_part + pair * splits * (P + 2);
  float mall = -INFINITY;
  for (int s = 0; s < splits; ++s) mall = fmaxf(mall, part[s * (P + 2)]);
  for (int p = threadIdx.x; p < P; p += blockDim.x) {
    float num = 0.f, den = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float m = part[s * (P + 2)];
      if (m > -INFINITY) {
        const float f = exp2_fast(m - mall);
        num += f * part[s * (P + 2) + 2 + p];
        den += f * part[s * (P + 2) + 1];
      }
    }
    const float o = den > 0.f ? num / den : 0.f;
    y[pair * P + p] = from_f32<T>(ws_yssd[pair * P + p] + gate * o);
  }
  if (pair % H == 0 && threadIdx.x == 0) {
    const int b = static_cast<int>(pair / H);
    advance_position(n_chunks, pos, b, ws_kc[b], S, max_chunks);
  }
}

// Store n_mem f32 memories per (batch, head) into fp8 cache slots first ..
// first + n_mem - 1: one workgroup per memory finds its largest magnitude,
// then writes the codes (one 32-bit word per four values) and the scale.
template <int N, int P>
__global__ __launch_bounds__(256) void k_fp8_store(const float* __restrict__ src, int n_mem,
                                                   int first, uint8_t* __restrict__ cache8,
                                                   float* __restrict__ cscale, int H,
                                                   int max_chunks) {
  constexpr int SQ = P * N / 4, SV = (SQ + 255) / 256;
  __shared__ float sh_m[4];
  const int mem = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const long pair = (long)b * H + h;
  const int tid = threadIdx.x;
  const floatx4* s4 = reinterpret_cast<const floatx4*>(src + (pair * n_mem + mem) * (long)(P * N));
  floatx4 v[SV];
  float m = 0.f;
#pragma unroll
  for (int k = 0; k < SV; ++k) {
    const int i = tid + k * 256;
    if (SQ % 256 == 0 || i < SQ) {
      v[k] = __builtin_nontemporal_load(s4 + i);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v[k][0]), fabsf(v[k][1])),
                         fmaxf(fabsf(v[k][2]), fabsf(v[k][3]))));
    }
  }
  const int e = fp8_scale_exp(block_max256(m, sh_m));
  const float inv = pow2i(-e);
  const long slot = pair * max_chunks + first + mem;
  unsigned* dst = reinterpret_cast<unsigned*>(cache8 + slot * (P * N));
#pragma unroll
  for (int k = 0; k < SV; ++k) {
    const int i = tid + k * 256;
    if (SQ % 256 == 0 || i < SQ) dst[i] = pack_fp8x4(v[k] * inv);
  }
  if (tid == 0) cscale[slot] = pow2i(e);
}

// Device scratch of the allocation-free decode entry point
// (dart_sma_decode_noalloc): the y_ssd rows and per-split partials that
// dart_sma_decode keeps in its caller's workspace.  One copy per GPU, held
// until the process ends.  Host code never names the array except to look
// up its device address (decode_scratch below).
static __device__ __align__(256) unsigned char scratch[DART_DECODE_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

struct DecodeWs {
  int* flag;
  int* kc;
  float* yssd;
  float* part;
};
constexpr long round256(long bytes) { return (bytes + 255) / 256 * 256; }
// Workspace layout, each part 256-byte aligned: the cache-full flag (256
// bytes), kc [B] int32, y_ssd [B·H, P] f32, the per-split partials
// [B·H, splits, P + 2] f32.  Every call writes what it reads, except the
// flag, which the library only ever sets.
DecodeWs decode_ws(void* workspace, int B, long pairs, int P) {
  char* ws = static_cast<char*>(workspace);
  const long o_kc = 256, o_y = o_kc + round256(B * 4L), o_part = o_y + round256(pairs * P * 4L);
  return {reinterpret_cast<int*>(ws), reinterpret_cast<int*>(ws + o_kc),
          reinterpret_cast<float*>(ws + o_y), reinterpret_cast<float*>(ws + o_part)};
}

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

template <typename T, int N, int P>
hipError_t launch_sma_decode(const DecodeShape& s, const T* x, const float* dt, const float* A,
                             const T* Bm, const T* C, const T* Q, const T* E, float gate,
                             T* cache, uint8_t* cache8, float* cscale, float* h, float* dH_cur,
                             int* n_chunks, int* pos, T* y, void* workspace, int* flag,
                             hipStream_t st) {
  const long pairs = (long)s.B * s.H;
  DecodeWs ws = decode_ws(workspace, s.B, pairs, P);
  if (flag) ws.flag = flag;
  const int cps = (s.max_chunks + s.splits - 1) / s.splits;
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(N));
  const bool f8 = cache8 != nullptr;
  const DecodeArgs<T> a{x,     Bm,      C,       Q,      E,      dt,       A,
                        cache, cache8,  cscale,  h,      dH_cur, n_chunks, pos,
                        ws.kc, ws.yssd, ws.part, y,      gate,   scale_log2,
                        s.B,   s.H,     s.G,     s.S,    s.max_chunks, s.splits, cps};
  if (f8)
    hipLaunchKernelGGL((k_decode_state<T, N, P, true>), dim3(1, s.H, s.B), dim3(256), 0, st, x,
                       dt, A, Bm, C, nullptr, cache8, cscale, h, dH_cur, n_chunks, pos, ws.flag,
                       ws.kc, ws.yssd, s.H, s.G, s.S, s.max_chunks);
  else
    hipLaunchKernelGGL((k_decode_state<T, N, P, false>), dim3(1, s.H, s.B), dim3(256), 0, st, x,
                       dt, A, Bm, C, cache, nullptr, nullptr, h, dH_cur, n_chunks, pos, ws.flag,
                       ws.kc, ws.yssd, s.H, s.G, s.S, s.max_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(s.splits, s.H, s.B);
  if (s.splits == 1) {
    // the streaming workgroups also write y and advance the positions
    if (f8)
      hipLaunchKernelGGL((k_sma_decode_f8<T, N, P, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((k_sma_decode<T, N, P, true>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (f8)
    hipLaunchKernelGGL((k_sma_decode_f8<T, N, P, false>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_sma_decode<T, N, P, false>), grid, dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode_combine<T>), dim3(pairs), dim3(128), 0, st, ws.yssd, ws.part,
                     ws.kc, gate, y, n_chunks, pos, s.H, P, s.splits, s.S, s.max_chunks);
  return hipGetLastError();
}

template <typename T, int N, int P>
hipError_t launch_fp8_store(int B, int H, int n_mem, int first, int max_chunks, const float* src,
                            uint8_t* cache8, float* cscale, hipStream_t st) {
  if (n_mem == 0) return hipSuccess;
  hipLaunchKernelGGL((k_fp8_store<N, P>), dim3(n_mem, H, B), dim3(256), 0, st, src, n_mem, first,
                     cache8, cscale, H, max_chunks);
  return hipGetLastError();
}

#define DART_INST_DECODE(T, N, P)                                                               \
  template hipError_t launch_sma_decode<T, N, P>(                                               \
      const DecodeShape&, const T*, const float*, const float*, const T*, const T*, const T*,   \
      const T*, float, T*, uint8_t*, float*, float*, float*, int*, int*, T*, void*, int*,       \
      hipStream_t);                                                                             \
  template hipError_t launch_fp8_store<T, N, P>(int, int, int, int, int, const float*, uint8_t*, \
                                                float*, hipStream_t);
DART_FOR_EACH_SHAPE(DART_INST_DECODE)

}  // namespace dart
