// Mamba-2 chunked scan on gfx950: chunk state memories, inter-chunk state
// passing and the native chunk output (Pith review of DART, axiom ledger:
// the chunked scan splits the SSM output into intra- and inter-chunk terms
// and yields the chunk contributions dH[c]; "What carries the argument":
// dH[c] is the N x P contribution of chunk c to the chunk-boundary state).
//
// Decays are always formed as exp of a non-positive difference of log-decay
// sums (never exp(-acum) on its own, which overflows fp32 for long chunks).
#include "dart_launch.hpp"
#include "dart_shapes.hpp"

namespace dart {
namespace {

constexpr int kThreads = 256;  // 4 waves
constexpr int kKB = 64;        // tokens per K-block staged by k_chunk_state

// One workgroup per (chunk c, head h, batch b).
//   acum[s] = inclusive prefix sum of dt·A over the chunk (wave scan)
//   w_s     = exp(acum_end - acum_s)·dt_s
//   dH[c]   = Σ_s B_s (w_s x_s)ᵀ   as 16x16 MFMA tiles D[n][p], K = tokens
// Tokens are the contraction axis but the slow axis in memory, so each
// K-block of B and w∘x is written transposed into LDS ([n][s], [p][s]) and
// read back as contiguous fragments.
template <typename T, int N, int P>
__global__ __launch_bounds__(kThreads) void k_chunk_state(
    const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, float* __restrict__ acum, T* __restrict__ dH,
    float* __restrict__ dHf, int L, int H, int G, int S) {
  using MM = Mma<T>;
  constexpr int K = MM::K, KL = MM::KL;
  constexpr int VE = Vec16<T>::n;
  constexpr int LDK = kKB + VE;            // LDS row stride in elements (16-byte pad)
  constexpr int NT = (N / 16) * (P / 16);  // 16x16 output tiles
  constexpr int TPW = (NT + 3) / 4;        // tiles per wave
  __shared__ float sh_w[kMaxChunk];
  __shared__ float sh_part[4];
  __shared__ __align__(16) T sh_bt[N * LDK];
  __shared__ __align__(16) T sh_xt[P * LDK];

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int M = L / S, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const long tok0 = (long)b * L + (long)c * S;  // row of the chunk's first token in [B*L]
  const long pair = (long)b * H + h;

  // 1. log-decay prefix sum, one token per thread (S <= 256)
  const float dtv = tid < S ? dt[(tok0 + tid) * H + h] : 0.f;
  float v = dtv * A[h];
  for (int off = 1; off < 64; off <<= 1) {
    const float u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) sh_part[w] = v;
  __syncthreads();
  for (int i = 0; i < w; ++i) v += sh_part[i];
  const float total = sh_part[0] + sh_part[1] + sh_part[2] + sh_part[3];
  if (tid < S) {
    acum[(pair * M + c) * S + tid] = v;
    sh_w[tid] = exp_neg(total - v) * dtv;
  }
  __syncthreads();

  // 2. dH = Bᵀ (w∘x) over K-blocks of kKB tokens; the global loads of block
  //    i+1 are in flight while the MFMAs of block i run
  typedef typename Vec16<T>::vec vec_t;
  constexpr int XV = kKB * (P / VE) / kThreads;  // vectors per thread per block
  constexpr int BV = kKB * (N / VE) / kThreads;
  static_assert(XV * kThreads == kKB * (P / VE) && BV * kThreads == kKB * (N / VE),
                "k_chunk_state staging split");
  vec_t xr[XV], br[BV];
  auto fetch = [&](int s0) {
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + v * kThreads, s = i % kKB, pv = i / kKB;
      xr[v] = s0 + s < S ? load16(x + ((tok0 + s0 + s) * H + h) * P + pv * VE) : vec_t{};
    }
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + v * kThreads, s = i % kKB, nv = i / kKB;
      br[v] = s0 + s < S ? load16(Bm + ((tok0 + s0 + s) * G + g) * N + nv * VE) : vec_t{};
    }
  };
  floatx4 accv[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) accv[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  fetch(0);
  for (int s0 = 0; s0 < S; s0 += kKB) {
    // lanes take consecutive tokens, so the transposed LDS writes of one row
    // are contiguous
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + v * kThreads, s = i % kKB, pv = i / kKB;
      const float wv = s0 + s < S ? sh_w[s0 + s] : 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) sh_xt[(pv * VE + e) * LDK + s] = from_f32<T>(to_f32(xr[v][e]) * wv);
    }
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + v * kThreads, s = i % kKB, nv = i / kKB;
#pragma unroll
      for (int e = 0; e < VE; ++e) sh_bt[(nv * VE + e) * LDK + s] = br[v][e];
    }
    __syncthreads();
    if (s0 + kKB < S) fetch(s0 + kKB);
#pragma unroll
    for (int ks = 0; ks < kKB; ks += K) {
#pragma unroll
      for (int j = 0; j < TPW; ++j) {
        const int tile = w + 4 * j;
        if (tile < NT) {
          const int nb = tile / (P / 16), pb = tile % (P / 16);
          const auto a = MM::load(&sh_bt[(nb * 16 + col) * LDK + ks + grp * KL]);
          const auto bb = MM::load(&sh_xt[(pb * 16 + col) * LDK + ks + grp * KL]);
          accv[j] = MM::mma(a, bb, accv[j]);
        }
      }
    }
    __syncthreads();
  }

  // 3. store memory c value-axis-major: lane holds n = nb*16 + 4*grp + i, p = pb*16 + col
  const long base = (pair * M + c) * (long)(P * N);
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tile = w + 4 * j;
    if (tile < NT) {
      const int nb = tile / (P / 16), pb = tile % (P / 16);
      const long off = base + (long)(pb * 16 + col) * N + nb * 16 + 4 * grp;
      store4(dH + off, accv[j]);
      store4(dHf + off, accv[j]);
    }
  }
}

constexpr int kStKB = 64;  // tokens per K-block of k_chunk_state_tr

// LDS of one chunk's memory product: the K-block tiles during the product,
// afterwards the finished memory as f32 rows [p][n] (a 16-byte pad keeps the
// fragment writes conflict-free), the chunk's decay weights and the
// log-decay at its last token.
template <int N, int P>
struct alignas(16) ChunkMemLds {
  static constexpr int LDB = N + 16, LDX = P + 16;  // K-block row strides (elements)
  static constexpr int LDO = N + 4;                 // f32 memory row stride
  static constexpr int KB_BYTES = kStKB * (LDB + LDX) * 2;
  static constexpr int OUT_BYTES = P * LDO * 4;
  static constexpr int RAW = KB_BYTES > OUT_BYTES ? KB_BYTES : OUT_BYTES;
  unsigned char raw[RAW];
  float w[kMaxChunk];
  float part[4];
  float aend;
  __device__ float* mem() { return reinterpret_cast<float*>(raw); }
};

// Chunk state memory c of (batch b, head h), 16-bit io, computed by the 256
// threads tid = 0..255 of one part of the workgroup: the arithmetic of
// k_chunk_state with every HBM access in whole token rows.  B and w∘x
// K-blocks sit row-major in LDS ([s][n], [s][p]) and both MFMA operands are
// read with LDS transpose reads, so the token axis becomes each lane's k-run
// without a transposing store.  Lane group grp takes the k-slots
// s = ks + 4·grp + 0..3 and ks + 16 + 4·grp + 0..3 of a 32-token step in
// both operands (each read covers 16 consecutive rows: no LDS bank conflicts
// at either row stride).  The loads of K-block i+1 are in flight while
// block i multiplies.
// Writes acum of the chunk and leaves the f32 memory as rows [p][n] in
// sm.mem() and acum at the last token in sm.aend, both visible to the whole
// workgroup on return.  Contains workgroup barriers: every part of the
// workgroup calls it once, with the same S.
template <int N, int P>
__device__ __forceinline__ void chunk_memory_tr(const bf16* __restrict__ x,
                                                const float* __restrict__ dt,
                                                const float* __restrict__ A,
                                                const bf16* __restrict__ Bm,
                                                float* __restrict__ acum, int L, int H, int G,
                                                int S, int c, int h, int b, int tid,
                                                ChunkMemLds<N, P>& sm) {
  using MM = Mma<bf16>;
  using Lds = ChunkMemLds<N, P>;
  typedef bf16x8 vec_t;
  constexpr int VE = 8, K = MM::K;
  constexpr int LDB = Lds::LDB, LDX = Lds::LDX, LDO = Lds::LDO;
  constexpr int NB = N / 16;
  constexpr int NPB = P / 16;
  constexpr int NT = NB * NPB;        // 16x16 output tiles
  constexpr int TPW = (NT + 3) / 4;   // tiles per wave
  // wave w owns n-blocks w, w+4, ... (NBW of them) for every p-block when
  // NB % 4 == 0 (each operand fragment then feeds several tiles); otherwise
  // tile w + 4·j
  constexpr bool kGrid = NB % 4 == 0;
  constexpr int NBW = kGrid ? NB / 4 : 1;
  constexpr int XV = kStKB * (P / VE) / kThreads;  // vectors per thread per K-block
  constexpr int BV = kStKB * (N / VE) / kThreads;
  static_assert(XV * kThreads == kStKB * (P / VE) && BV * kThreads == kStKB * (N / VE),
                "chunk_memory_tr staging split");
  bf16* sh_b = reinterpret_cast<bf16*>(sm.raw);
  bf16* sh_x = sh_b + kStKB * LDB;
  float* sh_o = sm.mem();

  const int M = L / S, g = h / (H / G);
  const int lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const long tok0 = (long)b * L + (long)c * S;
  const long pair = (long)b * H + h;

  vec_t xr[XV], br[BV];
  auto fetch = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + v * kThreads, s = i / (P / VE), pv = i % (P / VE);
      xr[v] = s0 + s < S ? load16(x + ((tok0 + s0 + s) * H + h) * P + pv * VE) : vec_t{};
    }
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + v * kThreads, s = i / (N / VE), nv = i % (N / VE);
      br[v] = s0 + s < S ? load16(Bm + ((tok0 + s0 + s) * G + g) * N + nv * VE) : vec_t{};
    }
  };
  const float dtv = tid < S ? dt[(tok0 + tid) * H + h] : 0.f;
  fetch(0);

  // 1. log-decay prefix sum, one token per thread (S <= 256)
  float v = dtv * A[h];
  for (int off = 1; off < 64; off <<= 1) {
    const float u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) sm.part[w] = v;
  __syncthreads();
  for (int i = 0; i < w; ++i) v += sm.part[i];
  const float total = sm.part[0] + sm.part[1] + sm.part[2] + sm.part[3];
  if (tid < S) {
    acum[(pair * M + c) * S + tid] = v;
    sm.w[tid] = exp_neg(total - v) * dtv;
  }
  if (tid == S - 1) sm.aend = v;
  __syncthreads();

  // 2. dH[n][p] = sum_s B[s][n]·w_s·x[s][p] over K-blocks of kStKB tokens
  floatx4 acc[TPW];
#pragma unroll
  for (int j = 0; j < TPW; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += kStKB) {
#pragma unroll
    for (int v2 = 0; v2 < BV; ++v2) {
      const int i = tid + v2 * kThreads, s = i / (N / VE), nv = i % (N / VE);
      *reinterpret_cast<vec_t*>(&sh_b[s * LDB + nv * VE]) = br[v2];
    }
#pragma unroll
    for (int v2 = 0; v2 < XV; ++v2) {
      const int i = tid + v2 * kThreads, s = i / (P / VE), pv = i % (P / VE);
      const float wv = s0 + s < S ? sm.w[s0 + s] : 0.f;
      vec_t o;
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] = from_f32<bf16>(to_f32(xr[v2][e]) * wv);
      *reinterpret_cast<vec_t*>(&sh_x[s * LDX + pv * VE]) = o;
    }
    __syncthreads();
    if (s0 + kStKB < S) fetch(s0 + kStKB);
#pragma unroll
    for (int ks = 0; ks < kStKB; ks += K) {
      const int r0 = ks + 4 * grp + (col >> 2), c0 = 4 * (col & 3);
      // k-slots r0 .. (4 rows) and r0 + 16 .. of column c + col
      auto frag = [&](const bf16* tile, int ld, int cc) __attribute__((always_inline)) {
        const bf16x4 lo = lds_read_tr4(&tile[r0 * ld + cc + c0]);
        const bf16x4 hi = lds_read_tr4(&tile[(r0 + 16) * ld + cc + c0]);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      if constexpr (kGrid) {
        bf16x8 af[NBW], bfr[NPB];
#pragma unroll
        for (int q = 0; q < NBW; ++q) af[q] = frag(sh_b, LDB, (w + 4 * q) * 16);
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) bfr[pb] = frag(sh_x, LDX, pb * 16);
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
          for (int q = 0; q < NBW; ++q)
            acc[pb * NBW + q] = MM::mma(af[q], bfr[pb], acc[pb * NBW + q]);
      } else {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          const int tt = w + 4 * j;
          if (tt < NT)
            acc[j] = MM::mma(frag(sh_b, LDB, (tt % NB) * 16), frag(sh_x, LDX, (tt / NB) * 16),
                             acc[j]);
        }
      }
    }
    __syncthreads();
  }

  // 3. memory c value-axis-major ([p][n]): lane holds n = nb*16 + 4*grp + i,
  //    p = pb*16 + col (the loop's last barrier has released the K-block
  //    tiles)
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int tt = w + 4 * j;
    if (kGrid || tt < NT) {
      const int nb = kGrid ? w + 4 * (j % NBW) : tt % NB, pb = kGrid ? j / NBW : tt / NB;
      *reinterpret_cast<floatx4*>(&sh_o[(pb * 16 + col) * LDO + nb * 16 + 4 * grp]) = acc[j];
    }
  }
  __syncthreads();
}

// Whole rows of memory c from sm.mem() to dH (io, rounded to nearest even)
// and, when dHf is not null, to dHf (f32), by the 256 threads tid.
template <int N, int P>
__device__ __forceinline__ void store_memory_rows(ChunkMemLds<N, P>& sm, bf16* __restrict__ dH,
                                                  float* __restrict__ dHf, long base, int tid) {
  constexpr int LDO = ChunkMemLds<N, P>::LDO;
  const float* sh_o = sm.mem();
  constexpr int F4 = P * N / 4;  // float4s of one memory
  if (dHf) {
#pragma unroll
    for (int v = 0; v < (F4 + kThreads - 1) / kThreads; ++v) {
      const int i = tid + v * kThreads;
      if (F4 % kThreads != 0 && i >= F4) break;
      const int p = i / (N / 4), n = (i % (N / 4)) * 4;
      *reinterpret_cast<floatx4*>(dHf + base + (long)i * 4) =
          *reinterpret_cast<const floatx4*>(&sh_o[p * LDO + n]);
    }
  }
#pragma unroll
  for (int v = 0; v < (F4 / 2 + kThreads - 1) / kThreads; ++v) {
    const int i = tid + v * kThreads;
    if ((F4 / 2) % kThreads != 0 && i >= F4 / 2) break;
    const int p = i / (N / 8), n = (i % (N / 8)) * 8;
    const floatx4 lo = *reinterpret_cast<const floatx4*>(&sh_o[p * LDO + n]);
    const floatx4 hi = *reinterpret_cast<const floatx4*>(&sh_o[p * LDO + n + 4]);
    *reinterpret_cast<bf16x8*>(dH + base + (long)i * 8) =
        bf16x8{from_f32<bf16>(lo[0]), from_f32<bf16>(lo[1]), from_f32<bf16>(lo[2]),
               from_f32<bf16>(lo[3]), from_f32<bf16>(hi[0]), from_f32<bf16>(hi[1]),
               from_f32<bf16>(hi[2]), from_f32<bf16>(hi[3])};
  }
}

// One workgroup per (chunk c, head h, batch b): memory c as io and f32 rows.
// At most 128 VGPRs (four waves per SIMD): at N = 128, P = 64 the kernel
// fits without spills and four workgroups share a CU instead of three
// (3.5% faster at the ~370M layer shape, same code otherwise).
template <int N, int P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(4))) void
k_chunk_state_tr(
    const bf16* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const bf16* __restrict__ Bm, float* __restrict__ acum, bf16* __restrict__ dH,
    float* __restrict__ dHf, int L, int H, int G, int S) {
  __shared__ ChunkMemLds<N, P> sm;
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  chunk_memory_tr<N, P>(x, dt, A, Bm, acum, L, H, G, S, c, h, b, threadIdx.x, sm);
  const long pair = (long)b * H + h;
  store_memory_rows<N, P>(sm, dH, dHf, (pair * (L / S) + c) * (long)(P * N), threadIdx.x);
}

// Chunk memories and the inter-chunk state recurrence in one pass, 16-bit io.
// A workgroup of CPW parts (256 threads each) takes CPW consecutive chunks
// j·CPW .. j·CPW + CPW - 1 of one (batch, head): each part computes its
// chunk's memory (chunk_memory_tr) and writes it as io rows; then the
// workgroup waits for the f32 state entering chunk j·CPW from the workgroup
// of link j - 1 (h0 or zero for j = 0), advances it through its chunks,
//   H[c+1] = exp(acum[c, S-1])·H[c] + dH[c]          (f32, in chunk order)
// hands H[(j+1)·CPW] to link j + 1 (or writes it as h_final), and writes
// H_in[c] = io(H[c]) for its chunks.  The hand-over goes through a
// two-slot f32 ring per (batch, head) (link j writes slot j % 2 after reading
// slot (j - 1) % 2, so a slot is rewritten only after its reader has
// published) and a 64-bit flag per (batch, head) holding (tag << 32) | links
// done.  Ring values and flag are relaxed agent-scope atomics, each access
// coherent across the XCDs' L2s by itself; the flag is stored only after
// every wave's ring stores are performed (vmcnt(0), then a barrier), and the
// ring is read only after the flag was seen (a barrier after the poll).  A
// release/acquire pair would add an L2-wide write-back per hand-over.  tag is
// distinct per call, so a flag left by an earlier call never matches.
// Link j waits only for link j - 1, whose block index is lower: blocks start
// in index order, so every awaited workgroup is already resident.  The wait
// is bounded all the same: after kScanSpinLimit polls (or once another
// wait of this call has given up) it counts a failure in err[0], records
// the tag in err[1] and continues, so the kernel always ends.
// Block order: with xcd_major, block i runs on XCD i % 8 and holds the
// (batch, group) pairs bg ≡ i % 8 (mod 8), chunk-major within the XCD, so
// a (batch, head)'s chain and a group's shared B rows stay in one L2.
constexpr int kScanSpinLimit = 1 << 20;
constexpr size_t kLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950

template <int N, int P, int CPW>
__global__ __launch_bounds__(kThreads * CPW) void k_chunk_scan(
    const bf16* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const bf16* __restrict__ Bm, const float* __restrict__ h0, float* __restrict__ acum,
    bf16* __restrict__ dH, float* __restrict__ dHf, bf16* __restrict__ H_in,
    float* __restrict__ h_final, float* __restrict__ ring, unsigned long long* flags, int* err,
    unsigned tag, int L, int H, int G, int S, int BH, int xcd_major) {
  constexpr int PN = P * N;
  constexpr int LDO = ChunkMemLds<N, P>::LDO;
  constexpr int TT = kThreads * CPW;
  constexpr int F4 = PN / 4;
  constexpr int V = (F4 + TT - 1) / TT;  // state float4s per thread
  __shared__ ChunkMemLds<N, P> sm[CPW];

  const int M = L / S, NJ = M / CPW;
  const int i = blockIdx.x;
  int pair, j;
  if (xcd_major) {
    const int per = BH >> 3, hpg = H / G;  // pairs per XCD, heads per group
    const int jj = i >> 3;
    j = jj / per;
    const int lp = jj - j * per;
    pair = ((i & 7) + 8 * (lp / hpg)) * hpg + lp % hpg;
  } else {
    j = i / BH;
    pair = i - j * BH;
  }
  const int b = pair / H, h = pair - b * H;
  const int part = threadIdx.x >> 8, tid = threadIdx.x & (kThreads - 1);
  const int c0 = j * CPW;

  chunk_memory_tr<N, P>(x, dt, A, Bm, acum, L, H, G, S, c0 + part, h, b, tid, sm[part]);
  store_memory_rows<N, P>(sm[part], dH, dHf, ((long)pair * M + c0 + part) * (long)PN, tid);

  // the state entering chunk c0
  floatx4 st[V];
  if (j == 0) {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e4 = threadIdx.x + v * TT;
      st[v] = h0 && e4 < F4 ? reinterpret_cast<const floatx4*>(h0 + (long)pair * PN)[e4]
                            : floatx4{0.f, 0.f, 0.f, 0.f};
    }
  } else {
    if (threadIdx.x == 0) {
      const unsigned long long want = ((unsigned long long)tag << 32) | (unsigned)j;
      for (int it = 0;; ++it) {
        if (__hip_atomic_load(&flags[pair], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want)
          break;
        if (it >= kScanSpinLimit ||
            ((it & 63) == 63 &&
             __hip_atomic_load(&err[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (int)tag)) {
          __hip_atomic_fetch_add(&err[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(&err[1], (int)tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();  // no thread reads the slot before the flag was seen
    const float* src = ring + ((long)pair * 2 + ((j + 1) & 1)) * PN;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e4 = threadIdx.x + v * TT;
      if (e4 < F4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          st[v][q] = __hip_atomic_load(&src[e4 * 4 + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        st[v] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // advance through the workgroup's chunks, keeping the entering states
  floatx4 hin[CPW][V];
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    const float dec = exp_neg(sm[k].aend);
    const float* mem = sm[k].mem();
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e4 = threadIdx.x + v * TT;
      hin[k][v] = st[v];
      if (e4 < F4) {
        const int p = e4 / (N / 4), n = (e4 % (N / 4)) * 4;
        st[v] = dec * st[v] + *reinterpret_cast<const floatx4*>(&mem[p * LDO + n]);
      }
    }
  }

  // hand the state to the next link, or write it as h_final
  if (j + 1 < NJ) {
    float* dst = ring + ((long)pair * 2 + (j & 1)) * PN;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e4 = threadIdx.x + v * TT;
      if (e4 < F4) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __hip_atomic_store(&dst[e4 * 4 + q], st[v][q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    wait_fence<vmcnt_imm(0)>();  // this wave's slot stores are performed at agent scope
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(&flags[pair], ((unsigned long long)tag << 32) | (unsigned)(j + 1),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e4 = threadIdx.x + v * TT;
      if (e4 < F4) reinterpret_cast<floatx4*>(h_final + (long)pair * PN)[e4] = st[v];
    }
  }

  // H_in rows of the workgroup's chunks
#pragma unroll
  for (int k = 0; k < CPW; ++k) {
    bf16* dst = H_in + ((long)pair * M + c0 + k) * PN;
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int e4 = threadIdx.x + v * TT;
      if (e4 < F4) store4(dst + e4 * 4, hin[k][v]);
    }
  }
}

// H[0] = h0, H[c+1] = exp(acum_end[c])·H[c] + dH_f32[c] in f32; H_in[c] =
// io(H[c]) for c < M and h_final = H[M].  One thread per four state entries
// of one (batch, head), serial over chunks.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_state_pass(
    const float* __restrict__ acum, const float* __restrict__ dHf, const float* __restrict__ h0,
    T* __restrict__ H_in, float* __restrict__ h_final, int H, int M, int S, int PN) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int e4 = blockIdx.x * kThreads + threadIdx.x;
  if (e4 * 4 >= PN) return;
  const long pair = (long)b * H + h;
  const int q = PN / 4;
  const floatx4* src = reinterpret_cast<const floatx4*>(dHf + pair * M * (long)PN) + e4;
  T* dst = H_in + pair * M * (long)PN + e4 * 4;
  const float* ac_end = acum + pair * M * (long)S + (S - 1);
  floatx4 st = h0 ? reinterpret_cast<const floatx4*>(h0 + pair * PN)[e4] : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int c = 0; c < M; ++c) {
    store4(dst + (long)c * PN, st);
    const float dec = exp_neg(ac_end[(long)c * S]);
    st = dec * st + src[(long)c * q];
  }
  reinterpret_cast<floatx4*>(h_final + pair * PN)[e4] = st;
}

constexpr int kOutWaves = 8;  // two per SIMD
constexpr int kOutThreads = 64 * kOutWaves;
constexpr int kMaxBlk = kMaxChunk / 16;  // 16-token blocks per chunk

// LDS of k_chunk_out: phase 1 holds B_k, phase 2 reuses the same bytes for
// xᵀ and H_in[k]ᵀ of one head
template <typename T, int N, int P>
struct ChunkOutLds {
  static constexpr int VE = Vec16<T>::n;
  static constexpr int LDX = kMaxChunk + VE;  // xᵀ rows [p][j]
  static constexpr int LDH = N + VE;          // H_inᵀ rows [p][n]
  static constexpr int LDB = N + VE;          // B rows [j][n]
  static constexpr size_t phase1 = size_t(kMaxChunk) * LDB * sizeof(T);
  static constexpr size_t phase2 = (size_t(P) * LDX + size_t(P) * LDH) * sizeof(T);
  static constexpr size_t bytes = phase1 > phase2 ? phase1 : phase2;
};

// Native chunk output for one (chunk k, head group g, batch b): the heads of
// a group share B and C, so the C·Bᵀ tiles are computed once per workgroup
// and reused for every head of the group.
//
// Phase 1: B_k is staged in LDS; each wave owns the 16-token blocks
//   tb0 = w and tb1 = 15 - w (balanced causal work) and computes the tiles
//   Gᵀ[j][t] = B_j·C_t (K = n) for every key block jb <= tb into registers.
// Phase 2, per head: xᵀ and H_in[k]ᵀ are staged in LDS (over B) and
//   inter: Yᵀ += H_in[k]ᵀ C_tᵀ              (K = n), scaled by exp(acum_t)
//   intra: Yᵀ += xᵀ (Gᵀ ∘ W)                (K = j)
//   with W[j][t] = exp(acum_t - acum_j)·dt_j for j <= t, 0 above.  W is
//   factored per tile through the end of its key block, e(jb):
//   u = 2^(A_t - A_e(jb)) (one exp per lane and tile) and
//   v_j = 2^(A_e(jb) - A_j + log2 dt_j) (per key, once per head), A = acum·log2(e),
//   for key blocks below the token's own block, where u <= 1 and v_j <= dt_j;
//   an underflowing u means a weight far below fp32 resolution of the sum.
//   On the diagonal block u would be a growth factor (up to the log-decay of
//   15 tokens, which overflows for large dt·|A|), so there each weight is
//   formed directly as 2^(A_t - A_j + log2 dt_j).
// The weighted tile stays in registers: its D layout (rows j = 16·jb +
// 4·grp + i of column t) is the B operand of the second product, with the
// k-slots of xᵀ's A operand assigned the same j's.
template <typename T, int N, int P>
__global__ __launch_bounds__(kOutThreads) void k_chunk_out(
    const T* __restrict__ x, const float* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ C, const float* __restrict__ acum, const T* __restrict__ H_in,
    T* __restrict__ y_ssd, int L, int H, int G, int S) {
  static_assert(std::is_same<T, float>::value, "16-bit io uses k_chunk_out_tr");
  using MM = Mma<T>;
  using Lds = ChunkOutLds<T, N, P>;
  typedef typename Vec16<T>::vec vec_t;
  constexpr int K = MM::K, KL = MM::KL, VE = Vec16<T>::n;
  constexpr int LDX = Lds::LDX, LDH = Lds::LDH, LDB = Lds::LDB;
  constexpr int NKK = N / K, NPB = P / 16;
  __shared__ __align__(16) unsigned char sh_raw[Lds::bytes];
  __shared__ __align__(16) float sh_at[kMaxChunk];  // A_s = acum_s·log2(e)
  __shared__ __align__(16) float sh_v[kMaxChunk];   // v_j
  __shared__ __align__(16) float sh_ld[kMaxChunk];  // log2 dt_j
  __shared__ float sh_ae[kMaxBlk];                  // A at the end of each block
  T* sh_b = reinterpret_cast<T*>(sh_raw);
  T* sh_xt = reinterpret_cast<T*>(sh_raw);
  T* sh_ht = reinterpret_cast<T*>(sh_raw) + P * LDX;

  const int k = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int M = L / S, hpg = H / G, NB = S / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const long tok0 = (long)b * L + (long)k * S;
  const int tb0 = w, tb1 = 2 * kOutWaves - 1 - w;
  const bool has0 = tb0 < NB, has1 = tb1 < NB;

  // ---- phase 1: C·Bᵀ tiles of this wave's token blocks ----
  {
    constexpr int BV = (kMaxChunk * (N / VE) + kOutThreads - 1) / kOutThreads;
    vec_t br[BV];
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + v * kOutThreads;
      if (i < S * (N / VE)) {
        const int s = i / (N / VE), nv = i % (N / VE);
        br[v] = load16(Bm + ((tok0 + s) * G + g) * N + nv * VE);
      }
    }
#pragma unroll
    for (int v = 0; v < BV; ++v) {
      const int i = tid + v * kOutThreads;
      if (i < S * (N / VE)) {
        const int s = i / (N / VE), nv = i % (N / VE);
        *reinterpret_cast<vec_t*>(&sh_b[s * LDB + nv * VE]) = br[v];
      }
    }
  }
  floatx4 g0[kMaxBlk], g1[kMaxBlk];
  {
  typename MM::frag cf0[NKK], cf1[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int t0 = has0 ? tb0 * 16 + col : 0, t1 = has1 ? tb1 * 16 + col : 0;
    cf0[kk] = MM::load(C + ((tok0 + t0) * G + g) * N + kk * K + grp * KL);
    cf1[kk] = MM::load(C + ((tok0 + t1) * G + g) * N + kk * K + grp * KL);
  }
  __syncthreads();
#pragma unroll
  for (int jb = 0; jb < kMaxBlk; ++jb) {
    g0[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
    g1[jb] = floatx4{0.f, 0.f, 0.f, 0.f};
    if (has0 && jb <= tb0) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        g0[jb] = MM::mma(MM::load(&sh_b[(jb * 16 + col) * LDB + kk * K + grp * KL]), cf0[kk],
                         g0[jb]);
    }
    if (has1 && jb <= tb1) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        g1[jb] = MM::mma(MM::load(&sh_b[(jb * 16 + col) * LDB + kk * K + grp * KL]), cf1[kk],
                         g1[jb]);
    }
  }
  }
  __syncthreads();  // B is dead; phase 2 reuses its LDS

  // ---- phase 2: the heads of the group ----
  constexpr int XV = (kMaxChunk * (P / VE) + kOutThreads - 1) / kOutThreads;
  constexpr int HV = (P * N / 4 + kOutThreads - 1) / kOutThreads;
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
    const float* hsrc = H_in + (pair * M + k) * (long)(P * N);
    vec_t xr[XV];
    floatx4 hr[HV];
    float ar = 0.f, ae = 0.f, dr = 1.f;
    if (tid < S) {
      ar = acum[(pair * M + k) * S + tid];
      ae = acum[(pair * M + k) * S + (tid | 15)];
      dr = dt[(tok0 + tid) * H + h];
    }
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + v * kOutThreads;
      if (i < S * (P / VE)) {
        const int s = i % S, pv = i / S;
        xr[v] = load16(x + ((tok0 + s) * H + h) * P + pv * VE);
      }
    }
#pragma unroll
    for (int v = 0; v < HV; ++v) {
      const int i = tid + v * kOutThreads;
      if (i < P * N / 4) hr[v] = reinterpret_cast<const floatx4*>(hsrc)[i];
    }
    if (tid < S) {
      const float a2 = ar * kLog2e, e2 = ae * kLog2e;
      const float ld = __builtin_amdgcn_logf(dr);
      sh_at[tid] = a2;
      sh_ld[tid] = ld;
      sh_v[tid] = exp2_fast(e2 - a2 + ld);
      if ((tid & 15) == 15) sh_ae[tid >> 4] = a2;
    }
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + v * kOutThreads;
      if (i < S * (P / VE)) {
        const int s = i % S, pv = i / S;
#pragma unroll
        for (int e = 0; e < VE; ++e) sh_xt[(pv * VE + e) * LDX + s] = xr[v][e];
      }
    }
#pragma unroll
    for (int v = 0; v < HV; ++v) {
      const int i = tid + v * kOutThreads;
      if (i < P * N / 4) {
        const int p = (i * 4) / N, n = (i * 4) % N;
#pragma unroll
        for (int e = 0; e < 4; ++e) sh_ht[p * LDH + n + e] = from_f32<T>(hr[v][e]);
      }
    }
    __syncthreads();

    auto one_block = [&](int tb, const floatx4 (&gt)[kMaxBlk]) {
      const int t = tb * 16 + col;
      // C fragments again (L2 hits): keeping them live across the head loop
      // would spill the tiles
      typename MM::frag cf[NKK];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        cf[kk] = MM::load(C + ((tok0 + t) * G + g) * N + kk * K + grp * KL);
      floatx4 yin[NPB], yia[NPB];
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        yin[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
        yia[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          yin[pb] = MM::mma(MM::load(&sh_ht[(pb * 16 + col) * LDH + kk * K + grp * KL]), cf[kk],
                            yin[pb]);
      const float at_t = sh_at[t];
      // weighted tile jb (rows j = jb*16 + 4*grp + i, column t).  Below the
      // diagonal block both factors are <= 1·dt_j; on it u would exceed 1
      // (by up to the log-decay of 15 tokens), so each weight is formed
      // directly as 2^(A_t - A_j + log2 dt_j) with A_t - A_j <= 0.
      auto weights = [&](int jb, floatx4 tile) {
        floatx4 wv;
        if (jb < tb) {
          const float u = exp2_fast(at_t - sh_ae[jb]);
          const floatx4 vj = *reinterpret_cast<const floatx4*>(&sh_v[jb * 16 + 4 * grp]);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) wv[i4] = tile[i4] * (u * vj[i4]);
        } else {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int j = jb * 16 + 4 * grp + i4;
            wv[i4] = j <= t ? tile[i4] * exp2_fast((at_t - sh_at[j]) + sh_ld[j]) : 0.f;
          }
        }
        return wv;
      };
      if constexpr (std::is_same<T, float>::value) {
#pragma unroll
        for (int jb = 0; jb < kMaxBlk; ++jb) {
          if (jb <= tb) {
            const floatx4 wv = weights(jb, gt[jb]);
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
              const int j = jb * 16 + 4 * grp + i4;
#pragma unroll
              for (int pb = 0; pb < NPB; ++pb)
                yia[pb] = MM::mma(sh_xt[(pb * 16 + col) * LDX + j], wv[i4], yia[pb]);
            }
          }
        }
      } else {
        // S % 32 == 0, so the pair (jb0, jb0 + 1) never leaves the chunk
#pragma unroll
        for (int jb0 = 0; jb0 < kMaxBlk; jb0 += 2) {
          if (jb0 <= tb) {
            const floatx4 w0 = weights(jb0, gt[jb0]), w1 = weights(jb0 + 1, gt[jb0 + 1]);
            const bf16x8 bfr = {from_f32<bf16>(w0[0]), from_f32<bf16>(w0[1]),
                                from_f32<bf16>(w0[2]), from_f32<bf16>(w0[3]),
                                from_f32<bf16>(w1[0]), from_f32<bf16>(w1[1]),
                                from_f32<bf16>(w1[2]), from_f32<bf16>(w1[3])};
#pragma unroll
            for (int pb = 0; pb < NPB; ++pb) {
              const bf16* row = &sh_xt[(pb * 16 + col) * LDX];
              const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + jb0 * 16 + 4 * grp);
              const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + (jb0 + 1) * 16 + 4 * grp);
              const bf16x8 afr = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
              yia[pb] = MM::mma(afr, bfr, yia[pb]);
            }
          }
        }
      }
      const float dec_t = exp2_fast(at_t);
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
        store4(y_ssd + ((tok0 + t) * H + h) * P + pb * 16 + 4 * grp, yia[pb] + dec_t * yin[pb]);
    };
    if (has0) one_block(tb0, g0);
    if (has1) one_block(tb1, g1);
    __syncthreads();  // the next head overwrites the LDS
  }
}

// LDS plan of k_chunk_out_tr.  Row strides carry a 32-byte pad (see the
// fragment-read notes in k_sma.hip); phase 1 holds the B and C tiles,
// phase 2 reuses the same bytes for x, H_in[k]ᵀ and, when it fits, y.
template <int N, int P>
struct ChunkOutTr {
  static constexpr int LDC = N + 16;  // B and C rows [s][n]
  static constexpr int LDX = P + 16;  // x rows [s][p]
  static constexpr int LDH = N + 16;  // H_in[k]ᵀ rows [p][n]
  static constexpr int LDY = P + 16;  // y rows [t][p]
  // the next head's x and H_in[k] are fetched into registers while the
  // current head computes, and y leaves through LDS as whole token rows,
  // when registers and LDS allow (P <= 64)
  static constexpr bool kPrefetch = P <= 64;
  static constexpr bool kStageY = P <= 64;
  static constexpr size_t phase1 = 2ull * kMaxChunk * LDC * sizeof(bf16);
  static constexpr size_t phase2 =
      (size_t(kMaxChunk) * LDX + size_t(P) * LDH + (kStageY ? size_t(kMaxChunk) * LDY : 0)) *
      sizeof(bf16);
  static constexpr size_t bytes = phase1 > phase2 ? phase1 : phase2;
};

// Native chunk output, 16-bit io: the arithmetic of k_chunk_out (same
// tiles, same factored weights, same k-slot pairing of two key blocks), with
// every HBM access in whole token rows.  x stays row-major in LDS and the
// xᵀ operand of the intra product is read with LDS transpose reads; B and C
// are staged row-major once per workgroup.  The C·Bᵀ tiles of a wave's two
// token blocks (at most kMaxBlk + 2 with the pairing) sit in one slot array:
// token block tb0's tile jb in slot jb, tb1's tile jb in slot
// kMaxBlk + 1 - jb, so every register index stays a compile-time constant.
template <int N, int P>
__global__ __launch_bounds__(kOutThreads) void k_chunk_out_tr(
    const bf16* __restrict__ x, const float* __restrict__ dt, const bf16* __restrict__ Bm,
    const bf16* __restrict__ C, const float* __restrict__ acum, const bf16* __restrict__ H_in,
    bf16* __restrict__ y_ssd, int L, int H, int G, int S) {
  using MM = Mma<bf16>;
  using Lds = ChunkOutTr<N, P>;
  typedef bf16x8 vec_t;
  constexpr int VE = 8, K = MM::K, KL = MM::KL;
  constexpr int LDC = Lds::LDC, LDX = Lds::LDX, LDH = Lds::LDH, LDY = Lds::LDY;
  constexpr int NKK = N / K, NPB = P / 16;
  constexpr int NSLOT = kMaxBlk + 2;
  constexpr int RV = kMaxChunk * (N / VE) / kOutThreads;  // B or C vectors per thread
  constexpr int XV = kMaxChunk * (P / VE) / kOutThreads;  // x or y vectors per thread
  constexpr int HQ = P * N / VE;                          // H_in[k] as 16-byte vectors
  constexpr int HV = (HQ + kOutThreads - 1) / kOutThreads;
  static_assert(RV * kOutThreads == kMaxChunk * (N / VE) &&
                    XV * kOutThreads == kMaxChunk * (P / VE),
                "k_chunk_out_tr staging split");
  static_assert(kOutWaves * 2 == kMaxBlk, "two token blocks per wave");
  __shared__ __align__(16) unsigned char sh_raw[Lds::bytes];
  __shared__ __align__(16) float sh_at[kMaxChunk];  // A_s = acum_s·log2(e)
  __shared__ __align__(16) float sh_v[kMaxChunk];   // v_j
  __shared__ __align__(16) float sh_ld[kMaxChunk];  // log2 dt_j
  bf16* sh_b = reinterpret_cast<bf16*>(sh_raw);
  bf16* sh_c = sh_b + kMaxChunk * LDC;
  bf16* sh_x = reinterpret_cast<bf16*>(sh_raw);
  bf16* sh_h = sh_x + kMaxChunk * LDX;
  bf16* sh_y = sh_h + P * LDH;

  const int k = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int M = L / S, hpg = H / G, NB = S / 16;
  // the wave index is uniform: scalar branches on the token blocks it owns
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const long tok0 = (long)b * L + (long)k * S;
  const int tb0 = w, tb1 = 2 * kOutWaves - 1 - w;
  const bool has0 = tb0 < NB, has1 = tb1 < NB;
  const int n0 = has0 ? 2 * (tb0 / 2 + 1) : 0;  // slots of tb0 (pairs of key blocks)
  const int n1 = has1 ? 2 * (tb1 / 2 + 1) : 0;

  // per-head inputs, fetched one head ahead when kPrefetch
  vec_t xr[XV], hr[HV];
  float ar = 0.f, dr = 1.f;
  auto load_head = [&](int hh) __attribute__((always_inline)) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + v * kOutThreads, s = i / (P / VE), pv = i % (P / VE);
      if (s < S) xr[v] = load16(x + ((tok0 + s) * H + h) * P + pv * VE);
    }
    const vec_t* hsrc = reinterpret_cast<const vec_t*>(H_in + (pair * M + k) * (long)(P * N));
#pragma unroll
    for (int v = 0; v < HV; ++v) {
      const int i = tid + v * kOutThreads;
      if (HQ % kOutThreads == 0 || i < HQ) hr[v] = hsrc[i];
    }
    if (tid < S) {
      ar = acum[(pair * M + k) * S + tid];
      dr = dt[(tok0 + tid) * H + h];
    }
  };

  // ---- phase 1: B and C rows -> LDS; C·Bᵀ tiles of this wave's blocks ----
  {
    vec_t br[RV], cr[RV];
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const int i = tid + v * kOutThreads, s = i / (N / VE), nv = i % (N / VE);
      if (s < S) {
        br[v] = load16(Bm + ((tok0 + s) * G + g) * N + nv * VE);
        cr[v] = load16(C + ((tok0 + s) * G + g) * N + nv * VE);
      }
    }
    if (Lds::kPrefetch) load_head(0);
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const int i = tid + v * kOutThreads, s = i / (N / VE), nv = i % (N / VE);
      if (s < S) {
        *reinterpret_cast<vec_t*>(&sh_b[s * LDC + nv * VE]) = br[v];
        *reinterpret_cast<vec_t*>(&sh_c[s * LDC + nv * VE]) = cr[v];
      }
    }
  }
  __syncthreads();
  // C fragments (B operand: column t, k-slots n) of the two token blocks
  typename MM::frag cf0[NKK], cf1[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int t0 = has0 ? tb0 * 16 + col : col, t1 = has1 ? tb1 * 16 + col : col;
    cf0[kk] = MM::load(&sh_c[t0 * LDC + kk * K + grp * KL]);
    cf1[kk] = MM::load(&sh_c[t1 * LDC + kk * K + grp * KL]);
  }
  floatx4 gs[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    gs[sl] = floatx4{0.f, 0.f, 0.f, 0.f};
    const bool is0 = sl < n0;
    const int jb = is0 ? sl : NSLOT - 1 - sl;
    const bool live = is0 ? sl <= tb0 : (jb < n1 && jb <= tb1);
    if (live) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        gs[sl] = MM::mma(MM::load(&sh_b[(jb * 16 + col) * LDC + kk * K + grp * KL]),
                         is0 ? cf0[kk] : cf1[kk], gs[sl]);
      // causal mask of the diagonal tile (key j = jb*16 + 4*grp + i after
      // query t = jb*16 + col), applied once for all heads
      if (jb == (is0 ? tb0 : tb1)) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) gs[sl][i4] = 4 * grp + i4 <= col ? gs[sl][i4] : 0.f;
      }
    }
  }
  __syncthreads();  // B and C are dead; phase 2 reuses their LDS

  // ---- phase 2: the heads of the group ----
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    if (!Lds::kPrefetch) load_head(hh);
    // stage head hh: x rows, H_in[k]ᵀ rows, log-decay factors
#pragma unroll
    for (int v = 0; v < XV; ++v) {
      const int i = tid + v * kOutThreads, s = i / (P / VE), pv = i % (P / VE);
      if (s < S) *reinterpret_cast<vec_t*>(&sh_x[s * LDX + pv * VE]) = xr[v];
    }
#pragma unroll
    for (int v = 0; v < HV; ++v) {
      const int i = tid + v * kOutThreads;
      if (HQ % kOutThreads == 0 || i < HQ) {
        const int p = (i * VE) / N, n = (i * VE) % N;
        *reinterpret_cast<vec_t*>(&sh_h[p * LDH + n]) = hr[v];
      }
    }
    {
      // A at the end of this thread's 16-token block comes from lane tid|15
      // of the same wave
      const float a2 = ar * kLog2e;
      const float e2 = __shfl(a2, lane | 15);
      if (tid < S) {
        const float ld = __builtin_amdgcn_logf(dr);
        sh_at[tid] = a2;
        sh_ld[tid] = ld;
        sh_v[tid] = exp2_fast(e2 - a2 + ld);
      }
    }
    __syncthreads();
    if (Lds::kPrefetch && hh + 1 < hpg) load_head(hh + 1);

    // one token block, in NPH passes over the value axis of NPP p-blocks each
    // (four passes at P = 128 keep the accumulators inside the register file)
    constexpr int NPH = NPB > 4 ? 4 : 1, NPP = NPB / NPH;
    auto block_out = [&](int tb, const typename MM::frag (&cf)[NKK], auto pick)
        __attribute__((always_inline)) {
      const int t = tb * 16 + col;
      const float at_t = sh_at[t];
#pragma unroll
      for (int ph = 0; ph < NPH; ++ph) {
      floatx4 yin[NPP], yia[NPP];
#pragma unroll
      for (int q = 0; q < NPP; ++q) {
        const int pb = ph * NPP + q;
        yin[q] = floatx4{0.f, 0.f, 0.f, 0.f};
        yia[q] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          yin[q] = MM::mma(MM::load(&sh_h[(pb * 16 + col) * LDH + kk * K + grp * KL]), cf[kk],
                           yin[q]);
      }
      // weighted tile jb (rows j = jb*16 + 4*grp + i, column t).  The tiles
      // are causally masked already.  Below the diagonal block the factored
      // weight u·v_j has both factors <= 1·dt_j; on the diagonal block each
      // weight is 2^(A_t - A_j + log2 dt_j) with A_t - A_j <= 0 for the
      // unmasked keys; above it (the second block of a pair) it is zero.
      // tb is wave-uniform, so these are scalar branches.
      auto weights = [&](int jb, floatx4 tile) __attribute__((always_inline)) {
        floatx4 wv = floatx4{0.f, 0.f, 0.f, 0.f};
        if (jb < tb) {
          const float u = exp2_fast(at_t - sh_at[jb * 16 + 15]);
          const floatx4 vj = *reinterpret_cast<const floatx4*>(&sh_v[jb * 16 + 4 * grp]);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) wv[i4] = (tile[i4] * u) * vj[i4];
        } else if (jb == tb) {
          const floatx4 aj = *reinterpret_cast<const floatx4*>(&sh_at[jb * 16 + 4 * grp]);
          const floatx4 lj = *reinterpret_cast<const floatx4*>(&sh_ld[jb * 16 + 4 * grp]);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            wv[i4] = 4 * grp + i4 <= col ? tile[i4] * exp2_fast((at_t - aj[i4]) + lj[i4]) : 0.f;
        }
        return wv;
      };
#pragma unroll
      for (int jb0 = 0; jb0 < kMaxBlk; jb0 += 2) {
        if (jb0 <= tb) {
          floatx4 t0, t1;
          pick(jb0, t0, t1);
          const floatx4 w0 = weights(jb0, t0), w1 = weights(jb0 + 1, t1);
          const bf16x8 bfr = {from_f32<bf16>(w0[0]), from_f32<bf16>(w0[1]),
                              from_f32<bf16>(w0[2]), from_f32<bf16>(w0[3]),
                              from_f32<bf16>(w1[0]), from_f32<bf16>(w1[1]),
                              from_f32<bf16>(w1[2]), from_f32<bf16>(w1[3])};
          // xᵀ operand: rows p, k-slots j = jb0*16 + 4*grp + 0..3 and
          // (jb0+1)*16 + 4*grp + 0..3, by transpose reads of the x rows
          const int r0 = jb0 * 16 + 4 * grp + (col >> 2), c0 = 4 * (col & 3);
#pragma unroll
          for (int q = 0; q < NPP; ++q) {
            const int pb = ph * NPP + q;
            const bf16x4 lo = lds_read_tr4(&sh_x[r0 * LDX + pb * 16 + c0]);
            const bf16x4 hi = lds_read_tr4(&sh_x[(r0 + 16) * LDX + pb * 16 + c0]);
            const bf16x8 afr = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            yia[q] = MM::mma(afr, bfr, yia[q]);
          }
        }
      }
      const float dec_t = exp2_fast(at_t);
#pragma unroll
      for (int q = 0; q < NPP; ++q) {
        const int pb = ph * NPP + q;
        const floatx4 v = yia[q] + dec_t * yin[q];
        if constexpr (Lds::kStageY)
          store4(&sh_y[t * LDY + pb * 16 + 4 * grp], v);
        else
          store4(y_ssd + ((tok0 + t) * H + h) * P + pb * 16 + 4 * grp, v);
      }
      }
    };
    if (has0)
      block_out(tb0, cf0, [&](int jb0, floatx4& t0, floatx4& t1) __attribute__((always_inline)) {
        t0 = gs[jb0];
        t1 = gs[jb0 + 1];
      });
    if (has1)
      block_out(tb1, cf1, [&](int jb0, floatx4& t0, floatx4& t1) __attribute__((always_inline)) {
        t0 = gs[NSLOT - 1 - jb0];
        t1 = gs[NSLOT - 2 - jb0];
      });
    __syncthreads();  // x, H and the factors of head hh are dead; y is complete
    if constexpr (Lds::kStageY) {
#pragma unroll
      for (int v = 0; v < XV; ++v) {
        const int i = tid + v * kOutThreads, t = i / (P / VE), pv = i % (P / VE);
        if (t < S)
          *reinterpret_cast<vec_t*>(y_ssd + ((tok0 + t) * H + h) * P + pv * VE) =
              *reinterpret_cast<const vec_t*>(&sh_y[t * LDY + pv * VE]);
      }
    }
  }
}

// LDS plan of k_chunk_out_dma (chunks of kMaxChunk tokens): the log-decay
// factors of the head being computed (first, so that their addresses fit
// the 16-bit offsets of LDS instructions), then three head slots, each
// holding x [s][p] and H_in[k] [p][n] as XOR-swizzled 16-byte chunks without
// padding (direct global-to-LDS copies fill whole 1 KB runs) and the head's
// raw acum and dt.  Phase 1's padded B rows share the bytes of slots 0 and 1.
template <int N, int P>
struct ChunkOutDma {
  static constexpr int S = kMaxChunk;
  static constexpr int LDC = N + 16;
  static constexpr int XB = S * P * 2, HB = P * N * 2;
  static constexpr int SLOT = XB + HB + 2 * S * 4;
  static constexpr int FAC = 3 * S * 4;  // A_s, v_s, log2 dt_s
  static constexpr size_t bytes = 3ull * SLOT + FAC;
  static constexpr bool fits = P == 64 && N % 64 == 0 && bytes <= 160 * 1024 &&
                               size_t(S) * LDC * 2 <= 2ull * SLOT;
};

// Native chunk output, 16-bit io, S = kMaxChunk and P = 64: the arithmetic
// of k_chunk_out_tr (same tiles, weights and k-slot pairing), with each
// head's x, H_in[k], acum and dt fetched by direct global-to-LDS copies two
// heads ahead into a ring of three slots, so that one workgroup per CU keeps
// two heads of input in flight while it computes a third.  The C operand is
// read from HBM straight into fragments and y leaves from the accumulators.
// Per head: wait for this wave's copies of the head, barrier (every wave's
// copies have landed and every wave is done with the previous head, whose
// slot now receives head + 2), log-decay factors, barrier, compute.
template <int N, int P>
__global__ __launch_bounds__(kOutThreads) void k_chunk_out_dma(
    const bf16* __restrict__ x, const float* __restrict__ dt, const bf16* __restrict__ Bm,
    const bf16* __restrict__ C, const float* __restrict__ acum, const bf16* __restrict__ H_in,
    bf16* __restrict__ y_ssd, int L, int H, int G) {
  using MM = Mma<bf16>;
  using Lds = ChunkOutDma<N, P>;
  typedef bf16x8 vec_t;
  constexpr int S = kMaxChunk;
  constexpr int VE = 8, K = MM::K, KL = MM::KL;
  constexpr int LDC = Lds::LDC;
  constexpr int NKK = N / K, NPB = P / 16;
  constexpr int NSLOT = kMaxBlk + 2;
  constexpr int RV = S * (N / VE) / kOutThreads;     // B vectors per thread (phase 1)
  constexpr int HCH = N / VE;                         // 16-byte chunks per H row
  constexpr int RPH = 64 / HCH;                       // H rows per 1 KB copy
  constexpr int XI = S * P * 2 / 1024 / kOutWaves;    // x copies per wave and head
  constexpr int HI = P * N * 2 / 1024 / kOutWaves;    // H_in copies per wave and head
  constexpr int NDMA = XI + HI + 1;                   // + acum (waves 0-3) or dt (4-7)
  static_assert(Lds::fits && P / VE == 8 && XI >= 1 && HI >= 1 &&
                    XI * kOutWaves * 1024 == S * P * 2 && HI * kOutWaves * 1024 == P * N * 2 &&
                    kOutWaves == 8 && RV * kOutThreads == S * (N / VE),
                "k_chunk_out_dma mapping");
  static_assert(kOutWaves * 2 == kMaxBlk, "two token blocks per wave");
  __shared__ __align__(16) unsigned char sh_raw[Lds::bytes];
  float* sh_at = reinterpret_cast<float*>(sh_raw);  // A_s = acum_s·log2(e)
  float* sh_v = sh_at + S;                           // v_j
  float* sh_ld = sh_v + S;                           // log2 dt_j
  unsigned char* sh_slots = sh_raw + Lds::FAC;
  bf16* sh_b = reinterpret_cast<bf16*>(sh_slots);

  const int k = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int M = L / S, hpg = H / G;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const long tok0 = (long)b * L + (long)k * S;
  const int tb0 = w, tb1 = 2 * kOutWaves - 1 - w;
  const int n0 = 2 * (tb0 / 2 + 1);  // slots of tb0 (pairs of key blocks)

  // head hh lives in slot (hh + 2) % 3: head 0 in slot 2, clear of phase 1.
  // The slot offset is opaque, so that addresses within the slot are formed
  // from it with immediate offsets instead of precomputed per slot.
  auto slot = [&](int hh) __attribute__((always_inline)) {
    int off = ((hh + 2) % 3) * Lds::SLOT;
    asm volatile("" : "+s"(off));
    return sh_slots + off;
  };
  // the lane index, opaque, so that the copy addresses are formed where the
  // copies are issued instead of being held in registers across the loop
  auto lane_now = [&]() __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // x row r keeps its logical 16-byte chunk c at c ^ 2·(r % 4); H_in row r
  // keeps chunk c at c ^ (r % HCH).  Copy I of x is rows 8I .. 8I+7, copy I
  // of H_in rows RPH·I ..; lane l writes the l-th 16 bytes of the copy.
  auto dma_head = [&](int hh) __attribute__((always_inline)) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
    unsigned char* sl = slot(hh);
    bf16* sx = reinterpret_cast<bf16*>(sl);
    bf16* sh = reinterpret_cast<bf16*>(sl + Lds::XB);
    float* sa = reinterpret_cast<float*>(sl + Lds::XB + Lds::HB);
    const int l = lane_now();
#pragma unroll
    for (int q = 0; q < XI; ++q) {
      const int I = w * XI + q, r = 8 * I + l / 8, c = (l % 8) ^ (2 * (r % 4));
      lds_copy16(x + ((tok0 + r) * H + h) * P + c * VE, lds_addr(sx + I * 512));
    }
    const bf16* hsrc = H_in + (pair * M + k) * (long)(P * N);
#pragma unroll
    for (int q = 0; q < HI; ++q) {
      const int I = w * HI + q, r = RPH * I + l / HCH, c = (l % HCH) ^ (r % HCH);
      lds_copy16(hsrc + r * N + c * VE, lds_addr(sh + I * 512));
    }
    if (w < 4)
      lds_copy4(acum + (pair * M + k) * S + w * 64 + l, lds_addr(sa + w * 64));
    else
      lds_copy4(dt + (tok0 + (w - 4) * 64 + l) * H + h, lds_addr(sa + S + (w - 4) * 64));
  };

  dma_head(0);

  // ---- phase 1: B rows -> LDS, C fragments from HBM; C·Bᵀ tiles ----
  typename MM::frag cf0[NKK], cf1[NKK];
  {
    vec_t br[RV];
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const int i = tid + v * kOutThreads, s = i / (N / VE), nv = i % (N / VE);
      br[v] = load16(Bm + ((tok0 + s) * G + g) * N + nv * VE);
    }
    // B operand fragments: column t, k-slots n of C row t
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      cf0[kk] = load16(C + ((tok0 + tb0 * 16 + col) * G + g) * N + kk * K + grp * KL);
      cf1[kk] = load16(C + ((tok0 + tb1 * 16 + col) * G + g) * N + kk * K + grp * KL);
    }
#pragma unroll
    for (int v = 0; v < RV; ++v) {
      const int i = tid + v * kOutThreads, s = i / (N / VE), nv = i % (N / VE);
      *reinterpret_cast<vec_t*>(&sh_b[s * LDC + nv * VE]) = br[v];
    }
  }
  lds_barrier();
  floatx4 gs[NSLOT];
#pragma unroll
  for (int sl = 0; sl < NSLOT; ++sl) {
    gs[sl] = floatx4{0.f, 0.f, 0.f, 0.f};
    const bool is0 = sl < n0;
    const int jb = is0 ? sl : NSLOT - 1 - sl;
    const bool live = is0 ? sl <= tb0 : jb <= tb1;
    if (live) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        gs[sl] = MM::mma(MM::load(&sh_b[(jb * 16 + col) * LDC + kk * K + grp * KL]),
                         is0 ? cf0[kk] : cf1[kk], gs[sl]);
      if (jb == (is0 ? tb0 : tb1)) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) gs[sl][i4] = 4 * grp + i4 <= col ? gs[sl][i4] : 0.f;
      }
    }
  }
  lds_barrier();  // B is dead: slots 0 and 1 are free
  if (hpg > 1) dma_head(1);

  // ---- phase 2: the heads of the group ----
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    // this wave's copies of head hh are done (head hh+1's, if issued, are
    // the only loads after them)
    if (hh + 1 < hpg)
      wait_fence<vmcnt_imm(NDMA)>();
    else
      wait_fence<vmcnt_imm(0)>();
    lds_barrier();  // every wave: head hh landed, head hh-1 done (its slot is free)
    if (hh + 2 < hpg) dma_head(hh + 2);
    const unsigned char* sl = slot(hh);
    const bf16* sx = reinterpret_cast<const bf16*>(sl);
    const bf16* shh = reinterpret_cast<const bf16*>(sl + Lds::XB);
    if (tid < S) {
      const float* sa = reinterpret_cast<const float*>(sl + Lds::XB + Lds::HB);
      const float a2 = sa[tid] * kLog2e;
      // A at the end of this thread's 16-token block, from lane tid|15
      const float e2 = __shfl(a2, lane | 15);
      const float ld = __builtin_amdgcn_logf(sa[S + tid]);
      sh_at[tid] = a2;
      sh_ld[tid] = ld;
      sh_v[tid] = exp2_fast(e2 - a2 + ld);
    }
    lds_barrier();

    auto block_out = [&](int tb, const typename MM::frag (&cf)[NKK], auto pick)
        __attribute__((always_inline)) {
      const int t = tb * 16 + col;
      const float at_t = sh_at[t];
      floatx4 yin[NPB], yia[NPB];
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        yin[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
        yia[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
        const int row = pb * 16 + col;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          yin[pb] = MM::mma(
              MM::load(&shh[row * N + (((kk * K + grp * KL) / VE) ^ (row % HCH)) * VE]), cf[kk],
              yin[pb]);
      }
      // weights of tile jb: as in k_chunk_out_tr
      auto weights = [&](int jb, floatx4 tile) __attribute__((always_inline)) {
        floatx4 wv = floatx4{0.f, 0.f, 0.f, 0.f};
        if (jb < tb) {
          const float u = exp2_fast(at_t - sh_at[jb * 16 + 15]);
          const floatx4 vj = *reinterpret_cast<const floatx4*>(&sh_v[jb * 16 + 4 * grp]);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) wv[i4] = (tile[i4] * u) * vj[i4];
        } else if (jb == tb) {
          const floatx4 aj = *reinterpret_cast<const floatx4*>(&sh_at[jb * 16 + 4 * grp]);
          const floatx4 lj = *reinterpret_cast<const floatx4*>(&sh_ld[jb * 16 + 4 * grp]);
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            wv[i4] = 4 * grp + i4 <= col ? tile[i4] * exp2_fast((at_t - aj[i4]) + lj[i4]) : 0.f;
        }
        return wv;
      };
#pragma unroll
      for (int jb0 = 0; jb0 < kMaxBlk; jb0 += 2) {
        if (jb0 <= tb) {
          floatx4 t0, t1;
          pick(jb0, t0, t1);
          const floatx4 w0 = weights(jb0, t0), w1 = weights(jb0 + 1, t1);
          const bf16x8 bfr = {from_f32<bf16>(w0[0]), from_f32<bf16>(w0[1]),
                              from_f32<bf16>(w0[2]), from_f32<bf16>(w0[3]),
                              from_f32<bf16>(w1[0]), from_f32<bf16>(w1[1]),
                              from_f32<bf16>(w1[2]), from_f32<bf16>(w1[3])};
          // xᵀ operand by transpose reads of the swizzled x rows
          const int r0 = jb0 * 16 + 4 * grp + (col >> 2);
          const int sw = 2 * (r0 % 4);  // r0 + 16 has the same swizzle
#pragma unroll
          for (int pb = 0; pb < NPB; ++pb) {
            const int c = ((2 * pb + ((col & 3) >> 1)) ^ sw) * VE + (col & 1) * 4;
            const bf16x4 lo = lds_read_tr4(&sx[r0 * P + c]);
            const bf16x4 hi = lds_read_tr4(&sx[(r0 + 16) * P + c]);
            const bf16x8 afr = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            yia[pb] = MM::mma(afr, bfr, yia[pb]);
          }
        }
      }
      const float dec_t = exp2_fast(at_t);
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
        store4(y_ssd + ((tok0 + t) * H + h) * P + pb * 16 + 4 * grp, yia[pb] + dec_t * yin[pb]);
    };
    block_out(tb0, cf0, [&](int jb0, floatx4& t0, floatx4& t1) __attribute__((always_inline)) {
      t0 = gs[jb0];
      t1 = gs[jb0 + 1];
    });
    block_out(tb1, cf1, [&](int jb0, floatx4& t0, floatx4& t1) __attribute__((always_inline)) {
      t0 = gs[NSLOT - 1 - jb0];
      t1 = gs[NSLOT - 2 - jb0];
    });
  }
}

}  // namespace

template <typename T, int N, int P>
hipError_t launch_chunk_state(const PrefillShape& s, const T* x, const float* dt, const float* A,
                              const T* Bm, float* acum, T* dH, float* dH_f32, hipStream_t st) {
  const int M = s.L / s.S;
  if constexpr (std::is_same<T, bf16>::value)
    hipLaunchKernelGGL((k_chunk_state_tr<N, P>), dim3(M, s.H, s.B), dim3(kThreads), 0, st, x, dt,
                       A, Bm, acum, dH, dH_f32, s.L, s.H, s.G, s.S);
  else
    hipLaunchKernelGGL((k_chunk_state<T, N, P>), dim3(M, s.H, s.B), dim3(kThreads), 0, st, x, dt,
                       A, Bm, acum, dH, dH_f32, s.L, s.H, s.G, s.S);
  return hipGetLastError();
}

template <typename T, int N, int P>
hipError_t launch_chunk_out(const PrefillShape& s, const T* x, const float* dt, const T* Bm,
                            const T* C, const float* acum, const T* H_in, T* y_ssd,
                            hipStream_t st) {
  const int M = s.L / s.S;
  if constexpr (std::is_same<T, bf16>::value && ChunkOutDma<N, P>::fits) {
    if (s.S == kMaxChunk) {
      hipLaunchKernelGGL((k_chunk_out_dma<N, P>), dim3(M, s.G, s.B), dim3(kOutThreads), 0, st, x,
                         dt, Bm, C, acum, H_in, y_ssd, s.L, s.H, s.G);
      return hipGetLastError();
    }
  }
  if constexpr (std::is_same<T, bf16>::value)
    hipLaunchKernelGGL((k_chunk_out_tr<N, P>), dim3(M, s.G, s.B), dim3(kOutThreads), 0, st, x, dt,
                       Bm, C, acum, H_in, y_ssd, s.L, s.H, s.G, s.S);
  else
    hipLaunchKernelGGL((k_chunk_out<T, N, P>), dim3(M, s.G, s.B), dim3(kOutThreads), 0, st, x, dt,
                       Bm, C, acum, H_in, y_ssd, s.L, s.H, s.G, s.S);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_state_recurrence(const PrefillShape& s, int PN, const float* acum,
                                          const float* dH_f32, const float* h0, T* H_in,
                                          float* h_final, hipStream_t st) {
  const int M = s.L / s.S;
  hipLaunchKernelGGL(k_state_pass<T>, dim3((PN / 4 + kThreads - 1) / kThreads, s.H, s.B),
                     dim3(kThreads), 0, st, acum, dH_f32, h0, H_in, h_final, s.H, M, s.S, PN);
  return hipGetLastError();
}

template <typename T, int N, int P>
hipError_t launch_state_pass(const PrefillShape& s, const T* x, const float* dt, const T* Bm,
                             const T* C, const float* acum, const float* dH_f32,
                             const float* h0, T* H_in, float* h_final, T* y_ssd,
                             hipStream_t st) {
  hipError_t e = launch_state_recurrence<T>(s, P * N, acum, dH_f32, h0, H_in, h_final, st);
  if (e != hipSuccess) return e;
  return launch_chunk_out<T, N, P>(s, x, dt, Bm, C, acum, H_in, y_ssd, st);
}

size_t chunk_scan_workspace_bytes(int io, int64_t B, int64_t L, int64_t H, int64_t N, int64_t P,
                                  int64_t S) {
  const size_t pairs = static_cast<size_t>(B * H), PN = static_cast<size_t>(N * P);
  if (io == DART_F32)  // the f32 memories of the two-kernel path
    return pairs * static_cast<size_t>(L / S) * PN * sizeof(float);
  // failure words, one flag per (batch, head), two ring slots per (batch, head)
  return 256 + ((pairs * 8 + 255) / 256) * 256 + pairs * 2 * PN * sizeof(float);
}

template <typename T, int N, int P>
hipError_t launch_chunk_scan(const PrefillShape& s, const T* x, const float* dt, const float* A,
                             const T* Bm, const float* h0, float* acum, T* dH, float* dH_f32,
                             T* H_in, float* h_final, void* workspace, unsigned tag,
                             hipStream_t st) {
  if constexpr (std::is_same<T, bf16>::value) {
    const int M = s.L / s.S, BH = s.B * s.H;
    char* w = static_cast<char*>(workspace);
    int* err = reinterpret_cast<int*>(w);
    auto* flags = reinterpret_cast<unsigned long long*>(w + 256);
    float* ring = reinterpret_cast<float*>(w + 256 + ((size_t(BH) * 8 + 255) / 256) * 256);
    const int xcd = (s.B * s.G) % 8 == 0 ? 1 : 0;
    // chunks per workgroup: 4, else 2, else 1, as M and the LDS allow
    constexpr size_t lds1 = sizeof(ChunkMemLds<N, P>);
    if constexpr (4 * lds1 <= kLdsBytes) {
      if (M % 4 == 0) {
        hipLaunchKernelGGL((k_chunk_scan<N, P, 4>), dim3(M / 4 * BH), dim3(kThreads * 4), 0, st,
                           x, dt, A, Bm, h0, acum, dH, dH_f32, H_in, h_final, ring, flags, err,
                           tag, s.L, s.H, s.G, s.S, BH, xcd);
        return hipGetLastError();
      }
    }
    if constexpr (2 * lds1 <= kLdsBytes) {
      if (M % 2 == 0) {
        hipLaunchKernelGGL((k_chunk_scan<N, P, 2>), dim3(M / 2 * BH), dim3(kThreads * 2), 0, st,
                           x, dt, A, Bm, h0, acum, dH, dH_f32, H_in, h_final, ring, flags, err,
                           tag, s.L, s.H, s.G, s.S, BH, xcd);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((k_chunk_scan<N, P, 1>), dim3(M * BH), dim3(kThreads), 0, st, x, dt, A,
                       Bm, h0, acum, dH, dH_f32, H_in, h_final, ring, flags, err, tag, s.L, s.H,
                       s.G, s.S, BH, xcd);
    return hipGetLastError();
  } else {
    (void)tag;
    float* f = dH_f32 ? dH_f32 : static_cast<float*>(workspace);
    hipError_t e = launch_chunk_state<T, N, P>(s, x, dt, A, Bm, acum, dH, f, st);
    if (e != hipSuccess) return e;
    return launch_state_recurrence<T>(s, P * N, acum, f, h0, H_in, h_final, st);
  }
}

#define DART_INST_SCAN(T, N, P)                                                              \
  template hipError_t launch_chunk_state<T, N, P>(const PrefillShape&, const T*, const float*, \
                                                  const float*, const T*, float*, T*, float*,  \
                                                  hipStream_t);                                \
  template hipError_t launch_state_pass<T, N, P>(const PrefillShape&, const T*, const float*,  \
                                                 const T*, const T*, const float*,             \
                                                 const float*, const float*, T*, float*, T*,   \
                                                 hipStream_t);                                 \
  template hipError_t launch_chunk_out<T, N, P>(const PrefillShape&, const T*, const float*,   \
                                                const T*, const T*, const float*, const T*, T*, \
                                                hipStream_t);                                  \
  template hipError_t launch_chunk_scan<T, N, P>(const PrefillShape&, const T*, const float*,  \
                                                 const float*, const T*, const float*, float*, \
                                                 T*, float*, T*, float*, void*, unsigned,      \
                                                 hipStream_t);
DART_FOR_EACH_SHAPE(DART_INST_SCAN)

}  // namespace dart
