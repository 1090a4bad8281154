// State-memory attention (SMA) on gfx950, prefill over all tokens (the
// single-token decode step is in k_decode.hip).
//
// Definitions (Pith review of DART, "Core claim" and "What carries the
// argument"; referee major comment 3, paper §3 Eq. 8; DART abstract): for a
// token t of chunk k and each completed chunk c < k
//   key    dH[c]·E_t (value axis contracted)   value  C_tᵀ·dH[c]
//   score  Q_tᵀ·dH[c]·E_t / sqrt(N)            o_t = Σ_c softmax_c(score)·value
// and y_t = y_ssd_t + gate·o_t (o_t = 0 for chunk 0).
//
// Evaluation order used here: with Zq = dH[c]ᵀQ_t and Zc = dH[c]ᵀC_t (both in
// R^P) the score is E_t·Zq / sqrt(N) and the value is Zc, so each memory is
// one product with the stacked [Q; C] operand.  The same quantities, summed
// in a different association order.
#include "dart_launch.hpp"
#include "dart_shapes.hpp"

namespace dart {
namespace {

// tokens per wave = 16·NTB; the largest shape keeps one 16-token block per
// wave to stay inside the register file
template <int N, int P>
struct SmaTile {
  static constexpr int NTB = (N * P >= 128 * 128) ? 1 : 2;
};

// (batch, head) pairs per ordering group of one XCD (see k_sma_fwd)
constexpr int kPairsPerGroup = 4;


template <int V>
using IC = std::integral_constant<int, V>;


// Per-wave tile arithmetic of the prefill kernel: a wave owns TW = 16·NTB
// tokens of the workgroup's tile.  Each policy holds the wave's resident
// [Q; C] operand fragments, its E values, the products Zq = dH[c]ᵀQ and
// Zc = dH[c]ᵀC of the current memory and the online-softmax state, with
// every register index a compile-time constant.
//
// SmaMath16: 16x16 MFMA tiles (rows p, columns tokens, K = 32 along n for
// 16-bit io, K = 4 for fp32); NTB 16-token blocks per wave.
template <typename T, int N, int P, int NTB>
struct SmaMath16 {
  using MM = Mma<T>;
  static constexpr int K = MM::K, KL = MM::KL;
  static constexpr int NPB = P / 16, NKK = N / K, TW = 16 * NTB;
  typedef typename std::conditional<std::is_same<T, bf16>::value, bf16x4, floatx4>::type e4_t;
  typename MM::frag qf[NTB][NKK], cf[NTB][NKK];
  e4_t ev[NTB][NPB];
  floatx4 zq[NTB][NPB], zc[NTB][NPB], acc[NTB][NPB];
  float mx[NTB], ls[NTB];
  float at[NTB];       // decayed variant: log-decay from the chunk start to the token
  int row0, col, grp;  // first token row of the wave; lane coordinates

  __device__ __forceinline__ void init(int w, int lane) {
    row0 = w * TW;
    col = lane & 15;
    grp = lane >> 4;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      mx[tb] = -INFINITY;
      ls[tb] = 0.f;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) acc[tb][pb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
  __device__ __forceinline__ int lrow(int tb) const { return row0 + tb * 16 + col; }
  // B operand fragments (column t, k-slots along n) from token rows [t][n]
  __device__ __forceinline__ void load_frags(typename MM::frag (&f)[NTB][NKK], const T* tile,
                                             int ld) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) f[tb][kk] = MM::load(&tile[lrow(tb) * ld + kk * K + grp * KL]);
  }
  __device__ __forceinline__ void load_q(const T* tile, int ld) { load_frags(qf, tile, ld); }
  __device__ __forceinline__ void load_c(const T* tile, int ld) { load_frags(cf, tile, ld); }
  // this lane's p rows of E (kept in the input type, widened in the score)
  __device__ __forceinline__ void load_e(const T* tile, int ld) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
        ev[tb][pb] = *reinterpret_cast<const e4_t*>(&tile[lrow(tb) * ld + pb * 16 + 4 * grp]);
  }
  // Zq, Zc of one memory held as rows [p][n] in LDS
  __device__ __forceinline__ void mma(const T* mem, int ld) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        zq[tb][pb] = floatx4{0.f, 0.f, 0.f, 0.f};
        zc[tb][pb] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    // A fragments of p-block pb+1 are read while the MFMAs of pb run
    typename MM::frag a[2][NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) a[0][kk] = MM::load(&mem[col * ld + kk * K + grp * KL]);
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      if (pb + 1 < NPB) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          a[(pb + 1) & 1][kk] = MM::load(&mem[((pb + 1) * 16 + col) * ld + kk * K + grp * KL]);
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          zq[tb][pb] = MM::mma(a[pb & 1][kk], qf[tb][kk], zq[tb][pb]);
          zc[tb][pb] = MM::mma(a[pb & 1][kk], cf[tb][kk], zc[tb][pb]);
        }
    }
    // schedule: LDS fragment reads run four fragments ahead of the MFMAs
    // that consume them (2·NTB MFMAs per fragment cover the LDS latency)
    constexpr int R = NPB * NKK;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int f = 0; f < R; ++f) {
      if (f + 4 < R) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NTB, 0);
    }
  }
  // DECAY: key and value of the memory are scaled by d = exp(at + dlog),
  // the SSM decay from the memory's chunk end to the token (dlog: the
  // log-decay over the chunks between that end and the token's chunk)
  template <bool DECAY = false>
  __device__ __forceinline__ void softmax(float scale_log2, float dlog = 0.f) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      float s = 0.f;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s += zq[tb][pb][i] * to_f32(ev[tb][pb][i]);
      s = sum_lane_groups(s) * scale_log2;
      const float d = DECAY ? exp2_fast((at[tb] + dlog) * kLog2e) : 1.f;
      if (DECAY) s *= d;
      // The reference max mx is raised only when a score passes it by more
      // than kLazyLog2 (a wave-uniform branch, taken at the first memory and
      // rarely after); otherwise the weights 2^(s - mx) stay below
      // 2^kLazyLog2 and the running sums need no rescale.
      if (__any(s > mx[tb] + kLazyLog2)) {
        const float mn = fmaxf(mx[tb], s);
        const float al = exp2_fast(mx[tb] - mn);  // 0 for the first memory
        ls[tb] *= al;
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) acc[tb][pb] *= al;
        mx[tb] = mn;
      }
      const float pw = exp2_fast(s - mx[tb]);
      ls[tb] += pw;
      const float pv = DECAY ? pw * d : pw;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) acc[tb][pb] += pv * zc[tb][pb];
    }
  }
  // Training statistics of the tile's tokens: the readout o_t (before the
  // gate) to o rows [t][stride] and the softmax log-normaliser in the
  // kernel's base-2 score units, lse_t = mx + log2(ls), to lse[t]; both 0
  // for tokens that see no memory.
  __device__ __forceinline__ void stats(float* o, long ostride, float* lse, bool any) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const float inv = any ? 1.f / ls[tb] : 0.f;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
        *reinterpret_cast<floatx4*>(o + lrow(tb) * ostride + pb * 16 + 4 * grp) =
            inv * acc[tb][pb];
      if (grp == 0) lse[lrow(tb)] = any ? mx[tb] + __builtin_amdgcn_logf(ls[tb]) : 0.f;
    }
  }
  // y = y_ssd + gate·o in the LDS rows [t][p] that hold y_ssd
  __device__ __forceinline__ void finish(T* ty, int ld, float gate, bool any) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const float f = any ? gate / ls[tb] : 0.f;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        T* q = &ty[lrow(tb) * ld + pb * 16 + 4 * grp];
        store4(q, load4_f32(q) + f * acc[tb][pb]);
      }
    }
  }
};


// Prefill SMA.  One workgroup = WAVES waves × 16·NTB tokens of ONE chunk k,
// so every token of the workgroup sees the same memories c < k (no mask).
// Per memory c, dH[c]ᵀ (P x N, value-axis-major in HBM) is staged in LDS
// (two buffers; each memory is fetched into registers one step before it is
// written to LDS).  Each wave multiplies it with its resident [Q; C]
// fragments (16x16 MFMA, rows p, columns = tokens), finishes the score with
// an in-lane dot against E_t plus two lane-group exchanges, and folds the
// value into an online softmax.  The waves are split in two halves that
// alternate between the MFMA phase and the softmax phase (see half_steps),
// so matrix core and vector ALU work of one SIMD overlap.
//
// Grid mapping: workgroups are dealt to the 8 XCDs round-robin, so
// blockIdx % 8 selects an XCD and all tiles of one (batch, head) pair land
// on the same XCD.  When heads share B/C/Q groups (and the batch·group count
// fills the 8 XCDs evenly) the heads of one (batch, group) go to the same
// XCD and are ordered next to each other, so the Q_t/C_t tiles they share
// are read from HBM once per XCD rather than once per head.  Inside an XCD
// the pairs are taken kPairsPerGroup at a time, heaviest tiles (largest k)
// first within each group: the memories of a group (4 x 512 KB at the
// largest shape) stay resident in the XCD's 4 MB L2 while the k-ordering
// keeps the tail short.
//
// DECAY (the decay-included variant): key and value of memory c are scaled
// for token t by the SSM decay from the end of chunk c to t, d_{t,c} =
// exp(acum_k[t] + Σ_{c<c'<k} acum_end[c']).  The memories are then taken
// newest first, so the chunk sum is a running sum of non-positive terms
// (no cancellation); the softmax does not depend on the order.
//
// Continuation (k0 > 0): the L tokens are chunks k0 .. k0+M-1 of their
// sequences; memories c < k0 come from `prior` (one row of `pstride`
// memories per (batch, head), the decode cache layout), memories c >= k0
// from dH (chunk c - k0).
//
// PRIOR8 (continuation from an fp8 cache): the prior memories are E4M3 codes
// (prior8, one power-of-two scale each in pscale); each is decoded while it
// is staged into LDS (code·scale is exact in bfloat16), so the rest of the
// kernel is unchanged and the loads stay one step ahead.
template <typename T, int N, int P, int NTB, int WAVES, bool DECAY, bool PRIOR8 = false>
__global__ __launch_bounds__(64 * WAVES) void k_sma_fwd(
    const T* __restrict__ Q, const T* __restrict__ E, const T* __restrict__ C,
    const T* __restrict__ dH, const T* __restrict__ y_ssd, const float* __restrict__ acum,
    float gate, T* __restrict__ y, int BH, int L, int H, int G, int S, int npq, int bg_major,
    float scale_log2, const T* __restrict__ prior, int k0, int pstride,
    float* __restrict__ o_out, float* __restrict__ lse_out, const uint8_t* __restrict__ prior8,
    const float* __restrict__ pscale) {
  using MM = Mma<T>;
  constexpr int K = MM::K, KL = MM::KL, VE = Vec16<T>::n;
  // LDS row strides (elements): a 32-byte pad keeps the 16-byte fragment reads
  // (16 rows x 4 column groups per instruction) free of bank conflicts on the
  // 64-bank LDS; a 16-byte pad leaves them 2-way conflicted
  constexpr int LDN = N + 2 * VE;  // memory rows [p][n], Q/C rows [t][n]
  constexpr int LDE = P + 2 * VE;  // E and y rows [t][p]
  constexpr int TW = 16 * NTB, TWG = TW * WAVES;
  constexpr int NVEC = P * N / VE;  // 16-byte vectors per memory
  constexpr int NTHR = 64 * WAVES;
  constexpr int VPT = (NVEC + NTHR - 1) / NTHR;
  constexpr int NPB = P / 16, NKK = N / K;
  constexpr int GP = kPairsPerGroup;
  // token-row tiles move between HBM and LDS as whole rows (a wave's 16-byte
  // vectors cover complete cache lines; fragment-shaped global accesses cost
  // about four times as much issue time per instruction)
  constexpr int QV = TWG * (N / VE) / NTHR;  // vectors per thread, Q or C tile
  constexpr int EV = TWG * (P / VE) / NTHR;  // vectors per thread, E or y tile
  static_assert(QV * NTHR == TWG * (N / VE) && EV * NTHR == TWG * (P / VE), "tile split");
  constexpr int R1A = TWG * LDN + TWG * LDE;
  constexpr int R1 = R1A > 2 * P * LDN ? R1A : 2 * P * LDN;
  typedef typename Vec16<T>::vec vec_t;
  // sh_r1: the Q and E tiles side by side, then the C tile, during the
  // prologue, then the two memory buffers; sh_ty: y_ssd, overwritten by y in
  // the epilogue
  __shared__ __align__(16) T sh_r1[R1];
  __shared__ __align__(16) T sh_ty[TWG * LDE];
  T(*sh_mem)[P * LDN] = reinterpret_cast<T(*)[P * LDN]>(sh_r1);

  const int M = L / S, tpc = S / TWG;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_group = GP * M * tpc;
  const int grp_i = slot / per_group, rem = slot % per_group;
  const int sub = rem % tpc, r = rem / tpc;
  const int qg = r % GP, kr = r / GP;
  const int ql = grp_i * GP + qg;
  const int kl = M - 1 - kr;  // the tile's chunk among the L tokens
  const int k = k0 + kl;      // memories it attends
  // bg_major: the heads of one (batch, group) run on one XCD, adjacent in
  // the ordering, so their shared Q_t/C_t tiles are reused from L2
  int pair;
  if (bg_major) {
    const int hpg = H / G;
    const int bg = (ql / hpg) * 8 + xcd;
    pair = (bg / G) * H + (bg % G) * hpg + ql % hpg;
    if (bg >= BH / hpg || ql >= npq) return;
  } else {
    pair = ql * 8 + xcd;
    if (pair >= BH || ql >= npq) return;  // uniform over the workgroup
  }
  const int b = pair / H, h = pair % H, g = h / (H / G);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const long row0 = (long)b * L + (long)kl * S + sub * TWG;  // first token of the tile

  if (k == 0) {  // no memory is visible: y = y_ssd, o = 0, lse = 0
#pragma unroll
    for (int v = 0; v < EV; ++v) {
      const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
      *reinterpret_cast<vec_t*>(y + ((row0 + t) * H + h) * P + pv * VE) =
          load16(y_ssd + ((row0 + t) * H + h) * P + pv * VE);
    }
    if (o_out) {
      for (int i = tid; i < TWG * (P / 4); i += NTHR) {
        const int t = i / (P / 4), p4 = i % (P / 4);
        *reinterpret_cast<floatx4*>(o_out + ((row0 + t) * H + h) * P + 4 * p4) =
            floatx4{0.f, 0.f, 0.f, 0.f};
      }
      for (int t = tid; t < TWG; t += NTHR)
        lse_out[(long)pair * L + (long)kl * S + sub * TWG + t] = 0.f;
    }
    return;
  }
  // ---- prologue: every load in flight before the first wait, in the
  // order they are staged ----
  vec_t qs[QV], cs[QV], es[EV], ys[EV];
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int i = tid + v * NTHR, t = i / (N / VE), nv = i % (N / VE);
    qs[v] = load16(Q + ((row0 + t) * G + g) * N + nv * VE);
  }
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    es[v] = load16(E + ((row0 + t) * H + h) * P + pv * VE);
  }
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int i = tid + v * NTHR, t = i / (N / VE), nv = i % (N / VE);
    cs[v] = load16(C + ((row0 + t) * G + g) * N + nv * VE);
  }
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    ys[v] = load16(y_ssd + ((row0 + t) * H + h) * P + pv * VE);
  }
  const T* mem = dH + (long)pair * M * (P * N);
  const T* pmem = k0 > 0 ? prior + (long)pair * pstride * (P * N) : nullptr;
  // loop step i multiplies memory mi(i): oldest first, or newest first with DECAY
  auto mi = [&](int i) __attribute__((always_inline)) { return DECAY ? k - 1 - i : i; };
  // a staged memory: 16-byte vectors of the io type, or (PRIOR8) the codes
  // of a prior memory with its scale (scale 0 marks an io-type memory)
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  struct Staged {
    vec_t v[VPT];
    u32x2 raw[PRIOR8 ? VPT : 1];
    float sc;
  };
  const uint8_t* pmem8 = PRIOR8 && k0 > 0 ? prior8 + (long)pair * pstride * (P * N) : nullptr;
  const float* psc = PRIOR8 && k0 > 0 ? pscale + (long)pair * pstride : nullptr;
  Staged stg0, stg;
  auto gload = [&](int i, Staged& dst) __attribute__((always_inline)) {
    const int c = mi(i);
    if constexpr (PRIOR8) {
      dst.sc = 0.f;
      if (c < k0) {  // uniform over the workgroup
        const u32x2* s8 = reinterpret_cast<const u32x2*>(pmem8 + (long)c * (P * N));
#pragma unroll
        for (int v = 0; v < VPT; ++v) {
          const int vi = tid + v * NTHR;
          if (NVEC % NTHR == 0 || vi < NVEC) dst.raw[v] = s8[vi];
        }
        dst.sc = psc[c];
        return;
      }
    }
    const vec_t* src = reinterpret_cast<const vec_t*>(
        c < k0 ? pmem + (long)c * (P * N) : mem + (long)(c - k0) * (P * N));
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int vi = tid + v * NTHR;
      if (NVEC % NTHR == 0 || vi < NVEC) dst.v[v] = src[vi];
    }
  };
  auto swrite = [&](int buf, const Staged& src) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int vi = tid + v * NTHR;
      if (NVEC % NTHR == 0 || vi < NVEC) {
        const int p = vi / (N / VE), nv = vi % (N / VE);
        vec_t val = src.v[v];
        if constexpr (PRIOR8) {
          if (src.sc != 0.f) {  // an E4M3 prior memory: decode and scale (exact)
            typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
              const b2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src.raw[v][wd], 1.0f, false);
              const b2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(src.raw[v][wd], 1.0f, true);
              val[4 * wd + 0] = from_f32<T>(to_f32(lo[0]) * src.sc);
              val[4 * wd + 1] = from_f32<T>(to_f32(lo[1]) * src.sc);
              val[4 * wd + 2] = from_f32<T>(to_f32(hi[0]) * src.sc);
              val[4 * wd + 3] = from_f32<T>(to_f32(hi[1]) * src.sc);
            }
          }
        }
        *reinterpret_cast<vec_t*>(&sh_mem[buf][p * LDN + nv * VE]) = val;
      }
    }
  };
  if (k > 0) {
    gload(0, stg0);
    gload(min(1, k - 1), stg);
  }
  // Q tile -> fragments; E tile -> this lane's p rows, kept in the input
  // type (bf16 pairs halve the registers) and widened when the score is
  // formed
  T* sh_e = sh_r1 + TWG * LDN;
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int i = tid + v * NTHR, t = i / (N / VE), nv = i % (N / VE);
    *reinterpret_cast<vec_t*>(&sh_r1[t * LDN + nv * VE]) = qs[v];
  }
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    *reinterpret_cast<vec_t*>(&sh_e[t * LDE + pv * VE]) = es[v];
  }
  __syncthreads();
  SmaMath16<T, N, P, NTB> tm;
  tm.init(w, lane);
  tm.load_q(sh_r1, LDN);
  tm.load_e(sh_e, LDE);
  const float* acum_pair = DECAY ? acum + (long)pair * M * S : nullptr;
  if (DECAY) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) tm.at[tb] = acum_pair[(long)kl * S + sub * TWG + tm.lrow(tb)];
  }
  __syncthreads();
  // C tile -> fragments; y_ssd parked for the epilogue
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int i = tid + v * NTHR, t = i / (N / VE), nv = i % (N / VE);
    *reinterpret_cast<vec_t*>(&sh_r1[t * LDN + nv * VE]) = cs[v];
  }
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    *reinterpret_cast<vec_t*>(&sh_ty[t * LDE + pv * VE]) = ys[v];
  }
  __syncthreads();
  tm.load_c(sh_r1, LDN);
  __syncthreads();  // sh_r1 becomes the memory buffers

  // DECAY: dlog is the log-decay over the chunks after the memory being
  // finished (a running sum over memories taken newest first); each wave
  // reads the next chunk-end value during its MFMA half
  float dlog = 0.f, ae = 0.f;
  auto mma_mem = [&](int cur, int c) __attribute__((always_inline)) {
    if (DECAY) ae = acum_pair[(long)mi(c) * S + (S - 1)];
    tm.mma(sh_mem[cur], LDN);
  };
  auto softmax_mem = [&]() __attribute__((always_inline)) {
    tm.template softmax<DECAY>(scale_log2, dlog);
    if (DECAY) dlog += ae;
  };
  // Ping-pong: the first half of the waves (one per SIMD) runs its MFMAs
  // while the second half runs its softmax, then they swap, so the matrix
  // core and the vector ALU of every SIMD stay busy together.  Two barriers
  // per memory; memory c sits in buffer c&1 during both halves of step c and
  // memory c+1 is written into the other buffer in the second half (its
  // previous content, memory c-1, was last read a full barrier earlier).
  const bool lead = w < WAVES / 2;
  auto half_steps = [&](int c, auto par_tag) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    // Each wave stages its share of memory c+1 (fetched during step c-1)
    // into the other buffer in its softmax half, off the MFMA path: that
    // buffer last held memory c-1, whose final reads ended at the previous
    // barrier.  Unconditional, indices clamped to the last memory: a
    // duplicate lands in a buffer that is not read again, and every path
    // issues the same loads (so the wait before the LDS write covers only
    // the older fetch).
    auto stage_next = [&]() __attribute__((always_inline)) {
      swrite(PAR ^ 1, stg);           // memory c+1
      gload(min(c + 2, k - 1), stg);  // memory c+2
    };
    // first half: lead waves multiply memory c, the others finish memory c-1
    if (lead) {
      if (c < k) mma_mem(PAR, c);
    } else {
      if (c > 0) softmax_mem();
      stage_next();
    }
    __syncthreads();
    // second half: lead waves finish memory c, the others multiply it
    if (lead) {
      if (c < k) softmax_mem();
      stage_next();
    } else if (c < k) {
      mma_mem(PAR, c);
    }
    __syncthreads();
  };
  if (k > 0) {
    swrite(0, stg0);
    // memory 1 has arrived too, so the loop's only load in flight is the
    // memory prefetch
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    for (int c = 0; c <= k; c += 2) {
      half_steps(c, IC<0>{});
      if (c + 1 <= k) half_steps(c + 1, IC<1>{});
    }
  }

  // ---- epilogue: y = y_ssd + gate·o in LDS, then whole-row stores ----
  if (o_out)
    tm.stats(o_out + (row0 * H + h) * P, (long)H * P,
             lse_out + (long)pair * L + (long)kl * S + sub * TWG, k > 0);
  tm.finish(sh_ty, LDE, gate, k > 0);
  __syncthreads();
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    *reinterpret_cast<vec_t*>(y + ((row0 + t) * H + h) * P + pv * VE) =
        *reinterpret_cast<const vec_t*>(&sh_ty[t * LDE + pv * VE]);
  }
}

// LDS of k_sma_grp: two padded memory buffers, and per wave one E region
// and one y_ssd region of its tokens
template <int N, int P, int NTB, int WAVES>
constexpr size_t sma_grp_lds_bytes() {
  return (2ull * P * (N + 16) + 2ull * WAVES * 16 * NTB * P) * 2;
}

// Prefill SMA over the heads of one B/C/Q group.  One workgroup = WAVES
// waves x 16·NTB tokens of ONE chunk k of one (batch, group); it runs the
// heads of the group one after the other with k_sma_fwd's arithmetic and
// ping-pong schedule (SmaMath16).  Q_t and C_t are shared by those heads,
// so their fragments are loaded once, straight from HBM into the MFMA
// B-operand registers, and stay resident for all of them; each head brings
// only its E and y_ssd rows and its k memories.
//
// The memories of all heads form one sequence of hpg·k steps (head-major)
// that the staging pipeline runs through without a break (buffer parity
// follows the flat step index).  Each wave finishes a head for its own
// tokens once the softmax of its last memory is done: y = y_ssd + gate·o
// through its private y_ssd rows in LDS, whole-row stores, then the next
// head's E values and a fresh softmax state.  All waves do so in the first
// half of the next head's first step (the lead waves behind that step's
// products), so the finishes of the two halves overlap; that step is
// peeled out of the inner loops, which match k_sma_fwd's.  E and y_ssd rows of a wave's tokens reach its private LDS
// regions by direct global-to-LDS loads one head ahead, so neither barriers
// nor staging registers are involved and a head change costs no HBM round
// trip.
//
// Grid mapping: blockIdx % 8 selects the XCD; an XCD takes every 8th (batch,
// group), one after the other, each one's chunks heaviest first: its
// running workgroups share one group's memories in L2, and a CU that drew
// chunk k draws about M - 1 - k next.
template <int N, int P, int NTB, int WAVES, bool STATS>
__global__ __launch_bounds__(64 * WAVES) void k_sma_grp(
    const bf16* __restrict__ Q, const bf16* __restrict__ E, const bf16* __restrict__ C,
    const bf16* __restrict__ dH, const bf16* __restrict__ y_ssd, float gate,
    bf16* __restrict__ y, int L, int H, int G, int S, int BG, int nbx, float scale_log2,
    float* __restrict__ o_out, float* __restrict__ lse_out) {
  typedef bf16 T;
  typedef bf16x8 vec_t;
  using TM = SmaMath16<T, N, P, NTB>;
  constexpr int VE = 8;
  constexpr int LDN = N + 2 * VE;  // memory rows [p][n] (see k_sma_fwd)
  constexpr int TW = 16 * NTB, TWG = TW * WAVES;
  constexpr int NVEC = P * N / VE;  // 16-byte vectors per memory
  constexpr int NTHR = 64 * WAVES;
  constexpr int VPT = (NVEC + NTHR - 1) / NTHR;
  // a wave's E / y_ssd rows: RV 16-byte vectors per row, RPI rows per
  // 64-lane direct load, NI loads per region.  Inside a row, vector v sits
  // in slot v ^ (row % SW): the lanes' 8-byte accesses at one p-offset of
  // 16 consecutive rows then fall into distinct banks (2-way at most)
  constexpr int RV = P / VE, RPI = 64 / RV, NI = TW / RPI, SW = RV < 8 ? RV : 8;
  constexpr int NPB = P / 16;
  static_assert(64 % RV == 0 && TW % RPI == 0, "k_sma_grp row split");
  static_assert(WAVES >= 2 && WAVES % 2 == 0, "k_sma_grp ping-pong halves");
  __shared__ __align__(16) T sh_mem[2 * P * LDN];
  __shared__ __align__(16) T sh_e[WAVES][TW * P];  // E rows of the next head to load
  __shared__ __align__(16) T sh_y[WAVES][TW * P];  // y_ssd rows of the current head
  static_assert(sizeof(sh_mem) + sizeof(sh_e) + sizeof(sh_y) ==
                    sma_grp_lds_bytes<N, P, NTB, WAVES>(), "k_sma_grp LDS plan");

  const int M = L / S, tpc = S / TWG, hpg = H / G;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per_bg = M * tpc;
  const int jb = slot / per_bg, rem = slot % per_bg;
  const int kr = rem / tpc, sub = rem % tpc;
  const int bg = jb * 8 + xcd;
  if (bg >= BG || jb >= nbx) return;  // uniform over the workgroup
  const int k = M - 1 - kr;
  const int b = bg / G, g = bg % G, h0 = g * hpg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long row0 = (long)b * L + (long)k * S + sub * TWG;  // first token of the tile
  const long wrow0 = row0 + w * TW;                         // first token of this wave
  const long HP = (long)H * P;

  if (k == 0) {  // no memory is visible: y = y_ssd for every head, o = 0, lse = 0
    const int rowv = hpg * RV;  // the group's heads are adjacent in a token row
    for (int i = tid; i < TWG * rowv; i += NTHR) {
      const int t = i / rowv, v = i % rowv;
      const long o = (row0 + t) * HP + (long)h0 * P + v * VE;
      *reinterpret_cast<vec_t*>(y + o) = load16(y_ssd + o);
    }
    if constexpr (STATS) {
      for (int i = tid; i < TWG * hpg * (P / 4); i += NTHR) {
        const int t = i / (hpg * (P / 4)), q = i % (hpg * (P / 4));
        *reinterpret_cast<floatx4*>(o_out + (row0 + t) * HP + (long)h0 * P + 4 * q) =
            floatx4{0.f, 0.f, 0.f, 0.f};
      }
      for (int i = tid; i < TWG * hpg; i += NTHR) {
        const int hh = i / TWG, t = i % TWG;
        lse_out[((long)b * H + h0 + hh) * L + (long)k * S + sub * TWG + t] = 0.f;
      }
    }
    return;
  }

  // the lane index, opaque: the swizzled LDS offsets derived from it are
  // computed where they are used (once per head) instead of being kept
  // in registers across the loops
  auto lane_now = [&]() __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  // direct global -> LDS copy of this wave's TW token rows of head hh into
  // its swizzled [t][p] region: lane l of load q fills slot l % RV of row
  // q·RPI + l / RV, i.e. vector (l % RV) ^ (row % SW) of that token row.
  // The lane's element offset is made opaque so that its address arithmetic
  // stays here instead of occupying registers across the loops.
  auto dma_rows = [&](const T* src, T* region, int hh) __attribute__((always_inline)) {
    const int l = lane_now(), r = l / RV;
    const int off = r * (int)HP + ((l % RV) ^ (r % SW)) * VE;
    const T* base = src + wrow0 * HP + (long)(h0 + hh) * P;
#pragma unroll
    for (int q = 0; q < NI; ++q)
      __builtin_amdgcn_global_load_lds(
          base + (long)q * RPI * HP + off,
          (__attribute__((address_space(3))) void*)(region + q * RPI * P), 16, 0, 0);
  };
  // element (row, p) of a swizzled region
  auto swz = [&](int row, int p) __attribute__((always_inline)) {
    return row * P + (((p / VE) ^ (row % SW)) * VE) + p % VE;
  };

  const int nsteps = hpg * k;
  // the memories are fetched in flat order (head-major): gh, gc are the
  // head and chunk of the next one; after the last, the last is fetched
  // again (a duplicate nobody reads)
  int gh = 0, gc = 0;
  vec_t stg0[VPT], stg[VPT];
  auto gload_next = [&](vec_t (&dst)[VPT]) __attribute__((always_inline)) {
    const T* m = dH + ((long)(b * H + h0 + gh) * M + gc) * (P * N);
    if (++gc == k) {
      gc = 0;
      if (gh + 1 < hpg) ++gh; else gc = k - 1;
    }
    const vec_t* src = reinterpret_cast<const vec_t*>(m);
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int vi = tid + v * NTHR;
      if (NVEC % NTHR == 0 || vi < NVEC) dst[v] = src[vi];
    }
  };
  auto swrite = [&](int buf, const vec_t (&src)[VPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int vi = tid + v * NTHR;
      if (NVEC % NTHR == 0 || vi < NVEC) {
        const int p = vi / (N / VE), nv = vi % (N / VE);
        *reinterpret_cast<vec_t*>(&sh_mem[buf * (P * LDN) + p * LDN + nv * VE]) = src[v];
      }
    }
  };

  TM tm;
  tm.init(w, lane);
  // this lane's E values (p = pb·16 + 4·grp .. +3 of its token rows)
  auto load_e = [&]() __attribute__((always_inline)) {
    const int l = lane_now(), col = l & 15, grp = l >> 4;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
        tm.ev[tb][pb] =
            *reinterpret_cast<const bf16x4*>(&sh_e[w][swz(tb * 16 + col, pb * 16 + 4 * grp)]);
  };
  // ---- prologue: E and y_ssd rows of the first head, the Q/C fragments
  // (resident for every head), the first two memories ----
  dma_rows(E, sh_e[w], 0);
  tm.load_q(Q + (row0 * G + g) * N, G * N);
  tm.load_c(C + (row0 * G + g) * N, G * N);
  dma_rows(y_ssd, sh_y[w], 0);
  gload_next(stg0);
  gload_next(stg);
  wait_fence<vmcnt_imm(0)>();
  load_e();
  swrite(0, stg0);
  wait_fence<kLgkm0>();  // the E reads are done before the region is refilled
  if (hpg > 1) dma_rows(E, sh_e[w], 1);
  __syncthreads();

  // Head hh is complete (the softmax of its last memory is done): y rows of
  // head hh for this wave's tokens, then the softmax state of head hh + 1.
  // Both halves of the waves run it in the first half of head hh + 1's
  // first step (the lead waves behind that step's products, the others
  // behind the softmax of head hh's last memory), so the two overlap
  // instead of each holding up the other at a barrier.  The direct loads
  // of head hh's y_ssd
  // and head hh + 1's E were issued at the previous head change; inside the
  // loops at least one memory fetch was issued after them, and only the
  // newest fetch may stay in flight.  After the loops (`last`) no fetch may
  // follow them (one memory per head), so everything is waited for.
  auto finish_head = [&](int hh, auto last) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);  // not interleaved with the products
    if constexpr (decltype(last)::value)
      wait_fence<vmcnt_imm(0)>();
    else
      wait_fence<vmcnt_imm(VPT)>();
    const int h = h0 + hh;
    if constexpr (STATS)
      tm.stats(o_out + (row0 * H + h) * P, HP,
               lse_out + ((long)b * H + h) * L + (long)k * S + sub * TWG, true);
    // y = y_ssd + gate·o in the lane's own places of the y_ssd rows
    const int l = lane_now(), col = l & 15, grp = l >> 4;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      const float f = gate / tm.ls[tb];
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        T* q = &sh_y[w][swz(tb * 16 + col, pb * 16 + 4 * grp)];
        store4(q, load4_f32(q) + f * tm.acc[tb][pb]);
      }
    }
    {
      // whole rows out (the slot a lane reads holds vector (l % RV) ^ (row % SW))
      const int r = l / RV;
      const int off = r * (int)HP + ((l % RV) ^ (r % SW)) * VE;
      T* dst = y + wrow0 * HP + (long)h * P;
#pragma unroll
      for (int q = 0; q < NI; ++q)
        *reinterpret_cast<vec_t*>(dst + (long)q * RPI * HP + off) =
            *reinterpret_cast<const vec_t*>(&sh_y[w][(q * RPI + r) * P + (l % RV) * VE]);
    }
    // the next head's E (after the last head: stale values, never used) and
    // a fresh softmax state: with the reference max at -inf the next
    // memory's rescale factor is 0, which clears ls and acc on its own
    load_e();
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) tm.mx[tb] = -INFINITY;
    wait_fence<kLgkm0>();  // this wave's y_ssd and E reads are done
    if (hh + 1 < hpg) dma_rows(y_ssd, sh_y[w], hh + 1);
    if (hh + 2 < hpg) dma_rows(E, sh_e[w], hh + 2);
  };

  // ping-pong (k_sma_fwd's schedule) over the flat steps i = 0 .. nsteps:
  // memory i sits in buffer i&1 during both halves of step i; each wave
  // stages its share of memory i+1 into the other buffer in its softmax
  // half and fetches memory i+2.  Lead waves multiply memory i in the
  // first half and fold it into the softmax in the second; the others fold
  // in memory i-1 in the first half and multiply memory i in the second.
  // The first step of each head is peeled: it carries the previous head's
  // finish in its MFMA half.
  auto stage_next = [&](int i) __attribute__((always_inline)) {
    swrite((i + 1) & 1, stg);
    gload_next(stg);
  };
  auto mma = [&](int i) __attribute__((always_inline)) {
    tm.mma(&sh_mem[(i & 1) * (P * LDN)], LDN);
  };
  auto softmax = [&]() __attribute__((always_inline)) { tm.template softmax<false>(scale_log2); };
  int i = 0;
  if (w < WAVES / 2) {
    for (int hh = 0; hh < hpg; ++hh) {
      mma(i);
      if (hh > 0) finish_head(hh - 1, IC<0>{});
      lds_barrier();
      softmax();
      stage_next(i);
      lds_barrier();
      ++i;
      for (int c = 1; c < k; ++c, ++i) {
        mma(i);
        lds_barrier();
        softmax();
        stage_next(i);
        lds_barrier();
      }
    }
    finish_head(hpg - 1, IC<1>{});  // step nsteps: the other waves fold in the last memory
    lds_barrier();
    lds_barrier();
  } else {
    for (int hh = 0; hh < hpg; ++hh) {
      if (hh > 0) {  // the previous head's last memory, and its finish in
        softmax();   // the same half as the lead waves' finish
        finish_head(hh - 1, IC<0>{});
      }
      stage_next(i);
      lds_barrier();
      mma(i);
      lds_barrier();
      ++i;
      for (int c = 1; c < k; ++c, ++i) {
        softmax();
        stage_next(i);
        lds_barrier();
        mma(i);
        lds_barrier();
      }
    }
    softmax();  // step nsteps: the last head's last memory
    finish_head(hpg - 1, IC<1>{});
    lds_barrier();
    lds_barrier();
  }
}

template <typename T, int N, int P, int NTB, int WAVES>
hipError_t sma_fwd_waves(const PrefillShape& s, const T* Q, const T* E, const T* C, const T* dH,
                         const T* y_ssd, const float* acum, float gate, T* y, const T* prior,
                         int k0, int pstride, float* o, float* lse, const uint8_t* prior8,
                         const float* pscale, hipStream_t st) {
  const int M = s.L / s.S;
  const int BH = s.B * s.H;
  const int hpg = s.H / s.G;
  const int bg_major = hpg > 1 && (s.B * s.G) % 8 == 0;
  const int npq = bg_major ? (s.B * s.G / 8) * hpg : (BH + 7) / 8;  // pairs per XCD
  const int tpc = s.S / (16 * NTB * WAVES);
  const int ngrp = (npq + kPairsPerGroup - 1) / kPairsPerGroup;
  const long blocks = 8L * ngrp * kPairsPerGroup * M * tpc;
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(N));
  if constexpr (std::is_same<T, bf16>::value) {
    if (prior8) {
      hipLaunchKernelGGL((k_sma_fwd<T, N, P, NTB, WAVES, false, true>), dim3(blocks),
                         dim3(64 * WAVES), 0, st, Q, E, C, dH, y_ssd, acum, gate, y, BH, s.L, s.H,
                         s.G, s.S, npq, bg_major, scale_log2, prior, k0, pstride, o, lse, prior8,
                         pscale);
      return hipGetLastError();
    }
  } else if (prior8) {
    return hipErrorNotSupported;
  }
  if constexpr (std::is_same<T, bf16>::value && WAVES >= 2 && P % 32 == 0 &&
                sma_grp_lds_bytes<N, P, NTB, WAVES>() <= 160 * 1024) {
    // heads sharing a group: one workgroup per (batch, group, tile), the
    // group's heads in turn (plain and training forward)
    if (hpg > 1 && !acum && k0 == 0) {
      const int BG = s.B * s.G, nbx = (BG + 7) / 8;
      const long gblocks = 8L * nbx * M * tpc;
      if (o)
        hipLaunchKernelGGL((k_sma_grp<N, P, NTB, WAVES, true>), dim3(gblocks), dim3(64 * WAVES),
                           0, st, Q, E, C, dH, y_ssd, gate, y, s.L, s.H, s.G, s.S, BG, nbx,
                           scale_log2, o, lse);
      else
        hipLaunchKernelGGL((k_sma_grp<N, P, NTB, WAVES, false>), dim3(gblocks), dim3(64 * WAVES),
                           0, st, Q, E, C, dH, y_ssd, gate, y, s.L, s.H, s.G, s.S, BG, nbx,
                           scale_log2, nullptr, nullptr);
      return hipGetLastError();
    }
  }
  if (acum)
    hipLaunchKernelGGL((k_sma_fwd<T, N, P, NTB, WAVES, true>), dim3(blocks), dim3(64 * WAVES), 0,
                       st, Q, E, C, dH, y_ssd, acum, gate, y, BH, s.L, s.H, s.G, s.S, npq,
                       bg_major, scale_log2, prior, k0, pstride, o, lse, nullptr, nullptr);
  else
    hipLaunchKernelGGL((k_sma_fwd<T, N, P, NTB, WAVES, false>), dim3(blocks), dim3(64 * WAVES), 0,
                       st, Q, E, C, dH, y_ssd, acum, gate, y, BH, s.L, s.H, s.G, s.S, npq,
                       bg_major, scale_log2, prior, k0, pstride, o, lse, nullptr, nullptr);
  return hipGetLastError();
}

}  // namespace

template <typename T, int N, int P>
hipError_t launch_sma_fwd(const PrefillShape& s, const T* Q, const T* E, const T* C,
                          const T* dH, const T* y_ssd, const float* acum, float gate, T* y,
                          const T* prior, int k0, int pstride, float* o, float* lse,
                          const uint8_t* prior8, const float* pscale, hipStream_t st) {
  constexpr int NTB = SmaTile<N, P>::NTB;
  const int r = s.S / (16 * NTB);  // S % 32 == 0, so r >= 1
  if (r % 8 == 0)
    return sma_fwd_waves<T, N, P, NTB, 8>(s, Q, E, C, dH, y_ssd, acum, gate, y, prior, k0,
                                           pstride, o, lse, prior8, pscale, st);
  if (r % 4 == 0)
    return sma_fwd_waves<T, N, P, NTB, 4>(s, Q, E, C, dH, y_ssd, acum, gate, y, prior, k0,
                                           pstride, o, lse, prior8, pscale, st);
  if (r % 2 == 0)
    return sma_fwd_waves<T, N, P, NTB, 2>(s, Q, E, C, dH, y_ssd, acum, gate, y, prior, k0,
                                           pstride, o, lse, prior8, pscale, st);
  return sma_fwd_waves<T, N, P, NTB, 1>(s, Q, E, C, dH, y_ssd, acum, gate, y, prior, k0, pstride,
                                        o, lse, prior8, pscale, st);
}


#define DART_INST_SMA(T, N, P)                                                                 \
  template hipError_t launch_sma_fwd<T, N, P>(const PrefillShape&, const T*, const T*, const T*, \
                                              const T*, const T*, const float*, float, T*,   \
                                              const T*, int, int, float*, float*,           \
                                              const uint8_t*, const float*, hipStream_t);
DART_FOR_EACH_SHAPE(DART_INST_SMA)

}  // namespace dart
