// State-memory attention (SMA) on gfx950: prefill over all tokens and the
// single-token decode step over the chunk-memory cache.
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

// online-softmax slack: weights may reach 2^kLazyLog2 before the running max
// (and with it every accumulator) is rescaled
constexpr float kLazyLog2 = 8.f;

template <int V>
using IC = std::integral_constant<int, V>;

// Sum of v over lanes l and l^16, then over l and l^32 (gfx950 permlane
// swaps: no LDS round trip).
__device__ __forceinline__ float sum_lane_groups(float v) {
  const unsigned u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const unsigned u2 = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(u2, u2, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

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

// Sum over all 64 lanes without LDS: DPP within each quad and row of 16
// lanes, then the two permlane swaps.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x124>(v);  // row_ror 4: quads q and q+1 of the row
  v += dpp_mov<0x128>(v);  // row_ror 8: the whole row of 16
  return sum_lane_groups(v);
}

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
template <typename T, int N, int P, int NTB, int WAVES, bool DECAY>
__global__ __launch_bounds__(64 * WAVES) void k_sma_fwd(
    const T* __restrict__ Q, const T* __restrict__ E, const T* __restrict__ C,
    const T* __restrict__ dH, const T* __restrict__ y_ssd, const float* __restrict__ acum,
    float gate, T* __restrict__ y, int BH, int L, int H, int G, int S, int npq, int bg_major,
    float scale_log2, const T* __restrict__ prior, int k0, int pstride) {
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
  constexpr int R1A = TWG * LDN > TWG * LDE ? TWG * LDN : TWG * LDE;
  constexpr int R1 = R1A > 2 * P * LDN ? R1A : 2 * P * LDN;
  typedef typename Vec16<T>::vec vec_t;
  // sh_r1: the Q, C and E tiles in turn during the prologue, then the two
  // memory buffers; sh_ty: y_ssd, overwritten by y in the epilogue
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

  // ---- prologue: every load in flight before the first wait ----
  vec_t qs[QV], cs[QV], es[EV], ys[EV];
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int i = tid + v * NTHR, t = i / (N / VE), nv = i % (N / VE);
    qs[v] = load16(Q + ((row0 + t) * G + g) * N + nv * VE);
  }
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    ys[v] = load16(y_ssd + ((row0 + t) * H + h) * P + pv * VE);
  }
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int i = tid + v * NTHR, t = i / (N / VE), nv = i % (N / VE);
    cs[v] = load16(C + ((row0 + t) * G + g) * N + nv * VE);
  }
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    es[v] = load16(E + ((row0 + t) * H + h) * P + pv * VE);
  }
  const T* mem = dH + (long)pair * M * (P * N);
  const T* pmem = k0 > 0 ? prior + (long)pair * pstride * (P * N) : nullptr;
  // loop step i multiplies memory mi(i): oldest first, or newest first with DECAY
  auto mi = [&](int i) __attribute__((always_inline)) { return DECAY ? k - 1 - i : i; };
  vec_t stg0[VPT], stg[VPT];
  auto gload = [&](int i, vec_t (&dst)[VPT]) __attribute__((always_inline)) {
    const int c = mi(i);
    const vec_t* src = reinterpret_cast<const vec_t*>(
        c < k0 ? pmem + (long)c * (P * N) : mem + (long)(c - k0) * (P * N));
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
        *reinterpret_cast<vec_t*>(&sh_mem[buf][p * LDN + nv * VE]) = src[v];
      }
    }
  };
  if (k > 0) {
    gload(0, stg0);
    gload(min(1, k - 1), stg);
  }
  // Q tile -> fragments; y_ssd parked for the epilogue
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int i = tid + v * NTHR, t = i / (N / VE), nv = i % (N / VE);
    *reinterpret_cast<vec_t*>(&sh_r1[t * LDN + nv * VE]) = qs[v];
  }
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    *reinterpret_cast<vec_t*>(&sh_ty[t * LDE + pv * VE]) = ys[v];
  }
  __syncthreads();
  SmaMath16<T, N, P, NTB> tm;
  tm.init(w, lane);
  tm.load_q(sh_r1, LDN);
  const float* acum_pair = DECAY ? acum + (long)pair * M * S : nullptr;
  if (DECAY) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) tm.at[tb] = acum_pair[(long)kl * S + sub * TWG + tm.lrow(tb)];
  }
  __syncthreads();
  // C tile -> fragments
#pragma unroll
  for (int v = 0; v < QV; ++v) {
    const int i = tid + v * NTHR, t = i / (N / VE), nv = i % (N / VE);
    *reinterpret_cast<vec_t*>(&sh_r1[t * LDN + nv * VE]) = cs[v];
  }
  __syncthreads();
  tm.load_c(sh_r1, LDN);
  __syncthreads();
  // E tile -> this lane's p rows, kept in the input type (bf16 pairs halve
  // the registers) and widened when the score is formed
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    *reinterpret_cast<vec_t*>(&sh_r1[t * LDE + pv * VE]) = es[v];
  }
  __syncthreads();
  tm.load_e(sh_r1, LDE);
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
  tm.finish(sh_ty, LDE, gate, k > 0);
  __syncthreads();
#pragma unroll
  for (int v = 0; v < EV; ++v) {
    const int i = tid + v * NTHR, t = i / (P / VE), pv = i % (P / VE);
    *reinterpret_cast<vec_t*>(y + ((row0 + t) * H + h) * P + pv * VE) =
        *reinterpret_cast<const vec_t*>(&sh_ty[t * LDE + pv * VE]);
  }
}

// Decode, step 1: one workgroup per (head, batch) advances the SSM state,
// forms y_ssd = C·h into the workspace and, when the token closes its chunk,
// appends the finished memory to the cache (at index n_chunks[b], which the
// streaming kernel never reads).  A launch of its own: done by the first of
// the streaming workgroups it held every stream back behind a latency-bound
// read-modify-write of 128 KB of state.
template <typename T, int N, int P>
__global__ __launch_bounds__(256) void k_decode_state(
    const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ C, T* __restrict__ cache,
    float* __restrict__ hst, float* __restrict__ dHc, const int* __restrict__ n_chunks,
    const int* __restrict__ pos, int* __restrict__ ws_flag, float* __restrict__ ws_yssd, int H,
    int G, int S, int max_chunks) {
  constexpr int Q4 = N / 4;
  static_assert((P * N / 4) % 64 == 0 && 64 % Q4 == 0, "decode state mapping");
  __shared__ float sh_c[N], sh_b[N], sh_x[P], sh_y[P];
  const int h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const long pair = (long)b * H + h;
  const int tid = threadIdx.x;
  int kc = n_chunks[b];
  kc = kc < 0 ? 0 : (kc > max_chunks ? max_chunks : kc);
  const int ps = pos[b];
  for (int i = tid; i < N; i += 256) {
    const long o = ((long)b * G + g) * N + i;
    sh_c[i] = to_f32(C[o]);
    sh_b[i] = to_f32(Bm[o]);
  }
  for (int i = tid; i < P; i += 256) sh_x[i] = to_f32(x[pair * P + i]);
  __syncthreads();
  {
    const float dtv = dt[pair];
    const float a = exp_neg(dtv * A[h]);
    const bool close = ps == S - 1;
    const bool append = close && kc < max_chunks;
    floatx4* hp = reinterpret_cast<floatx4*>(hst + pair * (P * N));
    floatx4* dp = reinterpret_cast<floatx4*>(dHc + pair * (P * N));
    T* cdst = cache + (pair * max_chunks + kc) * (long)(P * N);
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
      if (append) store4(cdst + (long)i * 4, dv[v]);
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
    if (close && !append && tid == 0) atomicOr(ws_flag, 1);
    __syncthreads();
    for (int p = tid; p < P; p += 256) ws_yssd[pair * P + p] = sh_y[p];
  }
}

// Decode, step 2: one workgroup (4 waves) per (split, head, batch) streams
// the cached memories of its split once from HBM.  Each wave takes whole
// memories c = first + wave, first + wave + 4, ... (non-temporal 16-byte
// loads): lane (nv, pr) holds key entries n in [nv·VE, nv·VE + VE) of rows
// p = it·RP + pr, forms partial Q·dH[c] and C·dH[c] over its n-range,
// reduces the score across the wave and keeps an online softmax whose value
// accumulator stays partial over n until the end.  The (max, denominator,
// numerator[P]) partial of the split goes to the workspace; k_decode_combine
// merges the splits and adds y_ssd.
template <typename T, int N, int P>
__global__ __launch_bounds__(256) void k_sma_decode(
    const T* __restrict__ C, const T* __restrict__ Q, const T* __restrict__ E,
    const T* __restrict__ cache, const int* __restrict__ n_chunks, float* __restrict__ ws_part,
    int H, int G, int max_chunks, int splits, int cps, float scale_log2) {
  constexpr int VE = Vec16<T>::n;
  constexpr int NV = N / VE;   // 16-byte vectors per memory row
  constexpr int RP = 64 / NV;  // rows per wave pass
  constexpr int NPASS = P / RP;
  constexpr int NW = 4;
  static_assert(64 % NV == 0 && P % RP == 0, "decode lane mapping");
  typedef typename Vec16<T>::vec vec_t;
  __shared__ float sh_q[N], sh_c[N], sh_e[P];
  __shared__ float sh_wm[NW], sh_wl[NW];
  __shared__ float sh_wacc[NW][P];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int g = h / (H / G);
  const long pair = (long)b * H + h;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int kc = n_chunks[b];
  kc = kc < 0 ? 0 : (kc > max_chunks ? max_chunks : kc);

  for (int i = tid; i < N; i += 256) {
    const long o = ((long)b * G + g) * N + i;
    sh_q[i] = to_f32(Q[o]);
    sh_c[i] = to_f32(C[o]);
  }
  for (int i = tid; i < P; i += 256) sh_e[i] = to_f32(E[pair * P + i]);
  __syncthreads();

  const int c_begin = split * cps;
  const int c_end = min(kc, c_begin + cps);
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
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  b2_t q2[VE / 2], c2[VE / 2];
  if constexpr (kDot2) {
#pragma unroll
    for (int e = 0; e < VE / 2; ++e) {
      q2[e] = b2_t{from_f32<bf16>(qv[2 * e]), from_f32<bf16>(qv[2 * e + 1])};
      c2[e] = b2_t{from_f32<bf16>(cv[2 * e]), from_f32<bf16>(cv[2 * e + 1])};
    }
  }
#pragma unroll
  for (int it = 0; it < NPASS; ++it) {
    ev[it] = sh_e[it * RP + pr];
    acc[it] = 0.f;
  }
  float mx = -INFINITY, ls = 0.f;
  const T* base = cache + pair * (long)max_chunks * (P * N);
  for (int c = c_begin + w; c < c_end; c += NW) {
    const T* src = base + (long)c * (P * N);
    vec_t raw[NPASS];
#pragma unroll
    for (int it = 0; it < NPASS; ++it) raw[it] = load16_nt(src + ((it * RP + pr) * NV + nv) * VE);
    float s = 0.f, zc[NPASS];
#pragma unroll
    for (int it = 0; it < NPASS; ++it) {
      float zq = 0.f, z2 = 0.f;
      if constexpr (kDot2) {
#pragma unroll
        for (int e = 0; e < VE / 2; ++e) {
          const b2_t v2 = b2_t{raw[it][2 * e], raw[it][2 * e + 1]};
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
    s = wave_sum_dpp(s) * scale_log2;
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
  }
#pragma unroll
  for (int it = 0; it < NPASS; ++it)
#pragma unroll
    for (int off = 1; off < NV; off <<= 1) acc[it] += __shfl_xor(acc[it], off);
  if (nv == 0) {
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
  for (int p = tid; p < P; p += 256) {
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      if (sh_wm[ww] > -INFINITY) {
        const float f = exp2_fast(sh_wm[ww] - mall);
        num += f * sh_wacc[ww][p];
        den += f * sh_wl[ww];
      }
    }
    float* part = ws_part + (pair * splits + split) * (P + 2);
    part[2 + p] = num;
    if (p == 0) {
      part[0] = mall;
      part[1] = den;
    }
  }
}

// Merge the per-split (max, denominator, numerator[P]) partials of one
// (batch, head) and apply the gate.
template <typename T>
__global__ __launch_bounds__(128) void k_decode_combine(const float* __restrict__ ws_yssd,
                                                        const float* __restrict__ ws_part,
                                                        float gate, T* __restrict__ y, int P,
                                                        int splits) {
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
}

// Advance the per-sequence position after every head has read it.
__global__ void k_decode_advance(int* __restrict__ n_chunks, int* __restrict__ pos, int B, int S,
                                 int max_chunks) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  if (pos[b] == S - 1) {
    const int k = n_chunks[b];
    n_chunks[b] = k < max_chunks ? k + 1 : max_chunks;
    pos[b] = 0;
  } else {
    pos[b] += 1;
  }
}

template <typename T, int N, int P, int NTB, int WAVES>
hipError_t sma_fwd_waves(const PrefillShape& s, const T* Q, const T* E, const T* C, const T* dH,
                         const T* y_ssd, const float* acum, float gate, T* y, const T* prior,
                         int k0, int pstride, hipStream_t st) {
  const int M = s.L / s.S;
  const int BH = s.B * s.H;
  const int hpg = s.H / s.G;
  const int bg_major = hpg > 1 && (s.B * s.G) % 8 == 0;
  const int npq = bg_major ? (s.B * s.G / 8) * hpg : (BH + 7) / 8;  // pairs per XCD
  const int tpc = s.S / (16 * NTB * WAVES);
  const int ngrp = (npq + kPairsPerGroup - 1) / kPairsPerGroup;
  const long blocks = 8L * ngrp * kPairsPerGroup * M * tpc;
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(N));
  if (acum)
    hipLaunchKernelGGL((k_sma_fwd<T, N, P, NTB, WAVES, true>), dim3(blocks), dim3(64 * WAVES), 0,
                       st, Q, E, C, dH, y_ssd, acum, gate, y, BH, s.L, s.H, s.G, s.S, npq,
                       bg_major, scale_log2, prior, k0, pstride);
  else
    hipLaunchKernelGGL((k_sma_fwd<T, N, P, NTB, WAVES, false>), dim3(blocks), dim3(64 * WAVES), 0,
                       st, Q, E, C, dH, y_ssd, acum, gate, y, BH, s.L, s.H, s.G, s.S, npq,
                       bg_major, scale_log2, prior, k0, pstride);
  return hipGetLastError();
}

}  // namespace

template <typename T, int N, int P>
hipError_t launch_sma_fwd(const PrefillShape& s, const T* Q, const T* E, const T* C,
                          const T* dH, const T* y_ssd, const float* acum, float gate, T* y,
                          const T* prior, int k0, int pstride, hipStream_t st) {
  constexpr int NTB = SmaTile<N, P>::NTB;
  const int r = s.S / (16 * NTB);  // S % 32 == 0, so r >= 1
  if (r % 8 == 0)
    return sma_fwd_waves<T, N, P, NTB, 8>(s, Q, E, C, dH, y_ssd, acum, gate, y, prior, k0,
                                           pstride, st);
  if (r % 4 == 0)
    return sma_fwd_waves<T, N, P, NTB, 4>(s, Q, E, C, dH, y_ssd, acum, gate, y, prior, k0,
                                           pstride, st);
  if (r % 2 == 0)
    return sma_fwd_waves<T, N, P, NTB, 2>(s, Q, E, C, dH, y_ssd, acum, gate, y, prior, k0,
                                           pstride, st);
  return sma_fwd_waves<T, N, P, NTB, 1>(s, Q, E, C, dH, y_ssd, acum, gate, y, prior, k0, pstride,
                                        st);
}

template <typename T, int N, int P>
hipError_t launch_sma_decode(const DecodeShape& s, const T* x, const float* dt, const float* A,
                             const T* Bm, const T* C, const T* Q, const T* E, float gate,
                             T* cache, float* h, float* dH_cur, int* n_chunks, int* pos, T* y,
                             void* workspace, hipStream_t st) {
  const long pairs = (long)s.B * s.H;
  char* ws = static_cast<char*>(workspace);
  int* flag = reinterpret_cast<int*>(ws);
  float* ws_yssd = reinterpret_cast<float*>(ws + 256);
  float* ws_part = reinterpret_cast<float*>(
      ws + 256 + ((pairs * P * sizeof(float) + 255) / 256) * 256);
  const int cps = (s.max_chunks + s.splits - 1) / s.splits;
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(N));
  hipLaunchKernelGGL((k_decode_state<T, N, P>), dim3(1, s.H, s.B), dim3(256), 0, st, x, dt, A, Bm,
                     C, cache, h, dH_cur, n_chunks, pos, flag, ws_yssd, s.H, s.G, s.S,
                     s.max_chunks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_sma_decode<T, N, P>), dim3(s.splits, s.H, s.B), dim3(256), 0, st, C, Q,
                     E, cache, n_chunks, ws_part, s.H, s.G, s.max_chunks, s.splits, cps,
                     scale_log2);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode_combine<T>), dim3(pairs), dim3(128), 0, st, ws_yssd, ws_part,
                     gate, y, P, s.splits);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_advance, dim3((s.B + 255) / 256), dim3(256), 0, st, n_chunks, pos,
                     s.B, s.S, s.max_chunks);
  return hipGetLastError();
}

#define DART_INST_SMA(T, N, P)                                                                 \
  template hipError_t launch_sma_fwd<T, N, P>(const PrefillShape&, const T*, const T*, const T*, \
                                              const T*, const T*, const float*, float, T*,   \
                                              const T*, int, int, hipStream_t);              \
  template hipError_t launch_sma_decode<T, N, P>(                                                \
      const DecodeShape&, const T*, const float*, const float*, const T*, const T*, const T*,    \
      const T*, float, T*, float*, float*, int*, int*, T*, void*, hipStream_t);
DART_FOR_EACH_SHAPE(DART_INST_SMA)

}  // namespace dart
