// Backward of state-memory attention and the gated add on gfx950 (16-bit io).
//
// Forward (Pith review of DART, "Core claim" and "What carries the argument";
// referee major comment 3, paper §3 Eq. 8): for token t of chunk k and each
// memory c < k, Zq = dH[c]ᵀQ_t and Zc = dH[c]ᵀC_t (in R^P), score
// s = E_t·Zq / sqrt(N), α = softmax_c(s), o_t = Σ_c α·Zc, y_t = y_ssd_t + g·o_t.
// Reverse mode, with do_t = g·dy_t and D_t = do_t·o_t:
//   ds_{t,c} = α_{t,c}·(do_t·Zc_{t,c} − D_t)
//   dE_t   = Σ_c ds·Zq / sqrt(N)
//   dQ_t   = Σ_c (ds / sqrt(N))·dH[c]·E_t        (summed over a group's heads)
//   dC_t   = Σ_c α·dH[c]·do_t                    (summed over a group's heads)
//   ddH[c] = Σ_t (ds / sqrt(N))·Q_t E_tᵀ + α·C_t do_tᵀ
//   dg     = Σ_t dy_t·o_t,  dy_ssd = dy
// α is recomputed from the forward's base-2 log-normaliser (lse), so no
// per-(token, memory) value is stored.
//
// k_sma_bwd_prep: dy·o per (token, head) and the gate gradient.
// k_sma_bwd_tok:  token-major (as the forward): dQ, dC, dE; it also leaves
//                 ds/sqrt(N) and g·α of every visible (token, memory) pair
//                 in the workspace.
// k_sma_bwd_mem4: memory-major: ddH[c] from every later token, from those
//                 factors (no recomputation).
// The token kernel recomputes Zq and Zc with the forward's MFMA tiles; the
// products with dH[c] taken along P (dQ, dC) and the token sums (ddH) read
// their operands with gfx950's LDS transpose reads.
#include "dart_launch.hpp"
#include "dart_shapes.hpp"

namespace dart {
namespace {


// (batch, token) rows per workgroup of the dy·o pass (each workgroup leaves
// one partial of the gate gradient)
constexpr int kPrepRows = 4;

// Eight values -> an MFMA operand fragment.
__device__ __forceinline__ bf16x8 pack8(const float (&v)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = from_f32<bf16>(v[e]);
  return r;
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// dy·o for every (batch, token, head): each workgroup takes kPrepRows
// consecutive (batch, token) rows of H·P values (all their loads issued
// before the first use), 16-byte vectors, the P/8 lanes of a head summed by
// lane exchanges.  Each workgroup's Σ dy·o goes to part[blockIdx] for the
// gate gradient.
template <int P>
__global__ __launch_bounds__(256) void k_sma_bwd_prep(const bf16* __restrict__ dy,
                                                      const float* __restrict__ o,
                                                      float* __restrict__ dyo,
                                                      float* __restrict__ part, long rows, int L,
                                                      int H) {
  constexpr int LPH = P / 8;  // lanes per head
  constexpr int IT = 4;  // 16-byte items per thread and pass (all loads of a pass in flight)
  static_assert(LPH <= 64 && 64 % LPH == 0, "prep lanes");
  __shared__ float sh[4];
  const int HL = H * LPH;  // 16-byte vectors of dy per row
  const int items = kPrepRows * HL;
  float tot = 0.f;
  for (int base = 0; base < items; base += IT * 256) {
    bf16x8 a[IT];
    floatx4 c0[IT], c1[IT];
#pragma unroll
    for (int k = 0; k < IT; ++k) {  // every load of the pass in flight first
      const int i = base + k * 256 + threadIdx.x;
      const long row = blockIdx.x * kPrepRows + i / HL;
      const int v = i % HL;
      a[k] = bf16x8{};
      c0[k] = c1[k] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (i < items && row < rows) {
        a[k] = *reinterpret_cast<const bf16x8*>(dy + row * H * P + v * 8);
        c0[k] = *reinterpret_cast<const floatx4*>(o + row * H * P + v * 8);
        c1[k] = *reinterpret_cast<const floatx4*>(o + row * H * P + v * 8 + 4);
      }
    }
#pragma unroll
    for (int k = 0; k < IT; ++k) {
      const int i = base + k * 256 + threadIdx.x;
      const long row = blockIdx.x * kPrepRows + i / HL;
      const int v = i % HL;
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) d += to_f32(a[k][e]) * c0[k][e] + to_f32(a[k][4 + e]) * c1[k][e];
#pragma unroll
      for (int off = 1; off < LPH; off <<= 1) d += __shfl_xor(d, off);
      if (v % LPH == 0 && i < items && row < rows) {
        const int b = static_cast<int>(row / L), t = static_cast<int>(row % L);
        dyo[((long)b * H + v / LPH) * L + t] = d;
        tot += d;
      }
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) tot += __shfl_xor(tot, off);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = tot;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = sh[0] + sh[1] + sh[2] + sh[3];
}

// Offset of memory c's factors within the backward workspace's factor
// array: (batch, head) pairs one after another, each holding, for c = 0 ..
// M-2, the S·(M-1-c) tokens of chunks c+1 .. M-1 in order.
__host__ __device__ __forceinline__ long dsga_offset(long pair, int c, int M, int S) {
  return (pair * M * (M - 1) / 2 + (long)c * (M - 1) - (long)c * (c - 1) / 2) * S;
}

// Σ part[0 .. n) -> *out (one workgroup, fixed order).
__global__ __launch_bounds__(256) void k_sum(const float* __restrict__ part, long n,
                                             float* __restrict__ out) {
  __shared__ float sh[4];
  float s = 0.f;
  for (long i = threadIdx.x; i < n; i += 256) s += part[i];
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) *out = sh[0] + sh[1] + sh[2] + sh[3];
}

// Token-major backward.  One workgroup = WAVES waves × 16 tokens of one
// chunk k of one (batch, group); it walks the heads of the group (Q and C,
// and so dQ and dC, are shared by them) and, per head, the memories c < k,
// each staged in LDS as rows [p][n] (two buffers, one barrier per memory).
// Per memory a wave
//   - forms Zq, Zc with the forward's fragments (A = memory rows p, K = n),
//   - recomputes α from lse and forms ds (two in-lane dots + lane-group
//     exchanges),
//   - accumulates dE in registers,
//   - multiplies the memory taken along P (A = rows n, K = p, by transpose
//     reads) with B operands E·ds/sqrt(N) and g·α·dy that it builds in
//     registers: the k-slots of lane group grp are the p values the lane
//     already holds (p = (2kk + e/4)·16 + 4·grp + e%4), so no exchange is needed.
// Grid: (batch, group) pairs dealt to the 8 XCDs (blockIdx % 8) when their
// count allows, heaviest chunks first.
//
// dsga: for each (batch, head) the factors (ds/sqrt(N), g·α) of memory c
// for the tokens of chunks c+1 .. M-1, memories one after another (see
// dsga_offset).
template <int N, int P, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_sma_bwd_tok(
    const bf16* __restrict__ Q, const bf16* __restrict__ E, const bf16* __restrict__ C,
    const bf16* __restrict__ dH, const bf16* __restrict__ dy, const float* __restrict__ lse,
    const float* __restrict__ dyo, float gate, float* __restrict__ dQ, float* __restrict__ dE,
    float* __restrict__ dC, float2* __restrict__ dsga, int B, int L, int H, int G, int S,
    float scale_log2, float rsn) {
  constexpr int NKK = N / 32, NPB = P / 16, NNB = N / 16, NK2 = P / 32;
  constexpr int LDN = N + 16;
  constexpr int NTHR = 64 * WAVES, NVEC = P * N / 8;
  constexpr int VPT = (NVEC + NTHR - 1) / NTHR;
  static_assert(P % 32 == 0 && N % 32 == 0, "backward tile shapes");
  __shared__ __align__(16) bf16 sh_mem[2][P * LDN];

  const int M = L / S, tpc = S / (16 * WAVES), nbg = B * G, hpg = H / G;
  int bg, kr, sub;
  if (nbg % 8 == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = nbg / 8;
    sub = slot % tpc;
    const int r = slot / tpc;
    bg = (r % per) * 8 + xcd;
    kr = r / per;
  } else {
    sub = blockIdx.x % tpc;
    const int r = blockIdx.x / tpc;
    bg = r % nbg;
    kr = r / nbg;
  }
  const int k = M - 1 - kr;
  const int b = bg / G, g = bg % G;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tok = k * S + sub * 16 * WAVES + w * 16 + col;  // this lane's token column
  const long row = (long)b * L + tok;

  floatx4 dq[NNB], dc[NNB];
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) {
    dq[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    dc[nb] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  if (k == 0) {  // no memory is visible: zero gradients
#pragma unroll
    for (int hh = 0; hh < hpg; ++hh)
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
        *reinterpret_cast<floatx4*>(dE + (row * H + g * hpg + hh) * P + pb * 16 + 4 * grp) =
            floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      *reinterpret_cast<floatx4*>(dQ + (row * G + g) * N + nb * 16 + 4 * grp) = dq[nb];
      *reinterpret_cast<floatx4*>(dC + (row * G + g) * N + nb * 16 + 4 * grp) = dc[nb];
    }
    return;
  }
  bf16x8 qf[NKK], cf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8*>(Q + (row * G + g) * N + kk * 32 + grp * 8);
    cf[kk] = *reinterpret_cast<const bf16x8*>(C + (row * G + g) * N + kk * 32 + grp * 8);
  }
  typedef typename Vec16<bf16>::vec vec_t;
  vec_t stg[VPT];
  auto gload = [&](const bf16* mem, int c) __attribute__((always_inline)) {
    const vec_t* src = reinterpret_cast<const vec_t*>(mem + (long)c * (P * N));
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int vi = threadIdx.x + v * NTHR;
      if (NVEC % NTHR == 0 || vi < NVEC) stg[v] = src[vi];
    }
  };
  auto swrite = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < VPT; ++v) {
      const int vi = threadIdx.x + v * NTHR;
      if (NVEC % NTHR == 0 || vi < NVEC) {
        const int p = vi / (N / 8), nv = vi % (N / 8);
        *reinterpret_cast<vec_t*>(&sh_mem[buf][p * LDN + nv * 8]) = stg[v];
      }
    }
  };

  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
    const bf16* mem = dH + pair * M * (P * N);
    gload(mem, 0);
    bf16x4 ev[NPB], dv[NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) {
      ev[pb] = *reinterpret_cast<const bf16x4*>(E + (row * H + h) * P + pb * 16 + 4 * grp);
      dv[pb] = *reinterpret_cast<const bf16x4*>(dy + (row * H + h) * P + pb * 16 + 4 * grp);
    }
    const float lse_t = lse[pair * L + tok];
    const float D_t = gate * dyo[pair * L + tok];
    float2* fac = dsga + dsga_offset(pair, 0, M, S) + tok - S;  // memory 0's entry of tok
    floatx4 de[NPB];
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) de[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
    swrite(0);
    gload(mem, min(1, k - 1));
    __syncthreads();
    for (int c = 0; c < k; ++c) {
      const bf16* ml = sh_mem[c & 1];
      floatx4 zq[NPB], zc[NPB];
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        zq[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
        zc[pb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(&ml[(pb * 16 + col) * LDN + kk * 32 + grp * 8]);
          zq[pb] = Mma<bf16>::mma(a, qf[kk], zq[pb]);
          zc[pb] = Mma<bf16>::mma(a, cf[kk], zc[pb]);
        }
      }
      float s = 0.f, da = 0.f;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s += zq[pb][i] * to_f32(ev[pb][i]);
          da += zc[pb][i] * to_f32(dv[pb][i]);
        }
      s = sum_lane_groups(s) * scale_log2;
      da = sum_lane_groups(da) * gate;
      const float al = exp2_fast(s - lse_t);
      const float dsr = al * (da - D_t) * rsn;
      const float ga = gate * al;
      if (grp == 0) fac[0] = float2{dsr, ga};
      fac += (long)(M - 2 - c) * S;  // to memory c+1's entry of tok
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) de[pb] += dsr * zq[pb];
      bf16x8 b1[NK2], b2[NK2];
#pragma unroll
      for (int k2 = 0; k2 < NK2; ++k2) {
        float v1[8], v2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v1[e] = to_f32(ev[2 * k2 + e / 4][e % 4]) * dsr;
          v2[e] = to_f32(dv[2 * k2 + e / 4][e % 4]) * ga;
        }
        b1[k2] = pack8(v1);
        b2[k2] = pack8(v2);
      }
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb)
#pragma unroll
        for (int k2 = 0; k2 < NK2; ++k2) {
          const bf16* base = &ml[(k2 * 32 + 4 * grp + col / 4) * LDN + nb * 16 + 4 * (col % 4)];
          const bf16x8 a = cat8(lds_read_tr4(base), lds_read_tr4(base + 16 * LDN));
          dq[nb] = Mma<bf16>::mma(a, b1[k2], dq[nb]);
          dc[nb] = Mma<bf16>::mma(a, b2[k2], dc[nb]);
        }
      swrite((c + 1) & 1);
      gload(mem, min(c + 2, k - 1));
      __syncthreads();
    }
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
      *reinterpret_cast<floatx4*>(dE + (row * H + h) * P + pb * 16 + 4 * grp) = de[pb];
  }
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) {
    *reinterpret_cast<floatx4*>(dQ + (row * G + g) * N + nb * 16 + 4 * grp) = dq[nb];
    *reinterpret_cast<floatx4*>(dC + (row * G + g) * N + nb * 16 + 4 * grp) = dc[nb];
  }
}

// Memory-major backward: ddH[c] = Σ_t (Q_t·ds/sqrt(N)) E_tᵀ + (C_t·g·α) dy_tᵀ
// over the 64-token tiles of the chunks after c, one workgroup (8 waves) per
// (batch, head) and four memories c0 = 4j .. 4j+3.  The factors ds/sqrt(N)
// and g·α come from the token-major kernel, so a tile needs no
// recomputation, and the sums are MFMAs whose K axis is the token, both
// operands read as token columns by transpose reads.  The kernel's time
// goes to fetching the tiles (every later tile of the sequence, for every
// group of memories), so each staged tile serves four memories.  Q, C, E and dy rows are staged once per tile with the
// four memories' factor pairs (ds/sqrt(N), g·α) of its tokens
// (double-buffered, one barrier per tile, the next tile fetched into
// registers while the current one is multiplied); each wave scales its E
// and dy operands by its memory's factors after the transpose reads (the
// same f32 product and rounding as scaling them at staging).
// Waves 2m, 2m+1 take memory c0 + m, rows n of half w%2 of ddH[c], every
// token of the tile (two 32-token K-steps).
template <int N, int P>
__global__ __launch_bounds__(512) void k_sma_bwd_mem4(
    const bf16* __restrict__ Q, const bf16* __restrict__ E, const bf16* __restrict__ C,
    const bf16* __restrict__ dy, const float2* __restrict__ dsga, float* __restrict__ ddH,
    int B, int L, int H, int G, int S) {
  constexpr int NPB = P / 16, NNB = N / 16;
  constexpr int NBW = NNB / 2;  // n blocks per wave
  constexpr int LDN = N + 16, LDP = P + 16, T = 64, NT = 512, MEMS = 4;
  constexpr int QN = T * N / 8, EN = T * P / 8;  // 16-byte vectors of a Q (C) and an E (dy) tile
  constexpr int QV = (QN + NT - 1) / NT, EV = (EN + NT - 1) / NT;
  constexpr int TILE = 2 * T * LDN + 2 * T * LDP;  // bf16: Q, C, E, dy rows
  constexpr int BUF = TILE + MEMS * T * 4;         // then float2 factors [memory][token]
  static_assert((TILE * 2) % 16 == 0 && MEMS * T <= NT, "k_sma_bwd_mem4 layout");
  __shared__ __align__(16) bf16 sh[2 * BUF];

  const int M = L / S, BH = B * H, hpg = H / G;
  int pair, j;
  if ((B * G) % 8 == 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, per = BH / 8;
    const int jj = slot % per;
    j = slot / per;
    pair = ((jj / hpg) * 8 + xcd) * hpg + jj % hpg;
  } else {
    pair = blockIdx.x % BH;
    j = blockIdx.x / BH;
  }
  const int b = pair / H, h = pair % H, g = h / hpg;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mw = w >> 1, nh = w & 1;
  const int c0 = MEMS * j, c = c0 + mw;
  const bool live = c < M;

  floatx4 acc[NBW][NPB];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) acc[i][pb] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int ntile = (M - 1 - c0) * (S / T);
  auto kc = [&](int i) __attribute__((always_inline)) { return M - 1 - i / (S / T); };
  auto tok0 = [&](int i) __attribute__((always_inline)) {
    return kc(i) * S + (i % (S / T)) * T;
  };
  // this thread's factor slot: memory fm, token ft of the tile
  const int fm = tid / T, ft = tid % T;
  const bool fslot = tid < MEMS * T && c0 + fm < M;
  const long fbase = fslot ? dsga_offset(pair, c0 + fm, M, S) - (long)(c0 + fm + 1) * S : 0;
  bf16x8 rq[QV], rc[QV], re[EV], rd[EV];
  float2 rf;
  auto fetch = [&](int i) __attribute__((always_inline)) {
    const int t0 = tok0(i);
    const long r0 = (long)b * L + t0;
#pragma unroll
    for (int v = 0; v < QV; ++v) {
      const int vi = tid + v * NT, t = vi / (N / 8), nv = vi % (N / 8);
      if (QN % NT == 0 || vi < QN) {
        rq[v] = *reinterpret_cast<const bf16x8*>(Q + ((r0 + t) * G + g) * N + nv * 8);
        rc[v] = *reinterpret_cast<const bf16x8*>(C + ((r0 + t) * G + g) * N + nv * 8);
      }
    }
#pragma unroll
    for (int v = 0; v < EV; ++v) {
      const int vi = tid + v * NT, t = vi / (P / 8), pv = vi % (P / 8);
      if (EN % NT == 0 || vi < EN) {
        re[v] = *reinterpret_cast<const bf16x8*>(E + ((r0 + t) * H + h) * P + pv * 8);
        rd[v] = *reinterpret_cast<const bf16x8*>(dy + ((r0 + t) * H + h) * P + pv * 8);
      }
    }
    // memory c0 + fm takes part in the tiles of later chunks only
    rf = fslot && kc(i) > c0 + fm ? dsga[fbase + t0 + ft] : float2{0.f, 0.f};
  };
  auto stage = [&](int buf) __attribute__((always_inline)) {
    bf16* sQ = sh + buf * BUF;
    bf16* sC = sQ + T * LDN;
    bf16* sE = sC + T * LDN;
    bf16* sD = sE + T * LDP;
    float2* sF = reinterpret_cast<float2*>(sQ + TILE);
#pragma unroll
    for (int v = 0; v < QV; ++v) {
      const int vi = tid + v * NT, t = vi / (N / 8), nv = vi % (N / 8);
      if (QN % NT == 0 || vi < QN) {
        *reinterpret_cast<bf16x8*>(&sQ[t * LDN + nv * 8]) = rq[v];
        *reinterpret_cast<bf16x8*>(&sC[t * LDN + nv * 8]) = rc[v];
      }
    }
#pragma unroll
    for (int v = 0; v < EV; ++v) {
      const int vi = tid + v * NT, t = vi / (P / 8), pv = vi % (P / 8);
      if (EN % NT == 0 || vi < EN) {
        *reinterpret_cast<bf16x8*>(&sE[t * LDP + pv * 8]) = re[v];
        *reinterpret_cast<bf16x8*>(&sD[t * LDP + pv * 8]) = rd[v];
      }
    }
    if (tid < MEMS * T) sF[tid] = rf;
  };
  auto multiply = [&](int buf) __attribute__((always_inline)) {
    const bf16* sQ = sh + buf * BUF;
    const bf16* sC = sQ + T * LDN;
    const bf16* sE = sC + T * LDN;
    const bf16* sD = sE + T * LDP;
    const float2* sF = reinterpret_cast<const float2*>(sQ + TILE) + mw * T;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r0 = ks * 32 + 4 * grp;  // this lane's tokens r0 .. r0+3, r0+16 .. r0+19
      float2 f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = sF[r0 + e];
        f[4 + e] = sF[r0 + 16 + e];
      }
      bf16x8 be[NPB], bd[NPB];
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        const int o = (r0 + col / 4) * LDP + pb * 16 + 4 * (col % 4);
        const bf16x8 xe = cat8(lds_read_tr4(&sE[o]), lds_read_tr4(&sE[o + 16 * LDP]));
        const bf16x8 xd = cat8(lds_read_tr4(&sD[o]), lds_read_tr4(&sD[o + 16 * LDP]));
        float ve[8], vd[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ve[e] = to_f32(xe[e]) * f[e].x;
          vd[e] = to_f32(xd[e]) * f[e].y;
        }
        be[pb] = pack8(ve);
        bd[pb] = pack8(vd);
      }
#pragma unroll
      for (int i2 = 0; i2 < NBW; ++i2) {
        const int nb = nh * NBW + i2;
        const int o = (r0 + col / 4) * LDN + nb * 16 + 4 * (col % 4);
        const bf16x8 aq = cat8(lds_read_tr4(&sQ[o]), lds_read_tr4(&sQ[o + 16 * LDN]));
        const bf16x8 ac = cat8(lds_read_tr4(&sC[o]), lds_read_tr4(&sC[o + 16 * LDN]));
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) {
          acc[i2][pb] = Mma<bf16>::mma(aq, be[pb], acc[i2][pb]);
          acc[i2][pb] = Mma<bf16>::mma(ac, bd[pb], acc[i2][pb]);
        }
      }
    }
  };
  if (ntile > 0) {
    fetch(0);
    stage(0);
  }
  __syncthreads();
  for (int i = 0; i < ntile; ++i) {
    // buffer i&1 holds tile i; buffer (i+1)&1 was last read before the
    // previous barrier
    if (i + 1 < ntile) fetch(i + 1);
    if (live && kc(i) > c) multiply(i & 1);  // uniform over the wave
    if (i + 1 < ntile) stage((i + 1) & 1);
    __syncthreads();
  }
  // ddH[c] rows [p][n]: lane holds n = nb·16 + 4·grp .. +3 of column p = pb·16 + col
  if (live) {
    float* out = ddH + ((long)pair * M + c) * (P * N);
#pragma unroll
    for (int i2 = 0; i2 < NBW; ++i2)
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        const int nb = nh * NBW + i2;
        *reinterpret_cast<floatx4*>(out + (pb * 16 + col) * N + nb * 16 + 4 * grp) =
            acc[i2][pb];
      }
  }
}

}  // namespace

template <typename T, int N, int P>
hipError_t launch_sma_bwd(const PrefillShape& s, const T* Q, const T* E, const T* C,
                          const T* dH, const float* o, const float* lse, const T* dy,
                          float gate, float* dQ, float* dE, float* dC, float* ddH,
                          float* dgate, void* workspace, hipStream_t st) {
  if constexpr (std::is_same<T, float>::value) {
    return launch_sma_bwd_f32<N, P>(s, Q, E, C, dH, o, lse, dy, gate, dQ, dE, dC, ddH, dgate,
                                    workspace, st);
  } else if constexpr (!std::is_same<T, bf16>::value || P > 64) {
    return hipErrorNotSupported;
  } else {
    const int M = s.L / s.S;
    const long rows = (long)s.B * s.L;
    const long pblocks = (rows + kPrepRows - 1) / kPrepRows;
    float* dyo = static_cast<float*>(workspace);
    float* part = dyo + ((rows * s.H + 63) / 64) * 64;
    float2* dsga = reinterpret_cast<float2*>(part + (pblocks + 63) / 64 * 64);
    const float scale_log2 = kLog2e / sqrtf(static_cast<float>(N));
    const float rsn = 1.f / sqrtf(static_cast<float>(N));
    hipLaunchKernelGGL((k_sma_bwd_prep<P>), dim3(pblocks), dim3(256), 0, st, dy, o, dyo, part,
                       rows, s.L, s.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sum, dim3(1), dim3(256), 0, st, part, pblocks, dgate);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int waves = s.S % 128 == 0 ? 8 : 4;  // S is a multiple of 64
    const long tblocks = (long)s.B * s.G * M * (s.S / (16 * waves));
    if (waves == 8)
      hipLaunchKernelGGL((k_sma_bwd_tok<N, P, 8>), dim3(tblocks), dim3(512), 0, st, Q, E, C, dH,
                         dy, lse, dyo, gate, dQ, dE, dC, dsga, s.B, s.L, s.H, s.G, s.S,
                         scale_log2, rsn);
    else
      hipLaunchKernelGGL((k_sma_bwd_tok<N, P, 4>), dim3(tblocks), dim3(256), 0, st, Q, E, C, dH,
                         dy, lse, dyo, gate, dQ, dE, dC, dsga, s.B, s.L, s.H, s.G, s.S,
                         scale_log2, rsn);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_sma_bwd_mem4<N, P>), dim3((long)s.B * s.H * ((M + 3) / 4)), dim3(512),
                       0, st, Q, E, C, dy, dsga, ddH, s.B, s.L, s.H, s.G, s.S);
    return hipGetLastError();
  }
}

// dy·o [B,H,L] and the gate partials (f32, each padded to 64 values), then
// the factor pairs of every visible (token, memory): B·H·L·(M-1)/2 float2.
size_t sma_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t S) {
  const size_t rows = static_cast<size_t>(B * L), M = static_cast<size_t>(L / S);
  const size_t pblocks = (rows + kPrepRows - 1) / kPrepRows;
  return (((rows * H + 63) / 64) * 64 + (pblocks + 63) / 64 * 64) * sizeof(float) +
         static_cast<size_t>(B * H * S) * (M * (M - 1) / 2) * sizeof(float2);
}

#define DART_INST_SMA_BWD(T, N, P)                                                              \
  template hipError_t launch_sma_bwd<T, N, P>(const PrefillShape&, const T*, const T*, const T*, \
                                              const T*, const float*, const float*, const T*,    \
                                              float,                                             \
                                              float*, float*, float*, float*, float*, void*,     \
                                              hipStream_t);
DART_FOR_EACH_SHAPE(DART_INST_SMA_BWD)

}  // namespace dart
