// Backward of the chunked scan on gfx950 (16-bit io).
//
// Forward (Pith review of DART, "What carries the argument" and the axiom
// ledger: SSD as structured causal attention, paper Eq. 4, split into
// intra- and inter-chunk terms): with u_t = A·Σ_{l=kS}^{t} dt_l (acum, the
// log-decay from the start of token t's chunk k) and U_c = u at the last
// token of chunk c,
//   memory  dH[c]    = Σ_i exp(U_c − u_i)·dt_i·B_i x_iᵀ
//   state   H_in[c+1] = exp(U_c)·H_in[c] + dH[c]
//   output  y_t = Σ_{j<=t} (C_t·B_j)·exp(u_t − u_j)·dt_j·x_j + exp(u_t)·C_tᵀH_in[k]
// Reverse mode, given dy (of y_ssd), ddH (of the memories, from SMA) and
// dh_final:
//   k_ssd_bwd_yc:   Yc[c] = Σ_{t in c} exp(u_t)·C_t dy_tᵀ, the gradient the
//                   outputs of chunk c send to H_in[c]
//   k_ssd_bwd_pass: last chunk first, G = dh_final; dmem[c] = G + ddH[c];
//                   the log-decay gradient <G, exp(U_c)·H_in[c]>;
//                   G = exp(U_c)·G + Yc[c]; dh0 = G
//   k_ssd_bwd_j:    per 64-token key block j: dx, dB, the direct dt
//                   gradient and the log-decay gradients of the memory term
//                   and of the intra term's keys
//   k_ssd_bwd_t:    per 64-token query block t: dC of the intra and inter
//                   terms and the queries' log-decay gradients
//   k_ssd_bwd_fin:  log-decay gradients -> dt (reverse cumulative sum inside
//                   the chunk, times A) and partial dA
//   k_head_sum:     dA summed over batch and chunks.
// The key- and query-block kernels walk the heads of a group, so dB and dC
// (shared by those heads) are summed in registers.
// Intra-chunk products run on MFMA tiles of 16 tokens × 16 tokens whose D
// registers are fed back as the next product's B operand (K = tokens), the
// token-axis A operands read by LDS transpose reads.
#include "dart_launch.hpp"
#include "dart_shapes.hpp"

namespace dart {
namespace {

constexpr int kT = 64;  // tokens per block

__device__ __forceinline__ bf16x8 pack8f(const float (&v)[8]) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = from_f32<bf16>(v[e]);
  return r;
}
__device__ __forceinline__ bf16x8 cat8b(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
// A operand, rows f (feature block fb·16 + col), K = 32 tokens ks·32 +
// {4·grp .. +3, 16 + 4·grp .. +3}, from LDS rows [token][feature] (stride LD)
template <int LD>
__device__ __forceinline__ bf16x8 tr_frag(const bf16* tile, int ks, int fb, int col, int grp) {
  const bf16* p = tile + (ks * 32 + 4 * grp + col / 4) * LD + fb * 16 + 4 * (col % 4);
  return cat8b(lds_read_tr4(p), lds_read_tr4(p + 16 * LD));
}
// B operand, column = LDS row `r`, the same token-style K slots but along the
// row's features: elements ks·32 + 4·grp .. +3 and ks·32 + 16 + 4·grp .. +3
__device__ __forceinline__ bf16x8 row_frag_split(const bf16* row, int ks, int grp) {
  return cat8b(*reinterpret_cast<const bf16x4*>(row + ks * 32 + 4 * grp),
               *reinterpret_cast<const bf16x4*>(row + ks * 32 + 16 + 4 * grp));
}
// 64 rows of F features from a token-major tensor (row stride gs) into LDS
// rows of stride LD; 256 threads
template <int F, int LD>
__device__ __forceinline__ void stage_rows(bf16* dst, const bf16* src, long gs) {
  constexpr int VR = F / 8;
  for (int vi = threadIdx.x; vi < kT * VR; vi += 256) {
    const int t = vi / VR, v = vi % VR;
    *reinterpret_cast<bf16x8*>(dst + t * LD + v * 8) =
        *reinterpret_cast<const bf16x8*>(src + t * gs + v * 8);
  }
}
// The same 64 rows held in registers between their global loads and the LDS
// write (so the loads of the next block can be in flight during a block's
// products).
template <int F>
struct RowRegs {
  static constexpr int RV = kT * F / 8 / 256;
  static_assert(RV >= 1 && RV * 256 * 8 == kT * F, "row split");
  bf16x8 v[RV];
  __device__ __forceinline__ void fetch(const bf16* src, long gs) {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const int vi = threadIdx.x + r * 256, t = vi / (F / 8), c = vi % (F / 8);
      v[r] = *reinterpret_cast<const bf16x8*>(src + t * gs + c * 8);
    }
  }
  template <int LD>
  __device__ __forceinline__ void store(bf16* dst) const {
#pragma unroll
    for (int r = 0; r < RV; ++r) {
      const int vi = threadIdx.x + r * 256, t = vi / (F / 8), c = vi % (F / 8);
      *reinterpret_cast<bf16x8*>(dst + t * LD + c * 8) = v[r];
    }
  }
};
__device__ __forceinline__ float block_sum256(float v, float* sh) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  return sh[0] + sh[1] + sh[2] + sh[3];
}

// Yc[c] (rows n, columns p; stored [p][n] f32) for one (chunk, head,
// batch): wave w owns n blocks, K = the chunk's tokens in 64-token tiles,
// A = (exp(u)·C)ᵀ and B = dy, both by transpose reads.
template <int N, int P>
__global__ __launch_bounds__(256) void k_ssd_bwd_yc(const bf16* __restrict__ C,
                                                    const bf16* __restrict__ dy,
                                                    const float* __restrict__ acum,
                                                    float* __restrict__ Yc, int L, int H, int G,
                                                    int S) {
  constexpr int LDN = N + 16, LDP = P + 16, NNB = N / 16, NPB = P / 16;
  constexpr int NBW = NNB >= 8 ? NNB / 4 : 1, AW = NNB / NBW;
  __shared__ __align__(16) bf16 sC[kT * LDN], sDy[kT * LDP];
  __shared__ __align__(16) float se[kT];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, g = h / (H / G), M = L / S;
  const long pair = (long)b * H + h;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  floatx4 acc[NBW][NPB];
#pragma unroll
  for (int i = 0; i < NBW; ++i)
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb) acc[i][pb] = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int tile = 0; tile < S / kT; ++tile) {
    const long t0 = (long)b * L + (long)c * S + tile * kT;
    __syncthreads();
    stage_rows<N, LDN>(sC, C + (t0 * G + g) * N, (long)G * N);
    stage_rows<P, LDP>(sDy, dy + (t0 * H + h) * P, (long)H * P);
    if (threadIdx.x < kT)
      se[threadIdx.x] = exp_neg(acum[(pair * M + c) * S + tile * kT + threadIdx.x]);
    __syncthreads();
    if (w < AW) {
#pragma unroll
      for (int ks = 0; ks < kT / 32; ++ks) {
        const floatx4 ea = *reinterpret_cast<const floatx4*>(&se[ks * 32 + 4 * grp]);
        const floatx4 eb = *reinterpret_cast<const floatx4*>(&se[ks * 32 + 16 + 4 * grp]);
        bf16x8 bd[NPB];
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb) bd[pb] = tr_frag<LDP>(sDy, ks, pb, col, grp);
#pragma unroll
        for (int i2 = 0; i2 < NBW; ++i2) {
          const bf16x8 a = tr_frag<LDN>(sC, ks, w * NBW + i2, col, grp);
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = to_f32(a[e]) * ea[e];
            v[4 + e] = to_f32(a[4 + e]) * eb[e];
          }
          const bf16x8 ae = pack8f(v);
#pragma unroll
          for (int pb = 0; pb < NPB; ++pb) acc[i2][pb] = Mma<bf16>::mma(ae, bd[pb], acc[i2][pb]);
        }
      }
    }
  }
  if (w < AW) {
    float* out = Yc + (pair * M + c) * (long)(P * N);
#pragma unroll
    for (int i2 = 0; i2 < NBW; ++i2)
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb)
        *reinterpret_cast<floatx4*>(out + (pb * 16 + col) * N + (w * NBW + i2) * 16 + 4 * grp) =
            acc[i2][pb];
  }
}

// Reverse state pass: one thread per 4 state elements (as the forward pass),
// workgroup tile of 1024 elements; the log-decay gradient of each chunk
// end is left as one partial per tile in dus.
__global__ __launch_bounds__(256) void k_ssd_bwd_pass(
    const float* __restrict__ acum, const bf16* __restrict__ H_in, const float* __restrict__ Yc,
    const float* __restrict__ ddH, const float* __restrict__ dhf, bf16* __restrict__ dmem,
    float* __restrict__ dus, float* __restrict__ dh0, int H, int M, int S, int PN) {
  __shared__ float sh[4];
  const int b = blockIdx.z, h = blockIdx.y, e4 = blockIdx.x * 256 + threadIdx.x;
  const long pair = (long)b * H + h;
  floatx4 G = dhf ? *reinterpret_cast<const floatx4*>(dhf + pair * PN + e4 * 4)
                  : floatx4{0.f, 0.f, 0.f, 0.f};
  for (int c = M - 1; c >= 0; --c) {
    const float dec = exp_neg(acum[(pair * M + c) * S + S - 1]);
    const long off = (pair * M + c) * (long)PN + e4 * 4;
    const floatx4 dd =
        ddH ? *reinterpret_cast<const floatx4*>(ddH + off) : floatx4{0.f, 0.f, 0.f, 0.f};
    store4(dmem + off, G + dd);
    const floatx4 hv = load4_f32(H_in + off);
    const float part = dec * (G[0] * hv[0] + G[1] * hv[1] + G[2] * hv[2] + G[3] * hv[3]);
    const float tot = block_sum256(part, sh);
    if (threadIdx.x == 0) dus[(pair * M + c) * gridDim.x + blockIdx.x] = tot;
    G = dec * G + *reinterpret_cast<const floatx4*>(Yc + off);
  }
  *reinterpret_cast<floatx4*>(dh0 + pair * PN + e4 * 4) = G;
}

// Workgroup order of the block kernels: workgroups go to the 8 XCDs
// round-robin by linear index, and the nblk blocks of one (chunk, group,
// batch) unit read each other's token rows.  Units are taken eight at a
// time; block blk of unit 8q + r gets linear index 8·(nblk·q + blk) + r, so
// a unit's blocks share an XCD (and its L2) and follow each other there.
// Units past the last whole group of eight keep a plain order.
__device__ __forceinline__ void unit_block(int nblk, int M, int G, int B, int& c, int& blk,
                                           int& g, int& b) {
  const int lin = blockIdx.x, units = M * G * B;
  const int full = (units / 8) * 8 * nblk;
  int unit;
  if (lin < full) {
    const int q = lin / (8 * nblk), r = lin % (8 * nblk);
    blk = r / 8;
    unit = 8 * q + r % 8;
  } else {
    const int r = lin - full;
    unit = (units / 8) * 8 + r / nblk;
    blk = r % nblk;
  }
  c = unit % M;
  g = (unit / M) % G;
  b = unit / (M * G);
}

// Key-block backward: one workgroup (4 waves) per (64-token block j of
// chunk c, head group, batch); it walks the heads of the group (B, and so
// dB, is shared by them) and wave w owns key columns 16w .. 16w+15.  Per
// head:
//   memory term: BD = dmem[c]ᵀ-products give dx and dB of the keys, scaled
//                by w_j = exp(U_c − u_j)·dt_j, and Σ_p BD·x for dt and u;
//   intra term: for every query block t >= j, the 16×16 tiles cb = C·Bᵀ and
//                dw = dy·xᵀ (rows t), masked decay, then dx += dyᵀ(cb∘dec·dt)
//                and dB += Cᵀ(dw∘dec·dt) with the tiles as B operands.
// dB accumulates over the heads in registers and is written once.
template <int N, int P>
__global__ __launch_bounds__(256, 2) void k_ssd_bwd_j(
    const bf16* __restrict__ x, const float* __restrict__ dt, const bf16* __restrict__ Bm,
    const bf16* __restrict__ C, const bf16* __restrict__ dy, const float* __restrict__ acum,
    const bf16* __restrict__ dmem, float* __restrict__ dx, float* __restrict__ dB,
    float* __restrict__ ddtd, float* __restrict__ duj, float* __restrict__ gwj, int L, int H,
    int G, int S, int nB) {
  constexpr int LDN = N + 16, LDP = P + 16, NKK = N / 32, NK2 = P / 32, NNB = N / 16,
                NPB = P / 16;
  __shared__ __align__(16) bf16 sX[kT * LDP], sB[kT * LDN], sC[kT * LDN], sDy[kT * LDP],
      sD[P * LDN];
  __shared__ __align__(16) float su[kT];
  const int nblk = S / kT, hpg = H / G, M = L / S;
  int c, jb, g, b;
  unit_block(nblk, M, G, nB, c, jb, g, b);
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int jw = 16 * w + col;  // key within the block
  const int jl = jb * kT + jw;  // key within the chunk
  const long rowj = (long)b * L + (long)c * S + jl;
  const long r0j = (long)b * L + (long)c * S + jb * kT;
  stage_rows<N, LDN>(sB, Bm + (r0j * G + g) * N, (long)G * N);
  __syncthreads();
  bf16x8 bj[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    bj[kk] = *reinterpret_cast<const bf16x8*>(&sB[jw * LDN + kk * 32 + grp * 8]);
  floatx4 dBT[NNB];
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) dBT[nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
    const float* ac = acum + (pair * M + c) * S;
    __syncthreads();  // the previous head's reads of sX and sD are done
    stage_rows<P, LDP>(sX, x + (r0j * H + h) * P, (long)H * P);
    {
      const bf16* src = dmem + (pair * M + c) * (long)(P * N);
      for (int vi = threadIdx.x; vi < P * N / 8; vi += 256) {
        const int p = vi / (N / 8), v = vi % (N / 8);
        *reinterpret_cast<bf16x8*>(&sD[p * LDN + v * 8]) =
            *reinterpret_cast<const bf16x8*>(src + p * N + v * 8);
      }
    }
    __syncthreads();
    const float uj = ac[jl], dtj = dt[rowj * H + h], U = ac[S - 1];
    bf16x8 xj[NK2];
#pragma unroll
    for (int k2 = 0; k2 < NK2; ++k2)
      xj[k2] = *reinterpret_cast<const bf16x8*>(&sX[jw * LDP + k2 * 32 + grp * 8]);

    // memory term
    floatx4 dxT[NPB];
    float ddt_mem, gw;
    {
      float s = 0.f;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        floatx4 a4 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          a4 = Mma<bf16>::mma(
              *reinterpret_cast<const bf16x8*>(&sD[(pb * 16 + col) * LDN + kk * 32 + grp * 8]),
              bj[kk], a4);
        const bf16x4 xv = *reinterpret_cast<const bf16x4*>(&sX[jw * LDP + pb * 16 + 4 * grp]);
#pragma unroll
        for (int i = 0; i < 4; ++i) s += a4[i] * to_f32(xv[i]);
        dxT[pb] = a4;
      }
      const float dwi = sum_lane_groups(s);
      const float wd = exp_neg(U - uj), wj = wd * dtj;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) dxT[pb] *= wj;
      ddt_mem = wd * dwi;
      gw = dwi * wj;
#pragma unroll
      for (int nb = 0; nb < NNB; ++nb) {
        floatx4 a4 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k2 = 0; k2 < NK2; ++k2)
          a4 = Mma<bf16>::mma(tr_frag<LDN>(sD, k2, nb, col, grp),
                              row_frag_split(&sX[jw * LDP], k2, grp), a4);
        dBT[nb] += wj * a4;
      }
    }
    // intra term, query blocks t >= j
    float ddt_in = 0.f;
    RowRegs<N> rc;
    RowRegs<P> rd;
    auto fetch_t = [&](int tb) __attribute__((always_inline)) {
      const long r0t = (long)b * L + (long)c * S + tb * kT;
      rc.fetch(C + (r0t * G + g) * N, (long)G * N);
      rd.fetch(dy + (r0t * H + h) * P, (long)H * P);
    };
    fetch_t(jb);
    for (int tb = jb; tb < nblk; ++tb) {
      __syncthreads();
      rc.template store<LDN>(sC);
      rd.template store<LDP>(sDy);
      if (threadIdx.x < kT) su[threadIdx.x] = ac[tb * kT + threadIdx.x];
      __syncthreads();
      if (tb + 1 < nblk) fetch_t(tb + 1);
#pragma unroll
      for (int ks = 0; ks < kT / 32; ++ks) {
        if (tb == jb && 2 * ks + 1 < w) continue;  // every query of the pair precedes the keys
        floatx4 cb[2], dw[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int rb = 2 * ks + r;
          cb[r] = floatx4{0.f, 0.f, 0.f, 0.f};
          dw[r] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk)
            cb[r] = Mma<bf16>::mma(
                *reinterpret_cast<const bf16x8*>(&sC[(16 * rb + col) * LDN + kk * 32 + grp * 8]),
                bj[kk], cb[r]);
#pragma unroll
          for (int k2 = 0; k2 < NK2; ++k2)
            dw[r] = Mma<bf16>::mma(
                *reinterpret_cast<const bf16x8*>(&sDy[(16 * rb + col) * LDP + k2 * 32 + grp * 8]),
                xj[k2], dw[r]);
        }
        float g1[8], g2[8];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tw = 16 * (2 * ks + r) + 4 * grp + i;  // query within the block
            const bool ok = tb > jb || tw >= jw;
            const float dec = ok ? exp_neg(su[tw] - uj) : 0.f;
            const float cd = cb[r][i] * dec, wdc = dw[r][i] * dec;
            g1[4 * r + i] = cd * dtj;
            g2[4 * r + i] = wdc * dtj;
            ddt_in += wdc * cb[r][i];
          }
        const bf16x8 f1 = pack8f(g1), f2 = pack8f(g2);
#pragma unroll
        for (int pb = 0; pb < NPB; ++pb)
          dxT[pb] = Mma<bf16>::mma(tr_frag<LDP>(sDy, ks, pb, col, grp), f1, dxT[pb]);
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb)
          dBT[nb] = Mma<bf16>::mma(tr_frag<LDN>(sC, ks, nb, col, grp), f2, dBT[nb]);
      }
    }
    ddt_in = sum_lane_groups(ddt_in);
#pragma unroll
    for (int pb = 0; pb < NPB; ++pb)
      *reinterpret_cast<floatx4*>(dx + (rowj * H + h) * P + pb * 16 + 4 * grp) = dxT[pb];
    if (grp == 0) {
      ddtd[rowj * H + h] = ddt_mem + ddt_in;
      // Σ_t dw·cb·dec·dt_j: the keys' log-decay enters with a minus
      duj[pair * L + (long)c * S + jl] = -gw - ddt_in * dtj;
      gwj[pair * L + (long)c * S + jl] = gw;
    }
  }
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb)
    *reinterpret_cast<floatx4*>(dB + (rowj * G + g) * N + nb * 16 + 4 * grp) = dBT[nb];
}

// Query-block backward: one workgroup (4 waves) per (64-token block t of
// chunk c, head group, batch); it walks the heads of the group (C, and so
// dC, is shared by them) and wave w owns query columns 16w .. 16w+15.  Per
// head:
//   inter term: dC += exp(u_t)·H_in[c]·dy_t and the log-decay gradient
//               exp(u_t)·dy_t·(C_tᵀH_in[c]);
//   intra term: for every key block j <= t, the tiles cbᵀ = B·Cᵀ and
//               dwᵀ = x·dyᵀ (rows j), masked decay, dC += Bᵀ(dwᵀ∘dec·dt),
//               and the queries' log-decay gradient Σ_j dw·cb·dec·dt.
// dC (plus dC_in, the SMA part, when given) is written once.
template <int N, int P>
__global__ __launch_bounds__(256, 2) void k_ssd_bwd_t(
    const bf16* __restrict__ x, const float* __restrict__ dt, const bf16* __restrict__ Bm,
    const bf16* __restrict__ C, const bf16* __restrict__ dy, const float* __restrict__ acum,
    const bf16* __restrict__ H_in, const float* dC_in, float* dC, float* __restrict__ dut, int L,
    int H, int G, int S, int nB) {
  constexpr int LDN = N + 16, LDP = P + 16, NKK = N / 32, NK2 = P / 32, NNB = N / 16,
                NPB = P / 16;
  __shared__ __align__(16) bf16 sC[kT * LDN], sDy[kT * LDP], sX[kT * LDP], sB[kT * LDN],
      sH[P * LDN];
  __shared__ __align__(16) float su[kT], sdt[kT];
  const int nblk = S / kT, hpg = H / G, M = L / S;
  int c, tb, g, b;
  unit_block(nblk, M, G, nB, c, tb, g, b);
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tw = 16 * w + col;
  const int tl = tb * kT + tw;
  const long rowt = (long)b * L + (long)c * S + tl;
  const long r0t = (long)b * L + (long)c * S + tb * kT;
  stage_rows<N, LDN>(sC, C + (r0t * G + g) * N, (long)G * N);
  __syncthreads();
  bf16x8 ct[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk)
    ct[kk] = *reinterpret_cast<const bf16x8*>(&sC[tw * LDN + kk * 32 + grp * 8]);
  floatx4 dCT[NNB];
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) dCT[nb] = floatx4{0.f, 0.f, 0.f, 0.f};

  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
    const float* ac = acum + (pair * M + c) * S;
    __syncthreads();  // the previous head's reads of sDy and sH are done
    stage_rows<P, LDP>(sDy, dy + (r0t * H + h) * P, (long)H * P);
    {
      const bf16* src = H_in + (pair * M + c) * (long)(P * N);
      for (int vi = threadIdx.x; vi < P * N / 8; vi += 256) {
        const int p = vi / (N / 8), v = vi % (N / 8);
        *reinterpret_cast<bf16x8*>(&sH[p * LDN + v * 8]) =
            *reinterpret_cast<const bf16x8*>(src + p * N + v * 8);
      }
    }
    __syncthreads();
    const float ut = ac[tl], eu = exp_neg(ut);
    bf16x8 dyf[NK2];
#pragma unroll
    for (int k2 = 0; k2 < NK2; ++k2)
      dyf[k2] = *reinterpret_cast<const bf16x8*>(&sDy[tw * LDP + k2 * 32 + grp * 8]);
    // inter term
#pragma unroll
    for (int nb = 0; nb < NNB; ++nb) {
      floatx4 a4 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k2 = 0; k2 < NK2; ++k2)
        a4 = Mma<bf16>::mma(tr_frag<LDN>(sH, k2, nb, col, grp),
                            row_frag_split(&sDy[tw * LDP], k2, grp), a4);
      dCT[nb] += eu * a4;
    }
    float du;
    {
      float s = 0.f;
#pragma unroll
      for (int pb = 0; pb < NPB; ++pb) {
        floatx4 a4 = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          a4 = Mma<bf16>::mma(
              *reinterpret_cast<const bf16x8*>(&sH[(pb * 16 + col) * LDN + kk * 32 + grp * 8]),
              ct[kk], a4);
        const bf16x4 dv = *reinterpret_cast<const bf16x4*>(&sDy[tw * LDP + pb * 16 + 4 * grp]);
#pragma unroll
        for (int i = 0; i < 4; ++i) s += a4[i] * to_f32(dv[i]);
      }
      du = eu * sum_lane_groups(s);
    }
    // intra term, key blocks j <= t
    float du_in = 0.f;
    RowRegs<P> rx;
    RowRegs<N> rb;
    auto fetch_j = [&](int jb) __attribute__((always_inline)) {
      const long r0j = (long)b * L + (long)c * S + jb * kT;
      rx.fetch(x + (r0j * H + h) * P, (long)H * P);
      rb.fetch(Bm + (r0j * G + g) * N, (long)G * N);
    };
    fetch_j(0);
    for (int jb = 0; jb <= tb; ++jb) {
      const long r0j = (long)b * L + (long)c * S + jb * kT;
      __syncthreads();
      rx.template store<LDP>(sX);
      rb.template store<LDN>(sB);
      if (threadIdx.x < kT) {
        su[threadIdx.x] = ac[jb * kT + threadIdx.x];
        sdt[threadIdx.x] = dt[(r0j + threadIdx.x) * H + h];
      }
      __syncthreads();
      if (jb + 1 <= tb) fetch_j(jb + 1);
#pragma unroll
      for (int ks = 0; ks < kT / 32; ++ks) {
        if (jb == tb && 2 * ks > w) continue;  // every key of the pair follows the queries
        floatx4 cb[2], dw[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const int rb = 2 * ks + r;
          cb[r] = floatx4{0.f, 0.f, 0.f, 0.f};
          dw[r] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk)
            cb[r] = Mma<bf16>::mma(
                *reinterpret_cast<const bf16x8*>(&sB[(16 * rb + col) * LDN + kk * 32 + grp * 8]),
                ct[kk], cb[r]);
#pragma unroll
          for (int k2 = 0; k2 < NK2; ++k2)
            dw[r] = Mma<bf16>::mma(
                *reinterpret_cast<const bf16x8*>(&sX[(16 * rb + col) * LDP + k2 * 32 + grp * 8]),
                dyf[k2], dw[r]);
        }
        float g2[8];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int jw = 16 * (2 * ks + r) + 4 * grp + i;  // key within the block
            const bool ok = jb < tb || jw <= tw;
            const float dec = ok ? exp_neg(ut - su[jw]) : 0.f;
            const float v = dw[r][i] * dec * sdt[jw];
            g2[4 * r + i] = v;
            du_in += v * cb[r][i];
          }
        const bf16x8 f2 = pack8f(g2);
#pragma unroll
        for (int nb = 0; nb < NNB; ++nb)
          dCT[nb] = Mma<bf16>::mma(tr_frag<LDN>(sB, ks, nb, col, grp), f2, dCT[nb]);
      }
    }
    du += sum_lane_groups(du_in);
    if (grp == 0) dut[pair * L + (long)c * S + tl] = du;
  }
#pragma unroll
  for (int nb = 0; nb < NNB; ++nb) {
    const long o = (rowt * G + g) * N + nb * 16 + 4 * grp;
    floatx4 v = dCT[nb];
    if (dC_in) v += *reinterpret_cast<const floatx4*>(dC_in + o);
    *reinterpret_cast<floatx4*>(dC + o) = v;
  }
}

// Log-decay gradients of one (chunk, head, batch) -> dt and A: du_t = duj +
// dut (+ at the chunk's last token the memory term's Σ_j gw_j and the state
// pass's partials); ddt_t = direct part + A·Σ_{l>=t} du_l; the dA partial
// is Σ_t du_t·Σ_{l<=t} dt_l.  One thread per token (S <= 256), scans in LDS.
__global__ __launch_bounds__(256) void k_ssd_bwd_fin(
    const float* __restrict__ dt, const float* __restrict__ A, const float* __restrict__ duj,
    const float* __restrict__ dut, const float* __restrict__ gwj, const float* __restrict__ dus,
    const float* __restrict__ ddtd, float* __restrict__ ddt, float* __restrict__ dApart, int L,
    int H, int S, int ntile) {
  __shared__ float sa[256], sb[256], sh[4];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z, M = L / S, i = threadIdx.x;
  const long pair = (long)b * H + h;
  const bool on = i < S;
  const long lt = pair * L + (long)c * S + i;
  const long row = (long)b * L + (long)c * S + i;
  const float gws = block_sum256(on ? gwj[lt] : 0.f, sh);
  float ds = 0.f;
  for (int k = 0; k < ntile; ++k) ds += dus[(pair * M + c) * ntile + k];
  const float du = on ? duj[lt] + dut[lt] + (i == S - 1 ? gws + ds : 0.f) : 0.f;
  const float dtv = on ? dt[row * H + h] : 0.f;
  sa[i] = du;   // suffix sums of du
  sb[i] = dtv;  // prefix sums of dt
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const float va = i + off < 256 ? sa[i + off] : 0.f;
    const float vb = i >= off ? sb[i - off] : 0.f;
    __syncthreads();
    sa[i] += va;
    sb[i] += vb;
    __syncthreads();
  }
  if (on) ddt[row * H + h] = ddtd[row * H + h] + A[h] * sa[i];
  const float part = block_sum256(du * sb[i], sh);
  if (i == 0) dApart[pair * M + c] = part;
}

// dA[h] = Σ_{b, c} dApart[b, h, c]
__global__ __launch_bounds__(256) void k_head_sum(const float* __restrict__ dApart,
                                                  float* __restrict__ dA, int B, int H, int M) {
  __shared__ float sh[4];
  const int h = blockIdx.x;
  float s = 0.f;
  for (int i = threadIdx.x; i < B * M; i += 256) s += dApart[((long)(i / M) * H + h) * M + i % M];
  const float tot = block_sum256(s, sh);
  if (threadIdx.x == 0) dA[h] = tot;
}

struct ScanBwdWs {
  float* Yc;
  bf16* dmem;
  float *dus, *ddtd, *duj, *dut, *gwj, *dApart;
};

ScanBwdWs scan_bwd_ws(void* base, int64_t B, int64_t L, int64_t H, int64_t N, int64_t P,
                      int64_t S, size_t* total) {
  const int64_t M = L / S, PN = P * N, ntile = PN / 1024;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return r;
  };
  ScanBwdWs ws;
  ws.Yc = reinterpret_cast<float*>(take(size_t(B * H * M) * PN * 4));
  ws.dmem = reinterpret_cast<bf16*>(take(size_t(B * H * M) * PN * 2));
  ws.dus = reinterpret_cast<float*>(take(size_t(B * H * M * ntile) * 4));
  ws.ddtd = reinterpret_cast<float*>(take(size_t(B * L * H) * 4));
  ws.duj = reinterpret_cast<float*>(take(size_t(B * L * H) * 4));
  ws.dut = reinterpret_cast<float*>(take(size_t(B * L * H) * 4));
  ws.gwj = reinterpret_cast<float*>(take(size_t(B * L * H) * 4));
  ws.dApart = reinterpret_cast<float*>(take(size_t(B * H * M) * 4));
  if (total) *total = off;
  return ws;
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t N, int64_t P,
                                int64_t S) {
  size_t total = 0;
  scan_bwd_ws(nullptr, B, L, H, N, P, S, &total);
  return total;
}

template <typename T, int N, int P>
hipError_t launch_scan_bwd(const PrefillShape& s, const T* x, const float* dt, const float* A,
                           const T* Bm, const T* C, const float* acum, const T* H_in, const T* dy,
                           const float* ddH, const float* dh_final, const float* dC_sma,
                           float* dx, float* ddt, float* dA, float* dB, float* dC, float* dh0,
                           void* workspace, hipStream_t st) {
  if constexpr (std::is_same<T, float>::value) {
    return launch_scan_bwd_f32<N, P>(s, x, dt, A, Bm, C, acum, H_in, dy, ddH, dh_final, dC_sma,
                                     dx, ddt, dA, dB, dC, dh0, workspace, st);
  } else if constexpr (!std::is_same<T, bf16>::value || P > 64) {
    return hipErrorNotSupported;
  } else {
    const int M = s.L / s.S, PN = P * N, ntile = PN / 1024, nblk = s.S / kT;
    const ScanBwdWs ws = scan_bwd_ws(workspace, s.B, s.L, s.H, N, P, s.S, nullptr);
    hipLaunchKernelGGL((k_ssd_bwd_yc<N, P>), dim3(M, s.H, s.B), dim3(256), 0, st, C, dy, acum,
                       ws.Yc, s.L, s.H, s.G, s.S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_ssd_bwd_pass, dim3(ntile, s.H, s.B), dim3(256), 0, st, acum, H_in,
                       ws.Yc, ddH, dh_final, ws.dmem, ws.dus, dh0, s.H, M, s.S, PN);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const dim3 blocks(M * nblk * s.G * s.B);
    hipLaunchKernelGGL((k_ssd_bwd_j<N, P>), blocks, dim3(256), 0, st, x, dt, Bm, C, dy, acum,
                       ws.dmem, dx, dB, ws.ddtd, ws.duj, ws.gwj, s.L, s.H, s.G, s.S, s.B);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_ssd_bwd_t<N, P>), blocks, dim3(256), 0, st, x, dt, Bm, C, dy, acum,
                       H_in, dC_sma, dC, ws.dut, s.L, s.H, s.G, s.S, s.B);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_ssd_bwd_fin, dim3(M, s.H, s.B), dim3(256), 0, st, dt, A, ws.duj, ws.dut,
                       ws.gwj, ws.dus, ws.ddtd, ddt, ws.dApart, s.L, s.H, s.S, ntile);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_head_sum, dim3(s.H), dim3(256), 0, st, ws.dApart, dA, s.B, s.H, M);
    return hipGetLastError();
  }
}

#define DART_INST_SCAN_BWD(T, N, P)                                                             \
  template hipError_t launch_scan_bwd<T, N, P>(                                                 \
      const PrefillShape&, const T*, const float*, const float*, const T*, const T*,            \
      const float*, const T*, const T*, const float*, const float*, const float*, float*,       \
      float*, float*, float*, float*, float*, void*, hipStream_t);
DART_FOR_EACH_SHAPE(DART_INST_SCAN_BWD)

}  // namespace dart
