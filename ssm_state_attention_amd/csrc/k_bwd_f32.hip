// Backward of the prefill for f32 io (the small correctness shapes, N and P
// of 16 or 32): plain f32 arithmetic, one thread per token or per state
// element, every sum in a fixed order (no atomics).  The bf16 kernels in
// k_sma_bwd.hip and k_scan_bwd.hip serve the 16-bit shapes.
//
// SMA part (DART abstract: the path is trained end to end; Pith review,
// "What carries the argument": key dH[c]·E_t, value C_tᵀ·dH[c], query Q_t):
// for token t of chunk k and memory c < k, with K = dH[c]·E_t,
// V = dH[c]ᵀ·C_t, s = Q_t·K/sqrt(N), α the softmax weights over c, o the
// readout and do = gate·dy,
//   ds = α·(do·V − do·o),  dQ_t += ds·K/sqrt(N),  dE_t += (ds/sqrt(N))·dH[c]ᵀQ_t,
//   dC_t += α·dH[c]·do_t,  ddH[c] += (ds/sqrt(N))·Q_t E_tᵀ + α·C_t do_tᵀ,
//   dgate = Σ dy·o;  dQ and dC sum over the heads of a group.
// Scan part (Pith review, axiom ledger: the chunked scan's intra- and
// inter-chunk terms, paper Eq. 4, and the state passing): with u the
// in-chunk log-decay acum and U_c its value at the chunk's last token,
//   y_t   = Σ_{j<=t} (C_t·B_j)·e^{u_t−u_j}·dt_j·x_j + e^{u_t}·C_tᵀH_in[k]
//   dH[c] = Σ_i e^{U_c−u_i}·dt_i·B_i x_iᵀ,  H_in[c+1] = e^{U_c}·H_in[c] + dH[c]
// differentiated term by term, the state recursion last chunk first, and
// u = A·(running sum of dt) passing its gradient to dt and A at the end.
#include "dart_launch.hpp"
#include "dart_shapes.hpp"

namespace dart {
namespace {

constexpr int kMaxS = kMaxChunk;

// Sum of v over the workgroup (at most 1024 threads; the last wave may be
// partial, e.g. 32 threads), in a fixed order; the result is valid in
// thread 0.  red holds 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nt = blockDim.x, nw = (nt + 63) >> 6;
  const int active = nt - w * 64 < 64 ? nt - w * 64 : 64;  // lanes of this wave
  for (int off = 32; off > 0; off >>= 1) {
    const float u = __shfl_down(v, off);
    if (lane + off < active) v += u;
  }
  __syncthreads();  // red is free (an earlier call's reads are done)
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x == 0)
    for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// Offset of the factor pair of (token t of the sequence, memory c) in the
// memory-major list of a (batch, head): memory c holds the tokens of
// chunks c+1 .. M-1 in order.
__device__ __forceinline__ long fac_index(long pair, int c, int t, int M, int S) {
  const long per_pair = (long)S * M * (M - 1) / 2;
  const long before = (long)S * ((long)c * (M - 1) - (long)c * (c - 1) / 2);
  return pair * per_pair + before + (t - (long)(c + 1) * S);
}

// SMA, token-major: one workgroup per (chunk k, group g, batch b) with one
// thread per token of the chunk; the group's heads in turn.  Memory c of a
// head is staged in LDS ([p][n]) for the whole chunk.
template <int N, int P>
__global__ __launch_bounds__(kMaxS) void k_sma_bwd_f32_tok(
    const float* __restrict__ Q, const float* __restrict__ E, const float* __restrict__ C,
    const float* __restrict__ dH, const float* __restrict__ o, const float* __restrict__ lse,
    const float* __restrict__ dy, float gate, float* __restrict__ dQ, float* __restrict__ dE,
    float* __restrict__ dC, float2* __restrict__ fac, float* __restrict__ gpart, int L, int H,
    int G, int S, float scale_log2, float rsn) {
  constexpr int PN = P * N;
  __shared__ float mem[PN];
  __shared__ float red[16];
  const int k = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int M = L / S, hpg = H / G, i = threadIdx.x;
  const int ts = k * S + i;                // token in the sequence
  const long row = (long)b * L + ts;       // token row
  float q[N], cv[N], dq[N], dcv[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    q[n] = Q[(row * G + g) * N + n];
    cv[n] = C[(row * G + g) * N + n];
    dq[n] = 0.f;
    dcv[n] = 0.f;
  }
  float gsum = 0.f;
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
    float e[P], dov[P], de[P];
    float D = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const long at = (row * H + h) * P + p;
      e[p] = E[at];
      const float ov = o[at], dyv = dy[at];
      gsum += dyv * ov;
      dov[p] = gate * dyv;
      D += dov[p] * ov;
      de[p] = 0.f;
    }
    const float lse_t = lse[pair * L + ts];
    for (int c = 0; c < k; ++c) {
      __syncthreads();  // every thread is done with the previous memory
      for (int x = i; x < PN; x += S) mem[x] = dH[(pair * M + c) * PN + x];
      __syncthreads();
      float s = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        float kn = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) kn += mem[p * N + n] * e[p];
        s += q[n] * kn;
      }
      const float alpha = exp2f(s * scale_log2 - lse_t);
      float da = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float vp = 0.f;
#pragma unroll
        for (int n = 0; n < N; ++n) vp += cv[n] * mem[p * N + n];
        da += dov[p] * vp;
      }
      const float dsr = alpha * (da - D) * rsn;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        float kn = 0.f, md = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          kn += mem[p * N + n] * e[p];
          md += mem[p * N + n] * dov[p];
        }
        dq[n] += dsr * kn;
        dcv[n] += alpha * md;
      }
#pragma unroll
      for (int p = 0; p < P; ++p) {
        float mq = 0.f;
#pragma unroll
        for (int n = 0; n < N; ++n) mq += mem[p * N + n] * q[n];
        de[p] += dsr * mq;
      }
      fac[fac_index(pair, c, ts, M, S)] = float2{dsr, alpha};
    }
#pragma unroll
    for (int p = 0; p < P; ++p) dE[(row * H + h) * P + p] = de[p];
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    dQ[(row * G + g) * N + n] = dq[n];
    dC[(row * G + g) * N + n] = dcv[n];
  }
  const float tot = block_sum(gsum, red);
  if (i == 0) gpart[((long)b * G + g) * M + k] = tot;
}

// SMA, memory-major: one workgroup per (memory c, head h, batch b), one
// thread per element (p, n) of ddH[c], summing over the later tokens with
// the token kernel's factors.
template <int N, int P>
__global__ __launch_bounds__(1024) void k_sma_bwd_f32_mem(
    const float* __restrict__ Q, const float* __restrict__ E, const float* __restrict__ C,
    const float* __restrict__ dy, float gate, const float2* __restrict__ fac,
    float* __restrict__ ddH, int L, int H, int G, int S) {
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int M = L / S, g = h / (H / G);
  const long pair = (long)b * H + h;
  const int p = threadIdx.x / N, n = threadIdx.x % N;
  float acc = 0.f;
  for (int ts = (c + 1) * S; ts < L; ++ts) {
    const long row = (long)b * L + ts;
    const float2 f = fac[fac_index(pair, c, ts, M, S)];
    acc += f.x * Q[(row * G + g) * N + n] * E[(row * H + h) * P + p] +
           f.y * C[(row * G + g) * N + n] * (gate * dy[(row * H + h) * P + p]);
  }
  ddH[(pair * M + c) * (P * N) + p * N + n] = acc;
}

// Fixed-order sum of n partials into *out (one workgroup of 256).
__global__ __launch_bounds__(256) void k_sum_f32(const float* __restrict__ part, long n,
                                                 float* __restrict__ out) {
  __shared__ float red[16];
  float s = 0.f;
  for (long i = threadIdx.x; i < n; i += 256) s += part[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) *out = s;
}

// Scan, intra- and inter-chunk terms: one workgroup per (chunk k, group g,
// batch b), one thread per token; the group's heads in turn.  Writes dx,
// ddt, du (first writer of each), dHin[k] = ∂/∂H_in[k] through the outputs,
// and after the heads dB (intra part) and dC (+ dC_sma).
template <int N, int P>
__global__ __launch_bounds__(kMaxS) void k_ssd_bwd_f32_chunk(
    const float* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ Bm,
    const float* __restrict__ C, const float* __restrict__ acum, const float* __restrict__ H_in,
    const float* __restrict__ dy, const float* dC_sma, float* __restrict__ dx,
    float* __restrict__ ddt, float* __restrict__ dB, float* dC, float* __restrict__ du,
    float* __restrict__ dHin, int L, int H, int G, int S) {
  constexpr int PN = P * N;
  __shared__ float sB[kMaxS * N], sC[kMaxS * N], sX[kMaxS * P], sY[kMaxS * P];
  __shared__ float sU[kMaxS], sDt[kMaxS], sH[PN];
  const int k = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int M = L / S, hpg = H / G, i = threadIdx.x;
  const long row = (long)b * L + k * S + i;
  float bi[N], db[N], dcv[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    bi[n] = Bm[(row * G + g) * N + n];
    sB[i * N + n] = bi[n];
    sC[i * N + n] = C[(row * G + g) * N + n];
    db[n] = 0.f;
    dcv[n] = 0.f;
  }
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
    __syncthreads();  // the previous head is done with the head's LDS rows
    float xi[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      xi[p] = x[(row * H + h) * P + p];
      sX[i * P + p] = xi[p];
      sY[i * P + p] = dy[(row * H + h) * P + p];
    }
    sU[i] = acum[(pair * M + k) * S + i];
    sDt[i] = dt[row * H + h];
    for (int e = i; e < PN; e += S) sH[e] = H_in[(pair * M + k) * PN + e];
    __syncthreads();
    const float ui = sU[i], dti = sDt[i];
    // token i as the key j of the pairs (t >= i)
    float dxv[P];
#pragma unroll
    for (int p = 0; p < P; ++p) dxv[p] = 0.f;
    float ddt_i = 0.f, du_i = 0.f;
    for (int t = i; t < S; ++t) {
      const float w = __expf(sU[t] - ui);
      float cb = 0.f, dyx = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) cb += sC[t * N + n] * bi[n];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        dyx += sY[t * P + p] * xi[p];
        dxv[p] += cb * w * sY[t * P + p];
      }
      const float dcb = dyx * w * dti;
#pragma unroll
      for (int n = 0; n < N; ++n) db[n] += dcb * sC[t * N + n];
      ddt_i += dyx * cb * w;
      du_i -= dyx * cb * dti * w;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) dx[(row * H + h) * P + p] = dti * dxv[p];
    // token i as the query t of the pairs (j <= i)
    float yi[P], ci[N];
#pragma unroll
    for (int p = 0; p < P; ++p) yi[p] = sY[i * P + p];
#pragma unroll
    for (int n = 0; n < N; ++n) ci[n] = sC[i * N + n];
    for (int j = 0; j <= i; ++j) {
      const float w = __expf(ui - sU[j]);
      float cb = 0.f, dyx = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) cb += ci[n] * sB[j * N + n];
#pragma unroll
      for (int p = 0; p < P; ++p) dyx += yi[p] * sX[j * P + p];
      const float dcb = dyx * w * sDt[j];
#pragma unroll
      for (int n = 0; n < N; ++n) dcv[n] += dcb * sB[j * N + n];
      du_i += dyx * cb * sDt[j] * w;
    }
    // inter-chunk term: e^{u_i}·C_iᵀH_in[k] (H_in rows [p][n])
    const float eu = __expf(ui);
    float chy = 0.f;
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float hy = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) hy += sH[p * N + n] * yi[p];
      dcv[n] += eu * hy;
      chy += ci[n] * hy;
    }
    du_i += eu * chy;
    ddt[row * H + h] = ddt_i;
    du[pair * L + k * S + i] = du_i;
    // dHin[k][p][n] = Σ_t e^{u_t}·C_t[n]·dy_t[p]
    for (int e = i; e < PN; e += S) {
      const int p = e / N, n = e % N;
      float a = 0.f;
      for (int t = 0; t < S; ++t) a += __expf(sU[t]) * sC[t * N + n] * sY[t * P + p];
      dHin[(pair * M + k) * PN + e] = a;
    }
  }
#pragma unroll
  for (int n = 0; n < N; ++n) {
    const long at = (row * G + g) * N + n;
    dB[at] = db[n];
    dC[at] = dcv[n] + (dC_sma ? dC_sma[at] : 0.f);
  }
}

// Scan, reverse state pass: one workgroup per (batch, head), one thread per
// state element.  dmem[c] = G + ddH[c] with G the gradient of H_in[c+1];
// the chunk-end log-decay gradient Σ G·e^{U_c}·H_in[c] goes to du.
template <int N, int P>
__global__ __launch_bounds__(1024) void k_ssd_bwd_f32_pass(
    const float* __restrict__ acum, const float* __restrict__ H_in,
    const float* __restrict__ ddH, const float* __restrict__ dh_final,
    const float* __restrict__ dHin, float* __restrict__ dmem, float* __restrict__ du,
    float* __restrict__ dh0, int L, int S) {
  constexpr int PN = P * N;
  __shared__ float red[16];
  const long pair = blockIdx.x;
  const int M = L / S, e = threadIdx.x;
  float Gs = dh_final ? dh_final[pair * PN + e] : 0.f;
  for (int c = M - 1; c >= 0; --c) {
    const long at = (pair * M + c) * PN + e;
    dmem[at] = Gs + (ddH ? ddH[at] : 0.f);
    const float eU = __expf(acum[(pair * M + c) * S + S - 1]);
    const float v = block_sum(Gs * eU * H_in[at], red);
    if (e == 0) du[pair * L + c * S + S - 1] += v;
    Gs = eU * Gs + dHin[at];
  }
  dh0[pair * PN + e] = Gs;
}

// Scan, chunk-memory terms: one workgroup per (chunk k, group g, batch b),
// one thread per token; the group's heads in turn.  Adds to dx, ddt, du and
// (after the heads) dB.
template <int N, int P>
__global__ __launch_bounds__(kMaxS) void k_ssd_bwd_f32_mem(
    const float* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ Bm,
    const float* __restrict__ acum, const float* __restrict__ dmem, float* __restrict__ dx,
    float* __restrict__ ddt, float* __restrict__ dB, float* __restrict__ du, int L, int H,
    int G, int S) {
  constexpr int PN = P * N;
  __shared__ float sD[PN];
  __shared__ float red[16];
  const int k = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int M = L / S, hpg = H / G, i = threadIdx.x;
  const long row = (long)b * L + k * S + i;
  float bi[N], db[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    bi[n] = Bm[(row * G + g) * N + n];
    db[n] = 0.f;
  }
  for (int hh = 0; hh < hpg; ++hh) {
    const int h = g * hpg + hh;
    const long pair = (long)b * H + h;
    __syncthreads();
    for (int e = i; e < PN; e += S) sD[e] = dmem[(pair * M + k) * PN + e];
    __syncthreads();
    const float ui = acum[(pair * M + k) * S + i], U = acum[(pair * M + k) * S + S - 1];
    const float wd = __expf(U - ui), dti = dt[row * H + h];
    float xi[P];
#pragma unroll
    for (int p = 0; p < P; ++p) xi[p] = x[(row * H + h) * P + p];
    float dwi = 0.f;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      float bm = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) bm += bi[n] * sD[p * N + n];
      dx[(row * H + h) * P + p] += wd * dti * bm;
      dwi += bm * xi[p];
    }
#pragma unroll
    for (int n = 0; n < N; ++n) {
      float mx = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) mx += sD[p * N + n] * xi[p];
      db[n] += wd * dti * mx;
    }
    ddt[row * H + h] += wd * dwi;
    const float gw = dwi * wd * dti;
    du[pair * L + k * S + i] -= gw;
    const float tot = block_sum(gw, red);  // its barriers order the du updates
    if (i == 0) du[pair * L + k * S + S - 1] += tot;
  }
#pragma unroll
  for (int n = 0; n < N; ++n) dB[(row * G + g) * N + n] += db[n];
}

// Scan, log-decay gradients: u_t = A·Σ_{l<=t in chunk} dt_l, so
// ddt_t += A·Σ_{l>=t} du_l and dA += Σ_t du_t·Σ_{l<=t} dt_l (per chunk
// partials).  One workgroup per (chunk k, head h, batch b), one thread per
// token.
__global__ __launch_bounds__(kMaxS) void k_ssd_bwd_f32_fin(
    const float* __restrict__ dt, const float* __restrict__ A, const float* __restrict__ du,
    float* __restrict__ ddt, float* __restrict__ dApart, int L, int H, int S) {
  __shared__ float sdu[kMaxS], sdt[kMaxS];
  __shared__ float red[16];
  const int k = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int M = L / S, i = threadIdx.x;
  const long pair = (long)b * H + h;
  const long row = (long)b * L + k * S + i;
  sdu[i] = du[pair * L + k * S + i];
  sdt[i] = dt[row * H + h];
  __syncthreads();
  float rc = 0.f, cs = 0.f;
  for (int l = S - 1; l >= i; --l) rc += sdu[l];
  for (int l = 0; l <= i; ++l) cs += sdt[l];
  ddt[row * H + h] += A[h] * rc;
  const float tot = block_sum(sdu[i] * cs, red);
  if (i == 0) dApart[pair * M + k] = tot;
}

// dA[h] = Σ_b Σ_k dApart[b, h, k] in a fixed order.
__global__ __launch_bounds__(256) void k_dA_f32(const float* __restrict__ dApart,
                                                float* __restrict__ dA, int B, int H, int M) {
  __shared__ float red[16];
  const int h = blockIdx.x;
  float s = 0.f;
  for (long i = threadIdx.x; i < (long)B * M; i += 256) {
    const long b = i / M, k = i % M;
    s += dApart[(b * H + h) * M + k];
  }
  s = block_sum(s, red);
  if (threadIdx.x == 0) dA[h] = s;
}

size_t pad256(size_t bytes) { return (bytes + 255) / 256 * 256; }

}  // namespace

size_t sma_bwd_f32_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t G, int64_t S) {
  const size_t M = static_cast<size_t>(L / S);
  return pad256(static_cast<size_t>(B * G) * M * sizeof(float)) +  // dgate partials
         static_cast<size_t>(B * H * S) * (M * (M - 1) / 2) * sizeof(float2);
}

size_t scan_bwd_f32_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t N, int64_t P,
                                    int64_t S) {
  const size_t pairs = static_cast<size_t>(B * H), M = static_cast<size_t>(L / S);
  const size_t PN = static_cast<size_t>(N * P);
  return pad256(pairs * L * 4) + 2 * pad256(pairs * M * PN * 4) + pad256(pairs * M * 4);
}

template <int N, int P>
hipError_t launch_sma_bwd_f32(const PrefillShape& s, const float* Q, const float* E,
                              const float* C, const float* dH, const float* o, const float* lse,
                              const float* dy, float gate, float* dQ, float* dE, float* dC,
                              float* ddH, float* dgate, void* workspace, hipStream_t st) {
  static_assert(N * P <= 1024, "one thread per memory element");
  const int M = s.L / s.S;
  float* gpart = static_cast<float*>(workspace);
  float2* fac = reinterpret_cast<float2*>(
      static_cast<char*>(workspace) + pad256(static_cast<size_t>(s.B) * s.G * M * sizeof(float)));
  const float scale_log2 = kLog2e / sqrtf(static_cast<float>(N));
  const float rsn = 1.f / sqrtf(static_cast<float>(N));
  hipLaunchKernelGGL((k_sma_bwd_f32_tok<N, P>), dim3(M, s.G, s.B), dim3(s.S), 0, st, Q, E, C, dH,
                     o, lse, dy, gate, dQ, dE, dC, fac, gpart, s.L, s.H, s.G, s.S, scale_log2,
                     rsn);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_sma_bwd_f32_mem<N, P>), dim3(M, s.H, s.B), dim3(N * P), 0, st, Q, E, C,
                     dy, gate, fac, ddH, s.L, s.H, s.G, s.S);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_sum_f32, dim3(1), dim3(256), 0, st, gpart, (long)s.B * s.G * M, dgate);
  return hipGetLastError();
}

template <int N, int P>
hipError_t launch_scan_bwd_f32(const PrefillShape& s, const float* x, const float* dt,
                               const float* A, const float* Bm, const float* C,
                               const float* acum, const float* H_in, const float* dy,
                               const float* ddH, const float* dh_final, const float* dC_sma,
                               float* dx, float* ddt, float* dA, float* dB, float* dC,
                               float* dh0, void* workspace, hipStream_t st) {
  static_assert(N * P <= 1024 && N * P % 64 == 0, "one thread per state element");
  const int M = s.L / s.S;
  const size_t pairs = static_cast<size_t>(s.B) * s.H, PN = static_cast<size_t>(N) * P;
  char* w = static_cast<char*>(workspace);
  float* du = reinterpret_cast<float*>(w);
  w += pad256(pairs * s.L * 4);
  float* dHin = reinterpret_cast<float*>(w);
  w += pad256(pairs * M * PN * 4);
  float* dmem = reinterpret_cast<float*>(w);
  w += pad256(pairs * M * PN * 4);
  float* dApart = reinterpret_cast<float*>(w);
  hipLaunchKernelGGL((k_ssd_bwd_f32_chunk<N, P>), dim3(M, s.G, s.B), dim3(s.S), 0, st, x, dt, Bm,
                     C, acum, H_in, dy, dC_sma, dx, ddt, dB, dC, du, dHin, s.L, s.H, s.G, s.S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_ssd_bwd_f32_pass<N, P>), dim3(pairs), dim3(N * P), 0, st, acum, H_in,
                     ddH, dh_final, dHin, dmem, du, dh0, s.L, s.S);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((k_ssd_bwd_f32_mem<N, P>), dim3(M, s.G, s.B), dim3(s.S), 0, st, x, dt, Bm,
                     acum, dmem, dx, ddt, dB, du, s.L, s.H, s.G, s.S);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_ssd_bwd_f32_fin, dim3(M, s.H, s.B), dim3(s.S), 0, st, dt, A, du, ddt,
                     dApart, s.L, s.H, s.S);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(k_dA_f32, dim3(s.H), dim3(256), 0, st, dApart, dA, s.B, s.H, M);
  return hipGetLastError();
}

template hipError_t launch_sma_bwd_f32<16, 16>(const PrefillShape&, const float*, const float*,
                                               const float*, const float*, const float*,
                                               const float*, const float*, float, float*, float*,
                                               float*, float*, float*, void*, hipStream_t);
template hipError_t launch_sma_bwd_f32<32, 32>(const PrefillShape&, const float*, const float*,
                                               const float*, const float*, const float*,
                                               const float*, const float*, float, float*, float*,
                                               float*, float*, float*, void*, hipStream_t);
template hipError_t launch_scan_bwd_f32<16, 16>(const PrefillShape&, const float*, const float*,
                                                const float*, const float*, const float*,
                                                const float*, const float*, const float*,
                                                const float*, const float*, const float*, float*,
                                                float*, float*, float*, float*, float*, void*,
                                                hipStream_t);
template hipError_t launch_scan_bwd_f32<32, 32>(const PrefillShape&, const float*, const float*,
                                                const float*, const float*, const float*,
                                                const float*, const float*, const float*,
                                                const float*, const float*, const float*, float*,
                                                float*, float*, float*, float*, float*, void*,
                                                hipStream_t);

}  // namespace dart
