// Device-side building blocks for the DART kernels on gfx950 (CDNA4, wave64).
//
// Matrix-core fragments follow the 16x16 MFMA family:
//   v_mfma_f32_16x16x32_bf16 for bfloat16 inputs (K = 32, 8 values per lane)
//   v_mfma_f32_16x16x4_f32   for float32 inputs  (K = 4,  1 value per lane)
// With lane = 16·grp + col (grp in 0..3, col in 0..15):
//   A (16 x K, row-major rows):  lane supplies row `col`, k-slots grp·KL .. +KL
//   B (K x 16):                  lane supplies column `col`, the same k-slots
//   D (16 x 16, fp32):           lane holds D[4·grp + i][col], i = 0..3
// Only the pairing of A's and B's k-slots matters for the sum over K, so a
// kernel may assign any bijection of K indices to (grp, slot) as long as both
// operands use the same one.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dart {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
// e^x for x <= 0 (decays); exp2 of a prescaled argument
__device__ __forceinline__ float exp_neg(float x) { return exp2_fast(x * kLog2e); }

__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v) {
  return static_cast<T>(v);  // bfloat16: round to nearest even
}

template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int K = 32;
  static constexpr int KL = 8;
  typedef bf16x8 frag;
  __device__ __forceinline__ static floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const bf16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
};

template <>
struct Mma<float> {
  static constexpr int K = 4;
  static constexpr int KL = 1;
  typedef float frag;
  __device__ __forceinline__ static floatx4 mma(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const float* p) { return *p; }
};

// four consecutive elements <-> fp32
__device__ __forceinline__ floatx4 load4_f32(const bf16* p) {
  bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
  return floatx4{to_f32(v[0]), to_f32(v[1]), to_f32(v[2]), to_f32(v[3])};
}
__device__ __forceinline__ floatx4 load4_f32(const float* p) {
  return *reinterpret_cast<const floatx4*>(p);
}
__device__ __forceinline__ void store4(bf16* p, floatx4 v) {
  bf16x4 o;
  o[0] = from_f32<bf16>(v[0]);
  o[1] = from_f32<bf16>(v[1]);
  o[2] = from_f32<bf16>(v[2]);
  o[3] = from_f32<bf16>(v[3]);
  *reinterpret_cast<bf16x4*>(p) = o;
}
__device__ __forceinline__ void store4(float* p, floatx4 v) {
  *reinterpret_cast<floatx4*>(p) = v;
}

// 16-byte vector of T and its element count
template <typename T>
struct Vec16 {
  static constexpr int n = 16 / sizeof(T);
  typedef T vec __attribute__((ext_vector_type(16 / sizeof(T))));
};

template <typename T>
__device__ __forceinline__ typename Vec16<T>::vec load16(const T* p) {
  return *reinterpret_cast<const typename Vec16<T>::vec*>(p);
}
template <typename T>
__device__ __forceinline__ typename Vec16<T>::vec load16_nt(const T* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename Vec16<T>::vec*>(p));
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Inside each group of 16
// lanes, lane i receives element i%4 of the 8-byte reads addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4 of the group.  When lane j of a group
// addresses row r0 + j/4, columns c0 + 4·(j%4) .. +3 of a row-major tile,
// lane i therefore receives column c0 + i of rows r0 .. r0+3: four
// consecutive rows of one column, which is the k-run an MFMA operand lane
// supplies when the tile's rows are the contraction axis.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 lds_s4;
  const s4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(const_cast<bf16*>(p)));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

// online-softmax slack: weights may reach 2^kLazyLog2 before the running max
// (and with it every accumulator) is rescaled
constexpr float kLazyLog2 = 8.f;

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

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (lgkmcnt and expcnt left at their maxima).
__host__ __device__ constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Waits that order direct global-to-LDS loads with this wave's own LDS
// accesses; the empty asm keeps the compiler from moving LDS accesses
// across the wait.
template <int IMM>
__device__ __forceinline__ void wait_fence() {
  __builtin_amdgcn_s_waitcnt(IMM);
  asm volatile("" ::: "memory");
}
constexpr int kLgkm0 = 0xC07F;  // lgkmcnt(0)

// Workgroup barrier for LDS hand-offs only: this wave's LDS reads and writes
// are complete, then s_barrier.  Unlike __syncthreads it carries no release
// fence, which would also wait for every direct global-to-LDS load in
// flight (and with it for the memory fetched one step ahead).
// The scheduling barriers keep every instruction (MFMAs included) on its
// side of the workgroup barrier, as schedules that hand work between waves
// at the barrier require.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  wait_fence<kLgkm0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Direct global-to-LDS copies (this lane's 16 or 4 bytes at gptr go to LDS
// byte address lds + 16·lane, resp. lds + 4·lane; lds is wave-uniform),
// issued through inline assembly so that the compiler does not track them:
// it would otherwise wait for every copy in flight before LDS reads it
// cannot tell apart from the copies' targets.  The caller orders them with
// explicit waits (wait_fence<vmcnt_imm(n)>, counting these copies among the
// wave's vector-memory operations) and barriers.  No register receives data.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}
__device__ __forceinline__ void lds_copy16(const void* gptr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void* gptr, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(gptr), "s"(lds)
               : "memory", "m0");
}

}  // namespace dart
