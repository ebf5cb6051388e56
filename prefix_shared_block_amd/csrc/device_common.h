// device_common.h -- small device helpers shared by the gfx950 kernels:
// vector types, exp2/log2 on the hardware units, cross-lane swaps and the
// exact OCP e4m3fn -> bf16 conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// finite stand-in for -inf as the initial running maximum, so that a row whose
// first tile is fully masked gives exp2(-inf - (-1e30)) = 0, never NaN
constexpr float kNegBig = -1.0e30f;

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

template <int DT>
struct Elem;
template <>
struct Elem<DT_F32> {
  static constexpr int size = 4;
};
template <>
struct Elem<DT_BF16> {
  static constexpr int size = 2;
};
template <>
struct Elem<DT_FP8> {
  static constexpr int size = 1;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// value of the lane l ^ 32 (the other half of the wave, same query column)
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// two OCP e4m3fn codes (the low or high 16 bits of w) -> two bf16 (exact)
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  auto r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// 16 fp8 codes -> 16 bf16 (two 16-byte chunks)
__device__ __forceinline__ void fp8x16_to_bf16(const u32x4_t in, u32x4_t& lo, u32x4_t& hi) {
  lo[0] = fp8x2_to_bf16x2<false>(in[0]);
  lo[1] = fp8x2_to_bf16x2<true>(in[0]);
  lo[2] = fp8x2_to_bf16x2<false>(in[1]);
  lo[3] = fp8x2_to_bf16x2<true>(in[1]);
  hi[0] = fp8x2_to_bf16x2<false>(in[2]);
  hi[1] = fp8x2_to_bf16x2<true>(in[2]);
  hi[2] = fp8x2_to_bf16x2<false>(in[3]);
  hi[3] = fp8x2_to_bf16x2<true>(in[3]);
}

__device__ __forceinline__ uint32_t half_of(const u32x4_t& x, int e) {
  // 16-bit element e (0..7) of an 8 x 16-bit chunk
  return (x[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
}

template <int DT>
__device__ __forceinline__ float load_elem(const void* base, size_t idx) {
  if constexpr (DT == DT_F32) {
    return reinterpret_cast<const float*>(base)[idx];
  } else if constexpr (DT == DT_BF16) {
    uint32_t u = reinterpret_cast<const uint16_t*>(base)[idx];
    return __builtin_bit_cast(float, u << 16);
  } else {
    uint32_t u = reinterpret_cast<const uint8_t*>(base)[idx];
    uint32_t w = fp8x2_to_bf16x2<false>(u) & 0xFFFFu;
    return __builtin_bit_cast(float, w << 16);
  }
}

// LDS byte address of a __shared__ object (32-bit, as the DS and M0 forms take)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave-wide 16-byte-per-lane copy global -> LDS: lane l's 16 bytes land
// at LDS address lds + 16 * l.  Issued in asm so that the compiler does not
// fence every later LDS read on it; completion is awaited with wait_vmcnt.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

// The same copy with a wave-uniform 64-bit base in scalar registers and a
// 32-bit per-lane byte offset (the saddr form: no 64-bit address arithmetic
// per lane).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Cross-row swaps of gfx950 (v_permlane16_swap / v_permlane32_swap) used to
// reach lane l ^ 16 / l ^ 32: called with the same value in both operands the
// instruction returns (own, partner) in some order, so max(r[0], r[1]) is the
// pair's maximum.  The two results are copied into scalars before the bit
// cast: a bit cast applied to an element of a vector value reads element 0.
__device__ __forceinline__ float max_xor32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}
__device__ __forceinline__ float max_xor16(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t r0 = r[0], r1 = r[1];
  return fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

}  // namespace psattn
