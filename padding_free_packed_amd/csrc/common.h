// Shared device helpers for the gfx950 kernels: vector types, the 16-bit
// element types (bf16 and fp16) with their bit conversions and MFMA, wave
// reductions and the XCD-aware block mapping.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pe {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

// Element types of the kernels: float, or a 16-bit type (__bf16, _Float16)
// stored as raw uint16_t in memory and LDS and computed on by MFMA with fp32
// accumulation.
template <typename T>
constexpr bool kIs16 = !std::is_same<T, float>::value;

template <typename T>
struct Vec8Of;
template <>
struct Vec8Of<__bf16> { using type = bf16x8; };
template <>
struct Vec8Of<_Float16> { using type = f16x8; };
// eight 16-bit elements: one MFMA A or B operand of a 32x32x16 product
template <typename T>
using vec8 = typename Vec8Of<T>::type;

template <typename T>
__device__ __forceinline__ vec8<T> as_vec8(u16x8 x) { return __builtin_bit_cast(vec8<T>, x); }

// acc + A . B over 16 reduction elements (v_mfma_f32_32x32x16_{bf16,f16})
template <typename T>
__device__ __forceinline__ floatx16 mfma16(vec8<T> a, vec8<T> b, floatx16 acc) {
  if constexpr (std::is_same<T, __bf16>::value) return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}

// 16-bit pattern -> float (exact)
template <typename T>
__device__ __forceinline__ float h16_to_f32(uint16_t b) {
  if constexpr (std::is_same<T, __bf16>::value) return __uint_as_float(static_cast<uint32_t>(b) << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, b));
}

// float -> 16-bit pattern, round to nearest, ties to even (the hardware conversion)
template <typename T>
__device__ __forceinline__ uint16_t f32_to_h16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<T>(f));
}

// Store with the non-temporal hint (streaming writes of copies that no later
// kernel step reads back from the caches); U is a 1-16 byte unit.
template <typename U>
__device__ __forceinline__ void st_nt(U* p, const U& v) {
  if constexpr (sizeof(U) == 16) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(__builtin_bit_cast(u4, v), reinterpret_cast<u4*>(p));
  } else if constexpr (sizeof(U) == 8) {
    typedef unsigned int u2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(__builtin_bit_cast(u2, v), reinterpret_cast<u2*>(p));
  } else {
    __builtin_nontemporal_store(v, p);
  }
}

// smallest power of two >= x (x >= 1)
constexpr int pow2_ceil(int x) { return x <= 1 ? 1 : 2 * pow2_ceil((x + 1) / 2); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for minus infinity as the running maximum, so that
// exp2(m_old - m_new) never evaluates inf - inf.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float wave_max32(float x) {
  // maximum over the 32 lanes of each half wave
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = min(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Workgroups of one launch are handed to the 8 XCDs in round-robin order of
// their block index. This remaps block indices so that XCD x receives one
// contiguous range of logical work items; neighbouring items (the tiles of one
// sequence and head) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int x = bid & 7, i = bid >> 3;
  const int per = nblocks >> 3, rem = nblocks & 7;
  return x * per + min(x, rem) + i;
}

}  // namespace pe
