// Shared device helpers for the gfx950 kernels of the MC2 compute core.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mc2 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Storage element kinds handled by the contraction kernels.
enum class Elem : int { F16 = 0, BF16 = 1, I8 = 2 };

// Output kinds written by the epilogues.
enum class Out : int { F16 = 0, BF16 = 1, F32 = 3, I32 = 4 };

template <Elem E> struct ElemInfo;
template <> struct ElemInfo<Elem::F16> { static constexpr int bytes = 2; };
template <> struct ElemInfo<Elem::BF16> { static constexpr int bytes = 2; };
template <> struct ElemInfo<Elem::I8> { static constexpr int bytes = 1; };

template <Out O> struct OutInfo;
template <> struct OutInfo<Out::F16> { static constexpr int bytes = 2; };
template <> struct OutInfo<Out::BF16> { static constexpr int bytes = 2; };
template <> struct OutInfo<Out::F32> { static constexpr int bytes = 4; };
template <> struct OutInfo<Out::I32> { static constexpr int bytes = 4; };

template <class To, class From>
__device__ __forceinline__ To bit_cast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, f);
}

// float -> 16-bit storage, round to nearest even (the language conversions
// are RNE; on gfx950 they map to the hardware converts).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
  return bit_cast<uint16_t>(static_cast<__bf16>(v));
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float v) {
  return bit_cast<uint16_t>(static_cast<_Float16>(v));
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}
__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return static_cast<float>(bit_cast<_Float16>(static_cast<uint16_t>(b)));
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }
__device__ __forceinline__ u32x4_t zero_v4() { return u32x4_t{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ void atomic_or_err(int32_t* dev_err, uint32_t bit) {
  if (dev_err) atomicOr(dev_err, static_cast<int32_t>(bit));
}

}  // namespace mc2
