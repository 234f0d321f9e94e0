// Element-type helpers for the device code: raw storage types, 16-byte vector unpacking
// and rounding back to storage.  bf16 is handled as its raw 16-bit pattern.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pkv {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

struct F32 {
  using raw = float;
  static constexpr int kBytes = 4;
};
struct F16 {
  using raw = _Float16;
  static constexpr int kBytes = 2;
};
struct BF16 {
  using raw = uint16_t;
  static constexpr int kBytes = 2;
};

// Elements held by one 16-byte vector.
template <typename T>
constexpr int kVecElems = 16 / T::kBytes;

// Unpack a 16-byte vector into fp32 (exact widening).
__device__ __forceinline__ void unpack(F32, const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}
__device__ __forceinline__ void unpack(F16, const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    f[2 * i] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xffffu)));
    f[2 * i + 1] = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
  }
}
__device__ __forceinline__ void unpack(BF16, const u32x4& v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    f[2 * i] = __uint_as_float(w << 16);
    f[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
  }
}

// Round fp32 to the storage type, round-to-nearest-even.
__device__ __forceinline__ float to_raw(F32, float x) { return x; }
__device__ __forceinline__ _Float16 to_raw(F16, float x) { return static_cast<_Float16>(x); }
__device__ __forceinline__ uint16_t to_raw(BF16, float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Widen one stored element to fp32.
__device__ __forceinline__ float to_f32(F32, float x) { return x; }
__device__ __forceinline__ float to_f32(F16, _Float16 x) { return static_cast<float>(x); }
__device__ __forceinline__ float to_f32(BF16, uint16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

}  // namespace pkv
