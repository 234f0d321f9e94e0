// Device pieces shared by the evenly split decode (paged_attn_sk.hip) and the prefix-shared
// decode (paged_attn_prefix.hip): tile constants, the MFMA wrappers for one 16-token tile, the
// cross-lane reductions of its 4 x 16 layout, buffer-descriptor constants and the packed store.
#pragma once

#include <hip/hip_runtime.h>

#include "dtypes.h"

namespace pkv {
namespace sk {
namespace {

constexpr int kTile = 16;                 // tokens per tile (one MFMA row block)
constexpr float kNegBig = -1.0e30f;
constexpr float kTau = 8.0f;              // lazy-rescale threshold (log2 units)
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // buffer descriptor dword 3 for gfx9-class parts

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

template <typename T> struct Mma;
template <> struct Mma<BF16> {
  using v8 = bf16x8;
  __device__ static f32x4 qk(v8 a, v8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
  __device__ static f32x4 pv(i16x4_t a, i16x4_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
  __device__ static short pack(float x) { return __builtin_bit_cast(short, static_cast<__bf16>(x)); }
  __device__ static float unpack(short x) { return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(x)) << 16); }
};
template <> struct Mma<F16> {
  using v8 = f16x8;
  __device__ static f32x4 qk(v8 a, v8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }
  __device__ static f32x4 pv(i16x4_t a, i16x4_t b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  }
  __device__ static short pack(float x) { return __builtin_bit_cast(short, static_cast<_Float16>(x)); }
  __device__ static float unpack(short x) { return static_cast<float>(__builtin_bit_cast(_Float16, x)); }
};

__device__ __forceinline__ float swap16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum / max over the 16 lanes of each lane row (lanes 16j .. 16j+15), in every lane of the row:
// quad swaps, then the half-row and row mirrors (DPP, no LDS).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  return x + dpp<0x140>(x);  // row_mirror
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  return fmaxf(x, dpp<0x140>(x));
}

// Dot product of two 16-byte vectors of 8 elements, accumulated into c in fp32 (v_dot2c).  The
// pairs are taken as elements of the whole 8-element vector: bit-casting single 32-bit lanes of
// a u32x4 to 2-element vectors was compiled to four products of lane 0.
__device__ __forceinline__ float dot8(BF16, u32x4 a, u32x4 b, float c) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
  c = __builtin_amdgcn_fdot2_f32_bf16(x.s01, y.s01, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(x.s23, y.s23, c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(x.s45, y.s45, c, false);
  return __builtin_amdgcn_fdot2_f32_bf16(x.s67, y.s67, c, false);
}
__device__ __forceinline__ float dot8(F16, u32x4 a, u32x4 b, float c) {
  const f16x8 x = __builtin_bit_cast(f16x8, a), y = __builtin_bit_cast(f16x8, b);
  c = __builtin_amdgcn_fdot2(x.s01, y.s01, c, false);
  c = __builtin_amdgcn_fdot2(x.s23, y.s23, c, false);
  c = __builtin_amdgcn_fdot2(x.s45, y.s45, c, false);
  return __builtin_amdgcn_fdot2(x.s67, y.s67, c, false);
}

// Orders one wave's LDS writes before its own later LDS reads (and vice versa).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ int lane_val(int v, int i) { return __builtin_amdgcn_readlane(v, i); }

// Stores 4 fp32 values rounded to the element type as one 8-byte write.  Results and records
// are written with the non-temporal hint (they are not read again by this launch's waves), which
// keeps them from displacing K/V lines in L2.
template <typename T>
__device__ __forceinline__ void store4(typename T::raw* dst, f32x4 v) {
  uint2 w;
  w.x = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_raw(T{}, v[0]))) |
        (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_raw(T{}, v[1]))) << 16);
  w.y = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_raw(T{}, v[2]))) |
        (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, to_raw(T{}, v[3]))) << 16);
  __builtin_nontemporal_store(static_cast<unsigned long long>(w.x) | (static_cast<unsigned long long>(w.y) << 32),
                              reinterpret_cast<unsigned long long*>(dst));
}

// Range (within one KV head's list of n tiles cut into R equal ranges) whose tiles include
// tile t: the largest r with r*n/R <= t.
__device__ __forceinline__ int range_of(int t, int n, int R) {
  return static_cast<int>(((static_cast<int64_t>(t) + 1) * R - 1) / n);
}

// LDS row pitch of a K/V tile: the transposing V reads of one MFMA hit distinct banks.
__host__ __device__ constexpr int sk_pitch(int D) { return D == 128 ? 288 : 160; }

}  // namespace
}  // namespace sk
}  // namespace pkv
