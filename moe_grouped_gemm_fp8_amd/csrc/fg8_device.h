// Device helpers shared by the fg8 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr float kE4m3Max = 448.f;
constexpr int kGroup = 128;      // K block of the FP32 scales and of one MFMA
constexpr int kMxBlock = 32;     // elements sharing one E8M0 exponent

// Two floats -> two e4m3 codes in the low 16 bits.  v_cvt_pk_fp8_f32 rounds
// to nearest even and keeps the sign of zero but turns out-of-range values
// into NaN, so inputs are clamped to +-448 first (saturating encode).
__device__ __forceinline__ uint32_t cvt2_e4m3(float a, float b) {
  a = fminf(fmaxf(a, -kE4m3Max), kE4m3Max);
  b = fminf(fmaxf(b, -kE4m3Max), kE4m3Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t pack4_e4m3(float4 v) {
  return cvt2_e4m3(v.x, v.y) | (cvt2_e4m3(v.z, v.w) << 16);
}

// Round-to-nearest-even FP32 -> BF16 bits.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return 0x7FC0;  // NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Maximum over the lanes of one aligned group of `width` lanes (power of two
// <= 64), using butterfly exchanges; every lane of the group gets the result.
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float abs_max4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Sixteen bytes of a row as FP32: four floats, or eight BF16 values (raw
// 16-bit words) widened exactly.
template <class T>
struct RowVec;
template <>
struct RowVec<float> {
  static constexpr int kElems = 4;
  __device__ static void widen(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
};
template <>
struct RowVec<uint16_t> {   // BF16 bits widen exactly to FP32
  static constexpr int kElems = 8;
  __device__ static void widen(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

}  // namespace fg8
