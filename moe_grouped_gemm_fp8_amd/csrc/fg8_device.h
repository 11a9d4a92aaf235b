// Device helpers shared by the fg8 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang diagnostic ignored "-Winline-asm"   // m0 is written by the LDS-DMA asm

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

// Loads of 16 or 8 source bytes with the non-temporal hint, for the large
// quantize launches that read each source element once: 1x128 over
// 69,632 x 7168 467 -> 451 us, 128x128 813 -> 774 us, MX 875 -> 821 us.
// The decode-sized 1x128 launch, the routing scatter and the transposed
// quantize ran slower with them (by 0.45 us, 13% and 1%) and keep ordinary
// loads.  p is aligned to the load's size.
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const u4 v = __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 load_nt8(const void* p) {
  const uint64_t v = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(p));
  return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}

// Stores of 4, 8 or 16 code bytes with the non-temporal hint, for the
// quantize and routing kernels that write whole lines of codes: against
// ordinary stores, 3-5% faster on the large 1x128, 128x128 and MX quantize
// launches and 22% on the routing scatter (8192x7168 tokens, top-8 of 32).
// p is aligned to the store's size.
__device__ __forceinline__ void store_nt(uint8_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void store_nt(uint8_t* p, uint32_t lo, uint32_t hi) {
  __builtin_nontemporal_store(((uint64_t)hi << 32) | lo, reinterpret_cast<uint64_t*>(p));
}
__device__ __forceinline__ void store_nt(uint8_t* p, uint32_t a, uint32_t b, uint32_t c,
                                         uint32_t d) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(u4{a, b, c, d}, reinterpret_cast<u4*>(p));
}

// Two FP32 values -> two BF16 values (low half from a) with one
// v_cvt_pk_bf16_f32: round to nearest even, subnormals kept, NaN stays NaN
// (pinned against torch's CPU cast by the probe tests).
__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
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

// ---------------------------------------------------------------- GEMM helpers
// 16-byte chunk swizzle of LDS row r.  Measured with SQ_LDS_BANK_CONFLICT on
// gfx950: (r >> 1) & 7 leaves the MFMA operand reads (one chunk of 16
// consecutive rows per ds_read_b128) free of bank conflicts.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Global -> LDS copies without staging registers (global_load_lds_*).
// Lane i of the wave writes its 16 (or 4) bytes at LDS address m0 + 16 i
// (4 i); the global address is the uniform base plus the lane's 32-bit
// offset.  They are issued from inline assembly so that the compiler does not
// guard every later LDS read with a wait for all of them: the kernel counts
// these loads itself (wait_vmcnt) and orders LDS use with barriers.  The
// instructions write no VGPR.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
// The same copy with the non-temporal hint, for operand rows that no other
// workgroup of the launch reads.
__device__ __forceinline__ void dma16_nt(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
template <class T>
__device__ __forceinline__ T uniform(T v) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
  }
}

// One MFMA operand fragment: 16 rows starting at tile row r0.
__device__ __forceinline__ v8i load_frag(const uint8_t* tile, int r0, int lane) {
  const int r = r0 + (lane & 15), g = lane >> 4, s = swz(r);
  const uint8_t* row = tile + r * kGroup;
  const int4 lo = *reinterpret_cast<const int4*>(row + ((g ^ s) << 4));
  const int4 hi = *reinterpret_cast<const int4*>(row + (((g + 4) ^ s) << 4));
  v8i f;
  f[0] = lo.x; f[1] = lo.y; f[2] = lo.z; f[3] = lo.w;
  f[4] = hi.x; f[5] = hi.y; f[6] = hi.z; f[7] = hi.w;
  return f;
}

// Split-K partials are published with 16-byte buffer stores that carry the
// agent-scope coherence bit (sc1: written through to the point of coherence
// shared by all XCDs) and read back with sc1 buffer loads; a vmcnt(0) wait
// orders them before the arrival counter, so no L2 write-back is needed.
// Raw buffer descriptor: base, byte bound, no stride, gfx9 dword 3.
constexpr int kBufferDword3 = 0x00020000;
constexpr int kCoherent = 16;   // cache-policy operand of the buffer builtins: sc1
// Output tiles are written with the non-temporal bit (nt): nothing reads them
// again inside the launch, and on 4096x7168x2048 this ran 6% faster than
// ordinary stores (1-2% on the MoE GEMMs, the decode shapes unchanged).
constexpr int kStream = 2;      // cache-policy operand of the buffer builtins: nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferDword3);
}
__device__ __forceinline__ void wait_all_memory() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace fg8
