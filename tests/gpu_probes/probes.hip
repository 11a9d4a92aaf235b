// Hardware probes for gfx950, used only by tests/test_gpu_probes.py.
//
// Each probe runs one wavefront (or a plain grid-stride loop) on buffers the
// caller sized exactly: 64 lanes x 32 bytes per MFMA operand, 64 lanes x 4 or
// 16 floats per MFMA result.  The tests compare the results with what a
// stated hypothesis about the lane layout, the FP8 conversion or the scale
// encoding predicts.  These are facts the GEMM kernels rely on.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ void k_mfma16(const v8i* a, const v8i* b, v4f* d) {
  const int l = threadIdx.x;
  v4f z = {0.f, 0.f, 0.f, 0.f};
  d[l] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[l], b[l], z, 0, 0, 0, 0, 0, 0);
}

__global__ void k_mfma32(const v8i* a, const v8i* b, v16f* d) {
  const int l = threadIdx.x;
  v16f z = {};
  d[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], z, 0, 0, 0, 0, 0, 0);
}

__global__ void k_mfma16_scaled(const v8i* a, const v8i* b, const int* sa, const int* sb, v4f* d) {
  const int l = threadIdx.x;
  v4f z = {0.f, 0.f, 0.f, 0.f};
  d[l] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[l], b[l], z, 0, 0, 0, sa[l], 0, sb[l]);
}

__global__ void k_mfma32_scaled(const v8i* a, const v8i* b, const int* sa, const int* sb, v16f* d) {
  const int l = threadIdx.x;
  v16f z = {};
  d[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], z, 0, 0, 0, sa[l], 0, sb[l]);
}

// D = A B + C with the accumulator input C loaded per lane.
__global__ void k_mfma16_acc(const v8i* a, const v8i* b, const v4f* c, v4f* d) {
  const int l = threadIdx.x;
  d[l] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[l], b[l], c[l], 0, 0, 0, 0, 0, 0);
}
__global__ void k_mfma32_acc(const v8i* a, const v8i* b, const v16f* c, v16f* d) {
  const int l = threadIdx.x;
  d[l] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[l], b[l], c[l], 0, 0, 0, 0, 0, 0);
}

// n floats -> n/2 packed words (bytes 0 and 1 hold the two conversions).
__global__ void k_cvt(const float* x, uint32_t* out, int npairs, int clamp) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= npairs) return;
  float a = x[2 * i], b = x[2 * i + 1];
  if (clamp) {
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
  }
  out[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
}

// n floats -> n/2 words of two BF16 values (v_cvt_pk_bf16_f32: low half from
// the first float).
__global__ void k_cvt_bf16(const float* x, uint32_t* out, int npairs) {
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= npairs) return;
  const f2 v = {x[2 * i], x[2 * i + 1]};
  out[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
}

__global__ void k_copy(const float4* __restrict__ src, float4* __restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

extern "C" {

int probe_mfma16(const void* a, const void* b, void* d, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma16, dim3(1), dim3(64), 0, s, (const v8i*)a, (const v8i*)b, (v4f*)d);
  return (int)hipGetLastError();
}
int probe_mfma32(const void* a, const void* b, void* d, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma32, dim3(1), dim3(64), 0, s, (const v8i*)a, (const v8i*)b, (v16f*)d);
  return (int)hipGetLastError();
}
int probe_mfma16_scaled(const void* a, const void* b, const void* sa, const void* sb, void* d,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_mfma16_scaled, dim3(1), dim3(64), 0, s, (const v8i*)a, (const v8i*)b,
                     (const int*)sa, (const int*)sb, (v4f*)d);
  return (int)hipGetLastError();
}
int probe_mfma32_scaled(const void* a, const void* b, const void* sa, const void* sb, void* d,
                        hipStream_t s) {
  hipLaunchKernelGGL(k_mfma32_scaled, dim3(1), dim3(64), 0, s, (const v8i*)a, (const v8i*)b,
                     (const int*)sa, (const int*)sb, (v16f*)d);
  return (int)hipGetLastError();
}
int probe_mfma16_acc(const void* a, const void* b, const void* c, void* d, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma16_acc, dim3(1), dim3(64), 0, s, (const v8i*)a, (const v8i*)b,
                     (const v4f*)c, (v4f*)d);
  return (int)hipGetLastError();
}
int probe_mfma32_acc(const void* a, const void* b, const void* c, void* d, hipStream_t s) {
  hipLaunchKernelGGL(k_mfma32_acc, dim3(1), dim3(64), 0, s, (const v8i*)a, (const v8i*)b,
                     (const v16f*)c, (v16f*)d);
  return (int)hipGetLastError();
}
int probe_cvt_fp8(const void* x, void* out, int npairs, int clamp, hipStream_t s) {
  hipLaunchKernelGGL(k_cvt, dim3((npairs + 255) / 256), dim3(256), 0, s, (const float*)x,
                     (uint32_t*)out, npairs, clamp);
  return (int)hipGetLastError();
}
int probe_cvt_bf16(const void* x, void* out, int npairs, hipStream_t s) {
  hipLaunchKernelGGL(k_cvt_bf16, dim3((npairs + 255) / 256), dim3(256), 0, s, (const float*)x,
                     (uint32_t*)out, npairs);
  return (int)hipGetLastError();
}
int probe_copy(const void* src, void* dst, size_t n_float4, int blocks, hipStream_t s) {
  hipLaunchKernelGGL(k_copy, dim3(blocks), dim3(256), 0, s, (const float4*)src, (float4*)dst,
                     n_float4);
  return (int)hipGetLastError();
}

}  // extern "C"
