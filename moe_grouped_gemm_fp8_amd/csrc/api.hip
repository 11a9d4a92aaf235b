// C ABI of libfg8.so: argument checks, tile selection and launches.
// Every entry point validates before it launches anything; see fg8.h for the
// meaning, layout and ownership of each argument.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "fg8.h"
#include "fg8_internal.h"

namespace {

thread_local char g_err[512] = "";

fg8_status fail(fg8_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define FG8_CHECK_PTR(p)                                                                  \
  do {                                                                                    \
    if (!(p)) return fail(FG8_EINVAL, "%s: %s is NULL", fn, #p);                          \
    if (!aligned16(p)) return fail(FG8_EINVAL, "%s: %s is not 16-byte aligned", fn, #p);  \
  } while (0)

constexpr int64_t kMaxDim = (int64_t)1 << 31;   // row / column counts must fit int32
// 32-bit LDS-DMA offsets inside a tile of up to 256 rows: (256 - 1) * k < 2^32
constexpr int64_t kMaxK = ((int64_t)1 << 24) - 128;
constexpr int64_t kMaxKGrouped = kMaxK;

fg8_status check_k(const char* fn, int64_t k) {
  if (k < 128 || k > kMaxK) return fail(FG8_EUNSUPPORTED, "%s: k=%lld must be in [128, %lld]", fn,
                                        (long long)k, (long long)kMaxK);
  if (k % 128) return fail(FG8_EUNSUPPORTED, "%s: k=%lld is not a multiple of 128", fn, (long long)k);
  return FG8_OK;
}

// The kernels count work units (tiles times splits) in 32-bit integers.
fg8_status check_units(const fg8::GemmProblem& p, const fg8::TileChoice& t, const char* fn) {
  const int64_t units = (int64_t)(p.mode == fg8::kMasked || p.mode == fg8::kKGrouped ? p.groups : 1) *
                        ((p.M + t.bm - 1) / t.bm) * ((p.N + t.bn - 1) / t.bn) * t.splits *
                        (p.mode == fg8::kContiguous && t.bm > 128 ? 2 : 1);   // 256-row pair units
  if (units >= INT32_MAX)
    return fail(FG8_EUNSUPPORTED, "%s: %lld tiles exceed the 32-bit work-unit count", fn,
                (long long)units);
  return FG8_OK;
}

fg8_status run(fg8::GemmProblem& p, const char* fn, hipStream_t stream) {
  const fg8::TileChoice t = fg8::choose_tiles(p, fg8::device_cu_count());
  if (fg8_status st = check_units(p, t, fn)) return st;
  const hipError_t e = fg8::launch_gemm(p, t, stream);
  if (e != hipSuccess) return fail(FG8_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  g_err[0] = 0;
  return FG8_OK;
}

}  // namespace

extern "C" {

int fg8_version(void) { return 500; }   // 0.5.0

const char* fg8_last_error(void) { return g_err; }

}  // extern "C"

namespace {

fg8_status quantize_any(const char* fn, const void* x, bool bf16, int64_t batch, int64_t rows,
                        int64_t cols, fg8_scale_kind kind, uint8_t* q, void* scales,
                        hipStream_t stream) {
  FG8_CHECK_PTR(x);
  FG8_CHECK_PTR(q);
  FG8_CHECK_PTR(scales);
  if (batch < 1 || rows < 1 || cols < 1 || batch >= 65536 || rows >= kMaxDim || cols >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes batch=%lld rows=%lld cols=%lld", fn, (long long)batch,
                (long long)rows, (long long)cols);
  if (kind != FG8_SCALE_1x128 && kind != FG8_SCALE_128x128 && kind != FG8_SCALE_MX1x32 &&
      kind != FG8_SCALE_1x128_T)
    return fail(FG8_EINVAL, "%s: unknown scale kind %d", fn, (int)kind);
  if (kind == FG8_SCALE_1x128_T) {
    if (rows % 128 || cols % 64)
      return fail(FG8_EUNSUPPORTED, "%s: transposed 1x128 needs rows %% 128 == 0 and cols %% 64 == 0"
                  " (rows=%lld cols=%lld)", fn, (long long)rows, (long long)cols);
    if (rows / 128 >= 65536) return fail(FG8_EUNSUPPORTED, "%s: too many row blocks", fn);
  }
  const int64_t unit = kind == FG8_SCALE_MX1x32 ? 32 : kind == FG8_SCALE_1x128_T ? 64 : 128;
  if (cols % unit)
    return fail(FG8_EUNSUPPORTED, "%s: cols=%lld is not a multiple of %lld", fn, (long long)cols,
                (long long)unit);
  if (kind == FG8_SCALE_128x128 && (rows + 127) / 128 >= 65536)
    return fail(FG8_EUNSUPPORTED, "%s: too many row blocks", fn);
  if ((kind == FG8_SCALE_1x128 || kind == FG8_SCALE_128x128) && cols / 128 >= 65536)
    return fail(FG8_EUNSUPPORTED, "%s: too many column blocks", fn);
  const hipError_t e =
      fg8::launch_quantize(x, bf16, batch, rows, cols, (int)kind, q, scales, stream);
  if (e != hipSuccess) return fail(FG8_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  g_err[0] = 0;
  return FG8_OK;
}

}  // namespace

extern "C" {

fg8_status fp8_quantize(const float* x, int64_t batch, int64_t rows, int64_t cols,
                        fg8_scale_kind kind, uint8_t* q, void* scales, hipStream_t stream) {
  return quantize_any("fp8_quantize", x, false, batch, rows, cols, kind, q, scales, stream);
}

fg8_status fp8_quantize_bf16(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                             fg8_scale_kind kind, uint8_t* q, void* scales, hipStream_t stream) {
  return quantize_any("fp8_quantize_bf16", x, true, batch, rows, cols, kind, q, scales, stream);
}

size_t fg8_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 1 || n < 1 || k < 128 || k % 128 || k > kMaxK) return 0;
  return fg8::splitk_workspace_bytes(m, n, k, fg8::device_cu_count());
}

fg8_status gemm_fp8_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                const float* sb, void* d, fg8_out out, int64_t m, int64_t n,
                                int64_t k, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  const char* fn = "gemm_fp8_blockscaled";
  FG8_CHECK_PTR(a);
  FG8_CHECK_PTR(sa);
  FG8_CHECK_PTR(b);
  FG8_CHECK_PTR(sb);
  FG8_CHECK_PTR(d);
  if (out != FG8_OUT_F32 && out != FG8_OUT_BF16) return fail(FG8_EINVAL, "%s: bad out", fn);
  if (m < 1 || n < 1 || m >= kMaxDim || n >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes m=%lld n=%lld", fn, (long long)m, (long long)n);
  if (fg8_status s = check_k(fn, k)) return s;
  fg8::GemmProblem p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.d = d;
  p.out_bf16 = out == FG8_OUT_BF16;
  p.mode = fg8::kDense; p.M = m; p.N = n; p.K = k; p.groups = 1;
  const fg8::TileChoice t = fg8::choose_tiles(p, fg8::device_cu_count());
  if (fg8_status st = check_units(p, t, fn)) return st;
  if (t.splits > 1) {
    const size_t need = fg8::splitk_workspace_bytes(m, n, k, fg8::device_cu_count());
    if (!workspace || workspace_bytes < need)
      return fail(FG8_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(FG8_EINVAL, "%s: workspace misaligned", fn);
    p.ws_counters = (int32_t*)workspace;
    p.ws_partial = (float*)((char*)workspace + fg8::kSplitKCounterBytes);
  }
  const hipError_t e = fg8::launch_gemm(p, t, stream);
  if (e != hipSuccess) return fail(FG8_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  g_err[0] = 0;
  return FG8_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch of the allocation-free dense GEMM (gemm_fp8_blockscaled_noalloc):
// the split-K arrival counters and partial sums live in this array, one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it names a stand-in, not device memory):
// each device's address is looked up once with hipGetSymbolAddress and kept.
static_assert(FG8_NOALLOC_SCRATCH_BYTES > fg8::kSplitKCounterBytes, "scratch holds the counters");
static __device__ __align__(256) uint8_t scratch[FG8_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// Zeroes n 32-bit words (the arrival counters) without hipMemsetAsync, so
// that the first call on a device may be captured into a graph.
__global__ void zero_words(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// The device address of this device's scratch, looked up (and its counters
// cleared, on the caller's stream) at the first call on the device.
fg8_status scratch_ptr(const char* fn, hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FG8_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(FG8_EUNSUPPORTED, "%s: device %d", fn, dev);
  ScratchSlot& s = g_scratch[dev];
  std::call_once(s.once, [&] {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s.err == hipSuccess) {
      hipLaunchKernelGGL(zero_words, dim3(1), dim3(256), 0, stream, (uint32_t*)p,
                         (int)(fg8::kSplitKCounterBytes / 4));
      s.err = hipGetLastError();
    }
    if (s.err == hipSuccess) s.ptr = p;
  });
  if (s.err != hipSuccess)
    return fail(FG8_EHIP, "%s: scratch set-up failed: %s", fn, hipGetErrorString(s.err));
  *out = s.ptr;
  return FG8_OK;
}

}  // namespace

extern "C" {

fg8_status gemm_fp8_blockscaled_noalloc(const uint8_t* a, const float* sa, const uint8_t* b,
                                        const float* sb, void* d, fg8_out out, int64_t m,
                                        int64_t n, int64_t k, hipStream_t stream) {
  const char* fn = "gemm_fp8_blockscaled_noalloc";
  FG8_CHECK_PTR(a);
  FG8_CHECK_PTR(sa);
  FG8_CHECK_PTR(b);
  FG8_CHECK_PTR(sb);
  FG8_CHECK_PTR(d);
  if (out != FG8_OUT_F32 && out != FG8_OUT_BF16) return fail(FG8_EINVAL, "%s: bad out", fn);
  if (m < 1 || n < 1 || m >= kMaxDim || n >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes m=%lld n=%lld", fn, (long long)m, (long long)n);
  if (fg8_status s = check_k(fn, k)) return s;
  fg8::GemmProblem p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.d = d;
  p.out_bf16 = out == FG8_OUT_BF16;
  p.mode = fg8::kDense; p.M = m; p.N = n; p.K = k; p.groups = 1;
  const int cus = fg8::device_cu_count();
  const fg8::TileChoice t = fg8::choose_tiles(p, cus);
  if (fg8_status st = check_units(p, t, fn)) return st;
  if (t.splits > 1) {
    const size_t need = fg8::splitk_workspace_bytes(m, n, k, cus);
    if (need > (size_t)FG8_NOALLOC_SCRATCH_BYTES)
      return fail(FG8_EUNSUPPORTED, "%s: m=%lld n=%lld k=%lld needs %zu bytes of split-K scratch, "
                  "more than the %zu this entry point holds (use gemm_fp8_blockscaled with a "
                  "workspace)", fn, (long long)m, (long long)n, (long long)k, need,
                  (size_t)FG8_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (fg8_status st = scratch_ptr(fn, stream, &ws)) return st;
    p.ws_counters = (int32_t*)ws;
    p.ws_partial = (float*)((char*)ws + fg8::kSplitKCounterBytes);
  }
  const hipError_t e = fg8::launch_gemm(p, t, stream);
  if (e != hipSuccess) return fail(FG8_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  g_err[0] = 0;
  return FG8_OK;
}

fg8_status grouped_gemm_fp8_contiguous(const uint8_t* a, const float* sa, const uint8_t* b,
                                       const float* sb, const int32_t* block_expert, void* d,
                                       fg8_out out, int64_t m_total, int64_t n, int64_t k,
                                       int32_t num_experts, hipStream_t stream) {
  const char* fn = "grouped_gemm_fp8_contiguous";
  FG8_CHECK_PTR(a);
  FG8_CHECK_PTR(sa);
  FG8_CHECK_PTR(b);
  FG8_CHECK_PTR(sb);
  FG8_CHECK_PTR(block_expert);
  FG8_CHECK_PTR(d);
  if (out != FG8_OUT_F32 && out != FG8_OUT_BF16) return fail(FG8_EINVAL, "%s: bad out", fn);
  if (num_experts < 1) return fail(FG8_EINVAL, "%s: num_experts=%d", fn, (int)num_experts);
  if (m_total < 1 || n < 1 || m_total >= kMaxDim || n >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes m_total=%lld n=%lld", fn, (long long)m_total,
                (long long)n);
  if (m_total % 128)
    return fail(FG8_EUNSUPPORTED, "%s: m_total=%lld is not a multiple of 128", fn,
                (long long)m_total);
  if (fg8_status s = check_k(fn, k)) return s;
  fg8::GemmProblem p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.d = d;
  p.out_bf16 = out == FG8_OUT_BF16;
  p.mode = fg8::kContiguous; p.M = m_total; p.N = n; p.K = k; p.groups = num_experts;
  p.block_expert = block_expert;
  return run(p, fn, stream);
}

fg8_status grouped_gemm_fp8_contiguous_swiglu(const uint8_t* a, const float* sa,
                                              const uint8_t* b, const float* sb,
                                              const int32_t* block_expert, uint8_t* q_out,
                                              float* s_out, int64_t m_total, int64_t n, int64_t k,
                                              int32_t num_experts, hipStream_t stream) {
  const char* fn = "grouped_gemm_fp8_contiguous_swiglu";
  FG8_CHECK_PTR(a);
  FG8_CHECK_PTR(sa);
  FG8_CHECK_PTR(b);
  FG8_CHECK_PTR(sb);
  FG8_CHECK_PTR(block_expert);
  FG8_CHECK_PTR(q_out);
  FG8_CHECK_PTR(s_out);
  if (num_experts < 1) return fail(FG8_EINVAL, "%s: num_experts=%d", fn, (int)num_experts);
  if (m_total < 1 || n < 1 || m_total >= kMaxDim || n >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes m_total=%lld n=%lld", fn, (long long)m_total,
                (long long)n);
  if (m_total % 128)
    return fail(FG8_EUNSUPPORTED, "%s: m_total=%lld is not a multiple of 128", fn,
                (long long)m_total);
  if (n % 256)
    return fail(FG8_EUNSUPPORTED, "%s: n=%lld is not a multiple of 256 (gate/up block pairs)", fn,
                (long long)n);
  if (fg8_status s = check_k(fn, k)) return s;
  fg8::GemmProblem p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.d = nullptr;
  p.mode = fg8::kContiguous; p.M = m_total; p.N = n; p.K = k; p.groups = num_experts;
  p.block_expert = block_expert;
  p.swiglu = 1; p.q_out = q_out; p.s_out = s_out;
  return run(p, fn, stream);
}

fg8_status grouped_gemm_fp8_kgrouped(const uint8_t* a, const float* sa, const uint8_t* b,
                                     const float* sb, const int32_t* k_offsets, void* d,
                                     fg8_out out, int32_t num_groups, int64_t m, int64_t n,
                                     int64_t k_total, hipStream_t stream) {
  const char* fn = "grouped_gemm_fp8_kgrouped";
  FG8_CHECK_PTR(a);
  FG8_CHECK_PTR(sa);
  FG8_CHECK_PTR(b);
  FG8_CHECK_PTR(sb);
  FG8_CHECK_PTR(k_offsets);
  FG8_CHECK_PTR(d);
  if (out != FG8_OUT_F32 && out != FG8_OUT_BF16) return fail(FG8_EINVAL, "%s: bad out", fn);
  if (num_groups < 1 || num_groups > 65536)
    return fail(FG8_EINVAL, "%s: num_groups=%d must be in [1, 65536]", fn, (int)num_groups);
  if (m < 1 || n < 1 || m >= kMaxDim || n >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes m=%lld n=%lld", fn, (long long)m, (long long)n);
  // K is the whole token axis here: 32-bit LDS-DMA offsets of a 256-row tile
  // bound it to below 2^24
  if (k_total < 128 || k_total % 128 || k_total > kMaxKGrouped)
    return fail(FG8_EUNSUPPORTED, "%s: k_total=%lld must be a multiple of 128 in [128, %lld]", fn,
                (long long)k_total, (long long)kMaxKGrouped);
  fg8::GemmProblem p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.d = d;
  p.out_bf16 = out == FG8_OUT_BF16;
  p.mode = fg8::kKGrouped; p.M = m; p.N = n; p.K = k_total; p.groups = num_groups;
  p.k_offsets = k_offsets;
  return run(p, fn, stream);
}

fg8_status grouped_gemm_fp8_masked(const uint8_t* a, const float* sa, const uint8_t* b,
                                   const float* sb, const int32_t* valid_rows, void* d,
                                   fg8_out out, int32_t num_experts, int64_t cap, int64_t n,
                                   int64_t k, hipStream_t stream) {
  const char* fn = "grouped_gemm_fp8_masked";
  FG8_CHECK_PTR(a);
  FG8_CHECK_PTR(sa);
  FG8_CHECK_PTR(b);
  FG8_CHECK_PTR(sb);
  FG8_CHECK_PTR(valid_rows);
  FG8_CHECK_PTR(d);
  if (out != FG8_OUT_F32 && out != FG8_OUT_BF16) return fail(FG8_EINVAL, "%s: bad out", fn);
  if (num_experts < 1 || num_experts > 1024)
    return fail(FG8_EINVAL, "%s: num_experts=%d must be in [1, 1024]", fn, (int)num_experts);
  if (cap < 1 || n < 1 || cap >= kMaxDim || n >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes cap=%lld n=%lld", fn, (long long)cap, (long long)n);
  if (fg8_status s = check_k(fn, k)) return s;
  fg8::GemmProblem p{};
  p.a = a; p.sa = sa; p.b = b; p.sb = sb; p.d = d;
  p.out_bf16 = out == FG8_OUT_BF16;
  p.mode = fg8::kMasked; p.M = cap; p.N = n; p.K = k; p.groups = num_experts;
  p.valid = valid_rows;
  return run(p, fn, stream);
}

fg8_status gemm_mxfp8(const uint8_t* a, const uint8_t* sa_e8m0, const uint8_t* b,
                      const uint8_t* sb_e8m0, const int32_t* valid_rows, void* d, fg8_out out,
                      int32_t num_groups, int64_t m_per_group, int64_t n, int64_t k,
                      hipStream_t stream) {
  const char* fn = "gemm_mxfp8";
  FG8_CHECK_PTR(a);
  FG8_CHECK_PTR(sa_e8m0);
  FG8_CHECK_PTR(b);
  FG8_CHECK_PTR(sb_e8m0);
  FG8_CHECK_PTR(d);
  if (valid_rows && !aligned16(valid_rows))
    return fail(FG8_EINVAL, "%s: valid_rows is not 16-byte aligned", fn);
  if (out != FG8_OUT_F32 && out != FG8_OUT_BF16) return fail(FG8_EINVAL, "%s: bad out", fn);
  if (num_groups < 1 || num_groups > 1024)
    return fail(FG8_EINVAL, "%s: num_groups=%d must be in [1, 1024]", fn, (int)num_groups);
  if (m_per_group < 1 || n < 1 || m_per_group >= kMaxDim || n >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes m=%lld n=%lld", fn, (long long)m_per_group,
                (long long)n);
  if (fg8_status s = check_k(fn, k)) return s;
  fg8::GemmProblem p{};
  p.a = a; p.sa = sa_e8m0; p.b = b; p.sb = sb_e8m0; p.d = d;
  p.out_bf16 = out == FG8_OUT_BF16;
  p.mx = 1;
  p.mode = fg8::kMasked; p.M = m_per_group; p.N = n; p.K = k; p.groups = num_groups;
  p.valid = valid_rows;
  return run(p, fn, stream);
}

fg8_status grouped_gemm_mxfp8_contiguous(const uint8_t* a, const uint8_t* sa_e8m0,
                                         const uint8_t* b, const uint8_t* sb_e8m0,
                                         const int32_t* block_expert, void* d, fg8_out out,
                                         int64_t m_total, int64_t n, int64_t k,
                                         int32_t num_experts, hipStream_t stream) {
  const char* fn = "grouped_gemm_mxfp8_contiguous";
  FG8_CHECK_PTR(a);
  FG8_CHECK_PTR(sa_e8m0);
  FG8_CHECK_PTR(b);
  FG8_CHECK_PTR(sb_e8m0);
  FG8_CHECK_PTR(block_expert);
  FG8_CHECK_PTR(d);
  if (out != FG8_OUT_F32 && out != FG8_OUT_BF16) return fail(FG8_EINVAL, "%s: bad out", fn);
  if (num_experts < 1) return fail(FG8_EINVAL, "%s: num_experts=%d", fn, (int)num_experts);
  if (m_total < 1 || n < 1 || m_total >= kMaxDim || n >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes m_total=%lld n=%lld", fn, (long long)m_total,
                (long long)n);
  if (m_total % 128)
    return fail(FG8_EUNSUPPORTED, "%s: m_total=%lld is not a multiple of 128", fn,
                (long long)m_total);
  if (fg8_status s = check_k(fn, k)) return s;
  fg8::GemmProblem p{};
  p.a = a; p.sa = sa_e8m0; p.b = b; p.sb = sb_e8m0; p.d = d;
  p.out_bf16 = out == FG8_OUT_BF16;
  p.mx = 1;
  p.mode = fg8::kContiguous; p.M = m_total; p.N = n; p.K = k; p.groups = num_experts;
  p.block_expert = block_expert;
  return run(p, fn, stream);
}

fg8_status fg8_tile_choice(int32_t mode, int64_t m, int64_t n, int64_t k, int32_t groups,
                           int32_t num_cus, int32_t* out) {
  if (!out) return fail(FG8_EINVAL, "fg8_tile_choice: out is NULL");
  if (mode < fg8::kDense || mode > fg8::kKGrouped || m < 1 || n < 1 || k < 128 || k % 128 ||
      groups < 1 || num_cus < 1)
    return fail(FG8_EINVAL, "fg8_tile_choice: bad arguments (mode=%d m=%lld n=%lld k=%lld "
                "groups=%d num_cus=%d)", (int)mode, (long long)m, (long long)n, (long long)k,
                (int)groups, (int)num_cus);
  fg8::GemmProblem p{};
  p.mode = (int)mode; p.M = m; p.N = n; p.K = k; p.groups = groups;
  const fg8::TileChoice t = fg8::choose_tiles(p, num_cus);
  out[0] = t.bm; out[1] = t.bn; out[2] = t.splits; out[3] = t.grid; out[4] = t.raster;
  return FG8_OK;
}

int64_t fg8_moe_capacity(int64_t tokens, int32_t topk, int32_t num_experts) {
  if (tokens < 1 || tokens >= kMaxDim || topk < 1 || topk > 256 || num_experts < 1 ||
      num_experts > 1024)
    return 0;
  return (tokens * topk + (int64_t)num_experts * 127 + 127) / 128 * 128;
}

fg8_status moe_contiguous_layout_fp8(const void* x, int32_t x_is_bf16, int64_t tokens,
                                     int64_t hidden, const int32_t* topk_ids, int32_t topk,
                                     int32_t num_experts, int64_t m_cap, uint8_t* q, float* sa,
                                     int32_t* block_expert, int32_t* row_token,
                                     int32_t* token_row, int32_t* expert_offsets,
                                     int32_t* expert_counts, hipStream_t stream) {
  const char* fn = "moe_contiguous_layout_fp8";
  FG8_CHECK_PTR(x);
  FG8_CHECK_PTR(topk_ids);
  FG8_CHECK_PTR(q);
  FG8_CHECK_PTR(sa);
  FG8_CHECK_PTR(block_expert);
  FG8_CHECK_PTR(row_token);
  FG8_CHECK_PTR(token_row);
  FG8_CHECK_PTR(expert_offsets);
  FG8_CHECK_PTR(expert_counts);
  if (x_is_bf16 != 0 && x_is_bf16 != 1)
    return fail(FG8_EINVAL, "%s: x_is_bf16=%d must be 0 or 1", fn, (int)x_is_bf16);
  if (tokens < 1 || tokens >= kMaxDim || hidden < 1 || hidden >= kMaxDim)
    return fail(FG8_EINVAL, "%s: bad sizes tokens=%lld hidden=%lld", fn, (long long)tokens,
                (long long)hidden);
  if (topk < 1 || topk > 256) return fail(FG8_EINVAL, "%s: topk=%d must be in [1, 256]", fn, topk);
  if (num_experts < 1 || num_experts > 1024)
    return fail(FG8_EINVAL, "%s: num_experts=%d must be in [1, 1024]", fn, (int)num_experts);
  if (hidden % 128 || hidden / 128 >= 65536)
    return fail(FG8_EUNSUPPORTED, "%s: hidden=%lld must be a multiple of 128 below 2^23", fn,
                (long long)hidden);
  const int64_t need = fg8_moe_capacity(tokens, topk, num_experts);
  if (m_cap % 128 || m_cap < need || m_cap >= kMaxDim)
    return fail(FG8_EINVAL, "%s: m_cap=%lld must be a multiple of 128 in [%lld, 2^31)", fn,
                (long long)m_cap, (long long)need);
  const hipError_t e = fg8::launch_route_quantize(x, x_is_bf16 == 1, tokens, hidden, topk_ids, topk,
                                                  num_experts, m_cap, q, sa, block_expert,
                                                  row_token, token_row, expert_counts,
                                                  expert_offsets, stream);
  if (e != hipSuccess) return fail(FG8_EHIP, "%s: launch failed: %s", fn, hipGetErrorString(e));
  g_err[0] = 0;
  return FG8_OK;
}

}  // extern "C"
