// MoE routing -> contiguous grouped-GEMM layout, with the 1x128 quantization
// of the gathered rows fused in.
//
// The contiguous layout of DeepGEMM's MoE grouped GEMM (release news,
// ctol-kr.com, section 4) stacks the rows routed to each expert, expert after
// expert, each run padded to a multiple of the 128-row M block, and names the
// expert of every block.  Here it is built on the device from the router's
// top-k expert ids, so the counts never visit the host:
//   1. count: one workgroup per expert counts the tokens that chose it;
//   2. offsets: one workgroup turns the padded counts into run offsets and
//      labels every 128-row block with its expert (-1 past the last run);
//   3. place: one workgroup per expert walks the tokens in ascending order
//      (a block-wide scan gives each token its rank) and writes row_token;
//   4. gather + quantize: 1x128 groups of the source row of every layout row
//      (zeros, scale 1, for padding), as the 1x128 quantizer does.
// Steps 1-3 read only the ids (tokens x top-k int32); step 4 is the HBM
// stream: one read of every routed row, one write of the FP8 codes.
#include "fg8_device.h"
#include "fg8_internal.h"

namespace fg8 {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

// Does token t route to expert e?  A repeated id counts once; ids outside
// [0, E) route nowhere.
__device__ __forceinline__ int routes_to(const int32_t* __restrict__ ids, int64_t t, int topk,
                                         int e) {
  int hit = 0;
  for (int j = 0; j < topk; ++j) hit |= ids[t * topk + j] == e;
  return hit;
}

// Block-wide exclusive scan of one int per thread; also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wave_sum[kRouteWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kRouteWaves; ++w) {
    const int s = wave_sum[w];
    base += w < wave ? s : 0;
    all += s;
  }
  __syncthreads();   // wave_sum may be reused by the caller's next scan
  *total = all;
  return base + incl - v;
}

__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(
    const int32_t* __restrict__ ids, int64_t tokens, int topk, int32_t* __restrict__ counts) {
  const int e = blockIdx.x;
  int n = 0;
  for (int64_t t = threadIdx.x; t < tokens; t += kRouteThreads) n += routes_to(ids, t, topk, e);
  int total;
  block_exclusive_scan(n, &total);
  if (threadIdx.x == 0) counts[e] = total;
}

// One workgroup; num_experts <= kRouteThreads.
__global__ __launch_bounds__(kRouteThreads) void route_offsets_kernel(
    const int32_t* __restrict__ counts, int num_experts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ block_expert, int64_t nblocks) {
  __shared__ int off[kRouteThreads + 1];
  const int e = threadIdx.x;
  const int padded = e < num_experts ? (counts[e] + kGroup - 1) / kGroup * kGroup : 0;
  int total;
  const int start = block_exclusive_scan(padded, &total);
  if (e < num_experts) {
    off[e] = start;
    offsets[e] = start;
  }
  if (e == 0) {
    off[num_experts] = total;
    offsets[num_experts] = total;
  }
  __syncthreads();
  for (int64_t b = threadIdx.x; b < nblocks; b += kRouteThreads) {
    const int64_t row = b * kGroup;
    int lo = 0, hi = num_experts;   // last expert whose run starts at or before row
    while (lo + 1 < hi) {
      const int mid = (lo + hi) >> 1;
      if (off[mid] <= row) lo = mid; else hi = mid;
    }
    block_expert[b] = row < off[num_experts] && off[lo] <= row ? lo : -1;
  }
}

// Workgroup e < num_experts places expert e's tokens; workgroup num_experts
// marks the rows past the last run as padding.
__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(
    const int32_t* __restrict__ ids, int64_t tokens, int topk, int num_experts,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int64_t m_cap) {
  const int e = blockIdx.x;
  if (e == num_experts) {
    for (int64_t r = offsets[num_experts] + threadIdx.x; r < m_cap; r += kRouteThreads)
      row_token[r] = -1;
    return;
  }
  const int64_t base = offsets[e];
  int placed = 0;
  for (int64_t t0 = 0; t0 < tokens; t0 += kRouteThreads) {
    const int64_t t = t0 + threadIdx.x;
    const int hit = t < tokens ? routes_to(ids, t, topk, e) : 0;
    int total;
    const int rank = block_exclusive_scan(hit, &total);
    if (hit) row_token[base + placed + rank] = (int32_t)t;
    placed += total;
  }
  const int64_t end = offsets[e + 1];
  for (int64_t r = base + counts[e] + threadIdx.x; r < end; r += kRouteThreads) row_token[r] = -1;
}

hipError_t launch_route_quantize(const void* x, bool bf16, int64_t tokens, int64_t hidden,
                                 const int32_t* ids, int topk, int num_experts, int64_t m_cap,
                                 uint8_t* q, float* sa, int32_t* block_expert, int32_t* row_token,
                                 int32_t* counts, int32_t* offsets, hipStream_t stream) {
  hipLaunchKernelGGL(route_count_kernel, dim3(num_experts), dim3(kRouteThreads), 0, stream, ids,
                     tokens, topk, counts);
  hipLaunchKernelGGL(route_offsets_kernel, dim3(1), dim3(kRouteThreads), 0, stream, counts,
                     num_experts, offsets, block_expert, m_cap / kGroup);
  hipLaunchKernelGGL(route_place_kernel, dim3(num_experts + 1), dim3(kRouteThreads), 0, stream,
                     ids, tokens, topk, num_experts, counts, offsets, row_token, m_cap);
  if (const hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  return launch_quantize_gather(x, bf16, row_token, m_cap, hidden, q, sa, stream);
}

}  // namespace fg8
