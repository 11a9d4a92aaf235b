// MoE routing -> contiguous grouped-GEMM layout, with the 1x128 quantization
// of the token rows fused in.
//
// The contiguous layout of DeepGEMM's MoE grouped GEMM (release news,
// ctol-kr.com, section 4) stacks the rows routed to each expert, expert after
// expert, each run padded to a multiple of the 128-row M block, and names the
// expert of every block.  Here it is built on the device from the router's
// top-k expert ids, so the counts never visit the host:
//   1. count: one workgroup per (expert, token range) counts the tokens of
//      the range that chose the expert;
//   2. offsets: one workgroup sums the ranges, turns the padded counts into
//      run offsets, labels every 128-row block with its expert (-1 past the
//      last run) and gives every (expert, range) its first row;
//   3. place: one workgroup per (expert, token range) walks its tokens in
//      ascending order (a block-wide scan gives each token its rank) and
//      writes row_token;
//   4. quantize + scatter: each token row is read once, quantized 1x128 as
//      the 1x128 quantizer does, and its codes and scales are written into
//      every row that holds the token (token_row, the inverse of row_token,
//      written by steps 1 and 3); padding rows get code 0, scale 1.
// Steps 1-3 read only the ids (tokens x top-k int32); step 4 is the HBM
// stream: one read of every token row, one write of every layout row.
#include "fg8_device.h"
#include "fg8_internal.h"

namespace fg8 {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;

// The ids are walked in chunks of up to kChunkInts ids.  A chunk is loaded
// into registers (kIdsPerThread coalesced loads per thread, all in flight,
// issued while the previous chunk is being examined) and stored to LDS
// id-major: id j of chunk token t at lds[j * (ct + 1) + t], so the threads of
// a wave, which examine consecutive tokens, read consecutive words (the odd
// stride keeps the stores nearly conflict-free too).  Tokens are examined in
// rounds of kRouteThreads consecutive tokens, thread i taking token i of the
// round.
constexpr int kIdsPerThread = 8;
constexpr int kChunkInts = kRouteThreads * kIdsPerThread;   // 32 KB of ids
constexpr int kChunkLds = kChunkInts + 256;                 // + the odd-stride padding
constexpr int kMaxRouteSplits = 64;

struct IdChunks {
  const int32_t* ids;
  int64_t tokens;         // end of this workgroup's token range
  int topk, ct, stride;   // tokens per chunk, LDS stride
  __device__ IdChunks(const int32_t* i, int64_t end, int k)
      : ids(i), tokens(end), topk(k), ct(kChunkInts / k), stride(kChunkInts / k + 1) {}
  __device__ int64_t count(int64_t t0) const { return tokens - t0 < ct ? tokens - t0 : ct; }
  __device__ void load(int64_t t0, int32_t (&v)[kIdsPerThread]) const {
    const int64_t n = count(t0) * topk;
#pragma unroll
    for (int i = 0; i < kIdsPerThread; ++i) {
      const int64_t j = (int64_t)i * kRouteThreads + threadIdx.x;
      v[i] = j < n ? ids[t0 * topk + j] : -1;
    }
  }
  __device__ void store(const int32_t (&v)[kIdsPerThread], int32_t* lds) const {
#pragma unroll
    for (int i = 0; i < kIdsPerThread; ++i) {
      const int g = i * kRouteThreads + threadIdx.x;   // id g = token * topk + j of the chunk
      const int t = g / topk, j = g - t * topk;
      if (t < ct) lds[j * stride + t] = v[i];
    }
  }
  // Does chunk token t route to expert e?  A repeated id counts once; ids
  // outside [0, E) route nowhere.
  __device__ int hit(const int32_t* lds, int t, int e) const {
    int h = 0;
    for (int j = 0; j < topk; ++j) h |= lds[j * stride + t] == e;
    return h;
  }
  // The first position of expert e in chunk token t's ids.
  __device__ int first(const int32_t* lds, int t, int e) const {
    int j = 0;
    while (lds[j * stride + t] != e) ++j;   // only called for a hit
    return j;
  }
  // Does position j of chunk token t route nowhere (an id outside [0, E) or
  // a repeat of an earlier id of the token)?
  __device__ bool dead(const int32_t* lds, int t, int j, int num_experts) const {
    const int id = lds[j * stride + t];
    if (id < 0 || id >= num_experts) return true;
    for (int i = 0; i < j; ++i)
      if (lds[i * stride + t] == id) return true;
    return false;
  }
};

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

// The token axis is cut into `splits` ranges of tokens_per_split tokens;
// workgroup (e, s) examines range s for expert e, so that every range is about
// one chunk.  The per-range counts go to split_counts[e * splits + s].
// The expert-0 workgroup of each range also marks the top-k positions that
// route nowhere (token_row = -1); the place kernel fills in the others.
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(
    const int32_t* __restrict__ ids, int64_t tokens, int topk, int64_t tokens_per_split,
    int num_experts, int32_t* __restrict__ split_counts, int32_t* __restrict__ token_row) {
  __shared__ int32_t chunk[kChunkLds];
  const int e = blockIdx.x, sp = blockIdx.y;
  const int64_t first = (int64_t)sp * tokens_per_split;
  const int64_t last = first + tokens_per_split < tokens ? first + tokens_per_split : tokens;
  const IdChunks ch(ids, last, topk);
  int32_t v[kIdsPerThread];
  if (first < last) ch.load(first, v);
  int n = 0;
  for (int64_t t0 = first; t0 < last; t0 += ch.ct) {
    __syncthreads();   // the previous chunk has been examined
    ch.store(v, chunk);
    __syncthreads();
    if (t0 + ch.ct < last) ch.load(t0 + ch.ct, v);   // in flight meanwhile
    const int64_t nt = ch.count(t0);
    for (int t = threadIdx.x; t < nt; t += kRouteThreads) {
      n += ch.hit(chunk, t, e);
      if (e == 0)
        for (int j = 0; j < topk; ++j)
          if (ch.dead(chunk, t, j, num_experts)) token_row[(t0 + t) * topk + j] = -1;
    }
  }
  int total;
  block_exclusive_scan(n, &total);
  if (threadIdx.x == 0) split_counts[(int64_t)e * gridDim.y + sp] = total;
}

// One workgroup; num_experts <= kRouteThreads.  Sums the range counts of
// each expert into counts[e], turns them into exclusive prefixes in place
// (the first row of each range's tokens inside the expert's run), and lays
// the runs out.
__global__ __launch_bounds__(kRouteThreads) void route_offsets_kernel(
    int32_t* __restrict__ split_counts, int splits, int32_t* __restrict__ counts,
    int num_experts, int32_t* __restrict__ offsets, int32_t* __restrict__ block_expert,
    int64_t nblocks) {
  __shared__ int off[kRouteThreads + 1];
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < num_experts) {
    for (int sp = 0; sp < splits; ++sp) {
      const int c = split_counts[e * splits + sp];
      split_counts[e * splits + sp] = cnt;
      cnt += c;
    }
    counts[e] = cnt;
  }
  const int padded = e < num_experts ? (cnt + kGroup - 1) / kGroup * kGroup : 0;
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

// Workgroup e < num_experts places expert e's tokens in ascending token
// order: in each round of consecutive tokens an exclusive scan of the hits
// gives each hit its rank.  Workgroup num_experts marks the rows past the
// last run as padding.
__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(
    const int32_t* __restrict__ ids, int64_t tokens, int topk, int64_t tokens_per_split,
    int num_experts, const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ split_base, int32_t* __restrict__ row_token,
    int32_t* __restrict__ token_row, int64_t m_cap) {
  __shared__ int32_t chunk[kChunkLds];
  const int e = blockIdx.x, sp = blockIdx.y;
  if (e == num_experts) {
    if (sp == 0)
      for (int64_t r = offsets[num_experts] + threadIdx.x; r < m_cap; r += kRouteThreads)
        row_token[r] = -1;
    return;
  }
  const int64_t first = (int64_t)sp * tokens_per_split;
  const int64_t last = first + tokens_per_split < tokens ? first + tokens_per_split : tokens;
  const int64_t base = offsets[e] + split_base[(int64_t)e * gridDim.y + sp];
  const IdChunks ch(ids, last, topk);
  int32_t v[kIdsPerThread];
  if (first < last) ch.load(first, v);
  int64_t placed = 0;
  for (int64_t t0 = first; t0 < last; t0 += ch.ct) {
    __syncthreads();
    ch.store(v, chunk);
    __syncthreads();
    if (t0 + ch.ct < last) ch.load(t0 + ch.ct, v);
    const int64_t nt = ch.count(t0);
    for (int r0 = 0; r0 < nt; r0 += kRouteThreads) {
      const int t = r0 + threadIdx.x;
      const int h = t < nt ? ch.hit(chunk, t, e) : 0;
      int total;
      const int rank = block_exclusive_scan(h, &total);
      if (h) {
        const int64_t row = base + placed + rank;
        row_token[row] = (int32_t)(t0 + t);
        token_row[(t0 + t) * topk + ch.first(chunk, t, e)] = (int32_t)row;
      }
      placed += total;
    }
  }
  if (sp == 0) {   // the padding rows at the end of the expert's run
    const int64_t end = offsets[e + 1];
    for (int64_t r = offsets[e] + counts[e] + threadIdx.x; r < end; r += kRouteThreads)
      row_token[r] = -1;
  }
}

// 1x128 quantize of every token row, written into each row of the layout
// that holds the token (token_row), plus the padding rows (zeros: code 0,
// scale 1).  Items [0, tokens) are token rows, one wave each, read once and
// quantized once with 16-byte loads; items tokens + b clear the padding rows
// of 128-row block b.
//
// A wave issues all loads of a chunk of its row (up to kChunkLoads 16-byte
// loads per lane) and the token's destination rows (lane j holds the j-th)
// before any store, quantizes the chunk into registers, and only then writes
// it to every destination row, reading each row index from a lane with
// readlane.  The vector-memory counter counts stores as well as loads and
// completes in order, so a load issued after stores can only be waited for
// by waiting for those stores too: no load sits between the stores of a
// chunk.
constexpr int kChunkLoads = 16;   // 8192 BF16 or 4096 FP32 columns per chunk

template <class T>
__global__ __launch_bounds__(256) void route_scatter_quant_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ token_row,
    const int32_t* __restrict__ row_token, uint8_t* __restrict__ q, float* __restrict__ sa,
    int64_t tokens, int topk, int64_t hidden, int64_t m_cap) {
  constexpr int EPL = RowVec<T>::kElems;   // elements per lane per load
  constexpr int LPG = kGroup / EPL;        // lanes per 128-column group
  constexpr int SPAN = 64 * EPL;           // columns per wave load
  constexpr int U = kChunkLoads;
  const int lane = threadIdx.x & 63;
  const int64_t items = tokens + m_cap / kGroup;
  // Workgroup b runs on XCD b % 8 (workgroups are dealt to the XCDs in
  // turn).  Numbering the items so that each XCD takes a contiguous run of
  // them keeps consecutive tokens, whose destination rows share the lines of
  // the scale array, on one XCD, so those lines fill up in one L2 instead
  // of leaving eight of them as partial lines.
  const int64_t G = gridDim.x;
  const int64_t b = G % 8 == 0 ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int64_t it = b * 4 + (threadIdx.x >> 6); it < items; it += G * 4) {
    if (it < tokens) {
      const T* xr = x + it * hidden;
      const int32_t* rows = token_row + it * topk;
      int rv = 0;   // destination row j0 + lane of the token
      for (int64_t c0 = 0; c0 < hidden; c0 += U * SPAN) {
        if (c0 == 0 || topk > 64) rv = lane < topk ? rows[lane] : -1;
        uint4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t col = c0 + u * SPAN + lane * EPL;
          raw[u] = col < hidden ? *reinterpret_cast<const uint4*>(xr + col) : make_uint4(0, 0, 0, 0);
        }
        uint32_t code[U][EPL / 4];
        float sc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          float f[EPL];
          RowVec<T>::widen(raw[u], f);
          float m = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) m = fmaxf(m, fabsf(f[e]));
          const float amax = group_max<LPG>(m);
          sc[u] = amax == 0.f ? 1.f : amax / kE4m3Max;
#pragma unroll
          for (int e = 0; e < EPL / 4; ++e)
            code[u][e] = pack4_e4m3(make_float4(f[4 * e] / sc[u], f[4 * e + 1] / sc[u],
                                                f[4 * e + 2] / sc[u], f[4 * e + 3] / sc[u]));
        }
        for (int j0 = 0; j0 < topk; j0 += 64) {
          // more than 64 destinations: the next 64 row indices (this load,
          // like the reload of the first 64 for a later chunk, waits for the
          // stores before it; top-k routings stay far below 64)
          if (j0 > 0) rv = j0 + lane < topk ? rows[j0 + lane] : -1;
          const int nj = topk - j0 < 64 ? topk - j0 : 64;
          for (int j = 0; j < nj; ++j) {
            const int64_t r = __builtin_amdgcn_readlane(rv, j);
            if (r < 0) continue;
            uint8_t* qr = q + r * hidden;
#pragma unroll
            for (int u = 0; u < U; ++u) {
              const int64_t col = c0 + u * SPAN + lane * EPL;
              if (col < hidden) {
                if constexpr (EPL == 4)
                  store_nt(qr + col, code[u][0]);
                else
                  store_nt(qr + col, code[u][0], code[u][1]);
                if ((lane & (LPG - 1)) == 0) sa[(col / kGroup) * m_cap + r] = sc[u];
              }
            }
          }
        }
      }
    } else {
      // padding rows of one 128-row block: code 0, scale 1
      const int64_t r0 = (it - tokens) * kGroup;
      for (int h = 0; h < 2; ++h) {
        const int64_t mine = r0 + h * 64 + lane;
        uint64_t pad = __ballot(row_token[mine] < 0);
        while (pad) {
          const int i = __builtin_ctzll(pad);
          pad &= pad - 1;
          const int64_t r = r0 + h * 64 + i;
          for (int64_t c = (int64_t)lane * 16; c < hidden; c += 64 * 16)
            store_nt(q + r * hidden + c, 0u, 0u, 0u, 0u);
          for (int64_t kb = lane; kb < hidden / kGroup; kb += 64) sa[kb * m_cap + r] = 1.f;
        }
      }
    }
  }
}

hipError_t launch_route_quantize(const void* x, bool bf16, int64_t tokens, int64_t hidden,
                                 const int32_t* ids, int topk, int num_experts, int64_t m_cap,
                                 uint8_t* q, float* sa, int32_t* block_expert, int32_t* row_token,
                                 int32_t* token_row, int32_t* counts, int32_t* offsets,
                                 hipStream_t stream) {
  // token ranges of about one chunk each, at most kMaxRouteSplits of them; the
  // range counts live in the first num_experts * splits words of sa until the
  // place kernel has read them (sa holds m_cap * hidden/128 >= m_cap >= 127 *
  // num_experts words); the quantize that overwrites sa runs after it
  const int64_t ct = kChunkInts / topk;
  int64_t splits = (tokens + ct - 1) / ct;
  if (splits > kMaxRouteSplits) splits = kMaxRouteSplits;
  const int64_t per = (tokens + splits - 1) / splits;
  int32_t* split_counts = reinterpret_cast<int32_t*>(sa);
  hipLaunchKernelGGL(route_count_kernel, dim3(num_experts, (unsigned)splits), dim3(kRouteThreads),
                     0, stream, ids, tokens, topk, per, num_experts, split_counts, token_row);
  hipLaunchKernelGGL(route_offsets_kernel, dim3(1), dim3(kRouteThreads), 0, stream, split_counts,
                     (int)splits, counts, num_experts, offsets, block_expert, m_cap / kGroup);
  hipLaunchKernelGGL(route_place_kernel, dim3(num_experts + 1, (unsigned)splits),
                     dim3(kRouteThreads), 0, stream, ids, tokens, topk, per, num_experts, counts,
                     offsets, split_counts, row_token, token_row, m_cap);
  const int64_t items = tokens + m_cap / kGroup;
  const int64_t blocks = ((items + 3) / 4 + 7) / 8 * 8;   // whole rounds of the eight XCDs
  const unsigned grid = (unsigned)(blocks < (1 << 20) ? blocks : (1 << 20));
  if (bf16)
    hipLaunchKernelGGL(route_scatter_quant_kernel<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       (const uint16_t*)x, token_row, row_token, q, sa, tokens, topk, hidden,
                       m_cap);
  else
    hipLaunchKernelGGL(route_scatter_quant_kernel<float>, dim3(grid), dim3(256), 0, stream,
                       (const float*)x, token_row, row_token, q, sa, tokens, topk, hidden, m_cap);
  return hipGetLastError();
}

}  // namespace fg8
