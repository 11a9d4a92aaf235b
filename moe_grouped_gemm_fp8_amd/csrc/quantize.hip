// FP32 or BF16 -> e4m3 quantization with fine-grained scales.
//
// Scale then convert: the FP32 tensor is multiplied by a scaling factor and
// turned into FP8 (cuda-deepseek blog, hrletsgo.me, list item 5), per tile
// rather than per tensor as that blog's own comments ask for, at the
// granularities DeepGEMM uses (1x128 activation groups, 128x128 weight
// blocks), plus MX blocks of 32 elements sharing one power-of-two exponent
// (aitrends.kr B200 article, MXFP8 glossary entry).
//
// The kernels are HBM-bound streams (4 or 2 B read + ~1.03 B written per
// element): wide loads, the amax of a group by butterfly exchanges among the
// lanes that hold it (or through LDS where a group spans waves), packed
// stores of codes.  A fourth kind groups 128 rows of each column instead of
// 128 columns of each row and writes the codes transposed (the token-axis
// quantization of the weight gradient).  Results are bit-exact with the
// format rules in fg8.h: the scale is the correctly rounded float32 quotient
// amax / 448, elements use a correctly rounded float32 division by it, and
// the MX exponent comes straight from the float bits of amax.
#include "fg8_device.h"
#include "fg8_internal.h"

namespace fg8 {

// Four consecutive source elements as float4.  BF16 sources (raw 16-bit
// words) widen exactly, so a BF16 tensor quantizes exactly like its FP32
// value.
template <class T>
__device__ __forceinline__ float4 load4(const T* p);
template <>
__device__ __forceinline__ float4 load4<float>(const float* p) {
  return *reinterpret_cast<const float4*>(p);
}
template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}
// The same with the non-temporal hint.
template <class T>
__device__ __forceinline__ float4 load4_nt(const T* p) {
  if constexpr (sizeof(T) == 4) {
    const uint4 u = load_nt16(p);
    return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z),
                       __uint_as_float(u.w));
  } else {
    const uint2 u = load_nt8(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
}

// ---------------------------------------------------------------- 1 x 128
// Row streaming: a wave owns one run of columns of one row (the whole row when
// there are enough rows to fill the chip, else a shorter run) and walks it with
// 16-byte loads, kQUnroll of them in flight per lane.  One load instruction of
// a wave covers 64 x 16 bytes = 2 (FP32) or 4 (BF16) groups of 128 columns; the
// 32 or 16 lanes that hold a group reduce its amax with butterfly exchanges.
// Scales are written K-block major.
constexpr int kQUnroll = 8;

template <class T, int WPB>
__global__ __launch_bounds__(64 * WPB) void quant_1x128_kernel(const T* __restrict__ x,
                                                          uint8_t* __restrict__ q,
                                                          float* __restrict__ s, uint32_t rows,
                                                          int64_t cols, int64_t seg_cols,
                                                          uint32_t nseg, uint32_t items) {
  constexpr int EPL = RowVec<T>::kElems;   // elements per lane per load
  constexpr int LPG = kGroup / EPL;        // lanes per 128-column group
  constexpr int SPAN = 64 * EPL;           // columns per wave load
  const int lane = threadIdx.x & 63;
  // waves walk the items independently (there is no barrier in this kernel)
  // Workgroup b runs on XCD b % 8; on the large launches, numbering the
  // items so that each XCD takes a contiguous run of rows keeps the scale
  // lines (32 rows of one K block) that neighbouring rows share in one XCD's
  // L2 (69,632 x 7168: 0.489 -> 0.480 ms; the one-wave launches of a few
  // rows keep the plain order, which measured 0.04 us faster there).
  // The item decode divides in 32 bits (the host keeps items below 2^31):
  // GPUs have no integer divider, and the 64-bit quotients it used to take
  // cost ~0.3 us of a 64-row launch (64 x 7168: 3.82 -> 3.53 us).
  // One-wave launches have exactly one item per workgroup (grid == items),
  // so their stride needs no load of the grid size.
  const uint32_t G = WPB == 1 ? items : gridDim.x;
  const uint32_t b = WPB > 1 && G % 8 == 0 ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8
                                           : blockIdx.x;
  for (uint32_t it = b * WPB + (threadIdx.x >> 6); it < items; it += G * WPB) {
    const uint32_t grow = it / nseg;              // row over all batches
    const int64_t c_begin = (int64_t)(it - grow * nseg) * seg_cols;
    const int64_t c_end = c_begin + seg_cols < cols ? c_begin + seg_cols : cols;
    const uint32_t b = grow / rows, r = grow - b * rows;
    const T* xr = x + (int64_t)grow * cols;
    uint8_t* qr = q + (int64_t)grow * cols;
    float* sb = s + (int64_t)b * (cols / kGroup) * rows + r;
    for (int64_t c0 = c_begin; c0 < c_end; c0 += kQUnroll * SPAN) {
      uint4 raw[kQUnroll];
#pragma unroll
      for (int u = 0; u < kQUnroll; ++u) {
        if (c0 + u * SPAN >= c_end) break;   // past the run (uniform), as below
        const int64_t col = c0 + u * SPAN + lane * EPL;
        // (non-temporal loads on the multi-wave launches only: the one-wave
        // ones are decode-sized, where the hint cost latency)
        raw[u] = col >= c_end ? make_uint4(0, 0, 0, 0)
                 : WPB == 1   ? *reinterpret_cast<const uint4*>(xr + col)
                              : load_nt16(xr + col);
      }
#pragma unroll
      for (int u = 0; u < kQUnroll; ++u) {
        // a load wholly past the run: so are the rest (a uniform branch; the
        // amax exchanges of dead loads had cost ~1.1 us of a 64-row launch)
        if (c0 + u * SPAN >= c_end) break;
        const int64_t col = c0 + u * SPAN + lane * EPL;
        float f[EPL];
        RowVec<T>::widen(raw[u], f);
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) m = fmaxf(m, fabsf(f[e]));
        const float amax = group_max<LPG>(m);
        const float sc = amax == 0.f ? 1.f : amax / kE4m3Max;
        if (col < c_end) {
          uint32_t code[EPL / 4];
#pragma unroll
          for (int e = 0; e < EPL / 4; ++e)
            code[e] = pack4_e4m3(make_float4(f[4 * e] / sc, f[4 * e + 1] / sc, f[4 * e + 2] / sc,
                                             f[4 * e + 3] / sc));
          if constexpr (EPL == 4)
            store_nt(qr + col, code[0]);
          else
            store_nt(qr + col, code[0], code[1]);
          if ((lane & (LPG - 1)) == 0) sb[(col / kGroup) * rows] = sc;
        }
      }
    }
  }
}

// Decode-sized activations: one wave per span of 64 x 16 bytes of one row
// (whole spans only), no loops.  Fewer instructions between the load and the
// stores than the run-walking kernel above: 64 x 7168 FP32 2.40 -> 2.1 us.
template <class T>
__global__ __launch_bounds__(64) void quant_1x128_span_kernel(const T* __restrict__ x,
                                                              uint8_t* __restrict__ q,
                                                              float* __restrict__ s, uint32_t rows,
                                                              uint32_t cols, uint32_t spans) {
  constexpr int EPL = RowVec<T>::kElems;   // elements per lane
  constexpr int LPG = kGroup / EPL;        // lanes per 128-column group
  constexpr int SPAN = 64 * EPL;           // columns per wave
  const int lane = threadIdx.x;
  const uint32_t grow = blockIdx.x / spans;   // grid == rows over all batches * spans
  const uint32_t col = (blockIdx.x - grow * spans) * SPAN + lane * EPL;
  const uint32_t b = grow / rows, r = grow - b * rows;
  const uint4 raw = *reinterpret_cast<const uint4*>(x + (size_t)grow * cols + col);
  float f[EPL];
  RowVec<T>::widen(raw, f);
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) m = fmaxf(m, fabsf(f[e]));
  const float amax = group_max<LPG>(m);
  const float sc = amax == 0.f ? 1.f : amax / kE4m3Max;
  uint32_t code[EPL / 4];
#pragma unroll
  for (int e = 0; e < EPL / 4; ++e)
    code[e] = pack4_e4m3(make_float4(f[4 * e] / sc, f[4 * e + 1] / sc, f[4 * e + 2] / sc,
                                     f[4 * e + 3] / sc));
  uint8_t* qp = q + (size_t)grow * cols + col;
  if constexpr (EPL == 4)
    *reinterpret_cast<uint32_t*>(qp) = code[0];
  else
    *reinterpret_cast<uint2*>(qp) = make_uint2(code[0], code[1]);
  if ((lane & (LPG - 1)) == 0) s[((size_t)b * (cols / kGroup) + col / kGroup) * rows + r] = sc;
}

// Column-run length for the 1x128 kernel: whole rows when the rows alone give
// enough waves to fill the chip, else runs of whole wave loads.
static int64_t q1_seg_cols(int64_t rows, int64_t cols, int elems) {
  const int64_t span = 64 * (int64_t)elems;
  const int64_t spans = (cols + span - 1) / span;
  constexpr int64_t kTargetWaves = 8192;
  int64_t per = rows * spans / kTargetWaves;
  per = per < 1 ? 1 : per > spans ? spans : per;
  return per * span;
}

template <class T>
static hipError_t launch_q1(const T* x, int64_t rows_all, int64_t rows, int64_t cols, uint8_t* q,
                            float* s, hipStream_t stream) {
  const int64_t seg = q1_seg_cols(rows_all, cols, RowVec<T>::kElems);
  const int64_t nseg = (cols + seg - 1) / seg;
  const int64_t items = rows_all * nseg;
  if (items >= (int64_t(1) << 31) || rows >= (int64_t(1) << 31)) return hipErrorInvalidValue;
  const int64_t span = 64 * (int64_t)RowVec<T>::kElems;
  if (cols % span == 0 && cols < (int64_t(1) << 31) && rows_all * (cols / span) < 4096) {
    const unsigned grid = (unsigned)(rows_all * (cols / span));
    hipLaunchKernelGGL(quant_1x128_span_kernel<T>, dim3(grid), dim3(64), 0, stream, x, q, s,
                       (uint32_t)rows, (uint32_t)cols, (uint32_t)(cols / span));
    return hipGetLastError();
  }
  // Few items whose rows do not split into whole spans: one wave per
  // workgroup, which had measured 3.68 against 3.85 us per launch on
  // 64 x 1536 (64 x 7168 unchanged) before the span kernel took those.
  if (items < 4096) {
    const unsigned grid = (unsigned)items;
    hipLaunchKernelGGL((quant_1x128_kernel<T, 1>), dim3(grid), dim3(64), 0, stream, x, q, s,
                       (uint32_t)rows, cols, seg, (uint32_t)nseg, (uint32_t)items);
    return hipGetLastError();
  }
  const int64_t blocks = ((items + 3) / 4 + 7) / 8 * 8;   // whole rounds of the eight XCDs
  const unsigned grid = (unsigned)(blocks < (1 << 20) ? blocks : (1 << 20));
  hipLaunchKernelGGL((quant_1x128_kernel<T, 4>), dim3(grid), dim3(256), 0, stream, x, q, s,
                     (uint32_t)rows, cols, seg, (uint32_t)nseg, (uint32_t)items);
  return hipGetLastError();
}

// ---------------------------------------------------------- 1 x 128, transposed
// Groups of 128 consecutive ROWS of each column (the token axis of an
// activation), codes written transposed: q[c][r], scales [rows/128][cols].
// A workgroup takes a 128-row x 64-column tile: thread t loads rows
// 8 (t / 16) .. +7 of columns 4 (t % 16) .. +3 as float4 / 8-byte BF16 rows
// (coalesced along the row), the 16 row parts of a column meet in LDS for the
// amax, and the codes are transposed through LDS so that every column's 128
// codes leave as whole 128-byte lines.
template <class T>
__global__ __launch_bounds__(256) void quant_1x128_t_kernel(const T* __restrict__ x,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ s, int64_t rows,
                                                            int64_t cols) {
  __shared__ float part[16][64];
  __shared__ float col_scale[64];
  __shared__ uint32_t codes[64][33];   // 64 columns x 32 dwords of codes, padded
  const int64_t b = blockIdx.z;
  const int64_t rb = blockIdx.y;
  const int64_t c_tile = (int64_t)blockIdx.x * 64;
  const int t = threadIdx.x, cq = t & 15, rp = t >> 4;
  const T* xb = x + b * rows * cols;
  const int64_t r0 = rb * kGroup + rp * 8;
  float4 v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = load4(xb + (r0 + i) * cols + c_tile + cq * 4);
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m.x = fmaxf(m.x, fabsf(v[i].x)); m.y = fmaxf(m.y, fabsf(v[i].y));
    m.z = fmaxf(m.z, fabsf(v[i].z)); m.w = fmaxf(m.w, fabsf(v[i].w));
  }
  *reinterpret_cast<float4*>(&part[rp][cq * 4]) = m;
  __syncthreads();
  if (t < 64) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, part[j][t]);
    const float sc = amax == 0.f ? 1.f : amax / kE4m3Max;
    col_scale[t] = sc;
    s[b * (rows / kGroup) * cols + rb * cols + c_tile + t] = sc;
  }
  __syncthreads();
  const float4 sc4 = *reinterpret_cast<const float4*>(&col_scale[cq * 4]);
  const float scj[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 w = v[i];
      e[i] = (j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w) / scj[j];
    }
    codes[cq * 4 + j][rp * 2] = pack4_e4m3(make_float4(e[0], e[1], e[2], e[3]));
    codes[cq * 4 + j][rp * 2 + 1] = pack4_e4m3(make_float4(e[4], e[5], e[6], e[7]));
  }
  __syncthreads();
  // two passes over columns cc = t / 8 + 32 h of the tile, 16-byte piece t % 8
  // of their 128 codes: every store instruction writes eight whole lines,
  // which the non-temporal hint suits (0.312 -> 0.308 ms on 67,712 x 7168;
  // with each thread writing one 32-byte piece in two halves instead, the
  // hint had cost 8%)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cc = (t >> 3) + 32 * h, piece = t & 7;
    uint8_t* dst = q + b * cols * rows + (c_tile + cc) * rows + rb * kGroup + piece * 16;
    const uint32_t* src = &codes[cc][piece * 4];
    store_nt(dst, src[0], src[1], src[2], src[3]);
  }
}

// ---------------------------------------------------------------- 128 x 128
// Block: 256 threads over one 128x128 block.  Thread t owns column chunk
// (t % 32) * 4 of rows t / 32 + 8 i, i = 0..15: 16 float4 in registers, the
// amax is reduced across the wave and then across the 4 waves through LDS.
template <class T>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const T* __restrict__ x,
                                                            uint8_t* __restrict__ q,
                                                            float* __restrict__ s, int64_t rows,
                                                            int64_t cols) {
  __shared__ float wave_max[4];
  const int64_t b = blockIdx.z;
  const int cb = blockIdx.x, rb = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t kblocks = cols / kGroup;
  const int64_t rblocks = (rows + kGroup - 1) / kGroup;
  const T* xb = x + b * rows * cols;
  uint8_t* qb = q + b * rows * cols;
  const int64_t col = (int64_t)cb * kGroup + (tid & 31) * 4;
  const int64_t r0 = (int64_t)rb * kGroup + (tid >> 5);

  float4 v[16];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + 8 * i;
    v[i] = r < rows ? load4_nt(xb + r * cols + col) : make_float4(0.f, 0.f, 0.f, 0.f);
    m = fmaxf(m, abs_max4(v[i]));
  }
  m = group_max<64>(m);
  if ((tid & 63) == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
  const float sc = amax == 0.f ? 1.f : amax / kE4m3Max;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + 8 * i;
    if (r < rows) {
      const float4 y = make_float4(v[i].x / sc, v[i].y / sc, v[i].z / sc, v[i].w / sc);
      store_nt(qb + r * cols + col, pack4_e4m3(y));
    }
  }
  if (tid == 0) s[b * rblocks * kblocks + (int64_t)rb * kblocks + cb] = sc;
}

// ---------------------------------------------------------------- MX 1 x 32
// The tensor is a flat run of 32-element blocks (cols % 32 == 0, so no block
// crosses a row) and the E8M0 array is indexed by the same block number.
// Eight lanes hold one block; a grid-stride loop walks the blocks.
template <class T>
__global__ __launch_bounds__(256) void quant_mx_kernel(const T* __restrict__ x,
                                                       uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ e, int64_t nblocks) {
  const int64_t stride = (int64_t)gridDim.x * 32;   // blocks per grid sweep (256 threads / 8)
  const int sub = threadIdx.x & 7;
  for (int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3); blk < nblocks; blk += stride) {
    const float4 v = load4_nt(x + blk * kMxBlock + sub * 4);
    const float amax = group_max<8>(abs_max4(v));
    // floor(log2 amax) - 8 from the exponent field; subnormal or zero amax
    // lands below -127 and is clamped there with the largest normal result.
    const int expf = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    const int E = max(expf - 127 - 8, -127);
    const float inv = __uint_as_float((uint32_t)(127 - E) << 23);   // 2^-E, exact
    const float4 y = make_float4(v.x * inv, v.y * inv, v.z * inv, v.w * inv);
    store_nt(q + blk * kMxBlock + sub * 4, pack4_e4m3(y));
    if (sub == 0) e[blk] = (uint8_t)(E + 127);
  }
}

template <class T>
static hipError_t launch_quantize_t(const T* x, int64_t batch, int64_t rows, int64_t cols, int kind,
                                    uint8_t* q, void* scales, hipStream_t stream) {
  if (kind == 0) {
    return launch_q1<T>(x, batch * rows, rows, cols, q, (float*)scales, stream);
  } else if (kind == 1) {
    dim3 grid((unsigned)(cols / kGroup), (unsigned)((rows + kGroup - 1) / kGroup), (unsigned)batch);
    hipLaunchKernelGGL(quant_128x128_kernel<T>, grid, dim3(256), 0, stream, x, q, (float*)scales,
                       rows, cols);
  } else if (kind == 3) {
    dim3 grid((unsigned)(cols / 64), (unsigned)(rows / kGroup), (unsigned)batch);
    hipLaunchKernelGGL(quant_1x128_t_kernel<T>, grid, dim3(256), 0, stream, x, q, (float*)scales,
                       rows, cols);
  } else {
    const int64_t nblocks = batch * rows * cols / kMxBlock;
    const int64_t want = (nblocks + 31) / 32;
    const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(quant_mx_kernel<T>, dim3(grid), dim3(256), 0, stream, x, q,
                       (uint8_t*)scales, nblocks);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, bool bf16, int64_t batch, int64_t rows, int64_t cols,
                           int kind, uint8_t* q, void* scales, hipStream_t stream) {
  if (bf16)
    return launch_quantize_t((const uint16_t*)x, batch, rows, cols, kind, q, scales, stream);
  return launch_quantize_t((const float*)x, batch, rows, cols, kind, q, scales, stream);
}

}  // namespace fg8
