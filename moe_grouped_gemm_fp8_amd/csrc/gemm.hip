// Block-scaled FP8 GEMM with two-level accumulation, its MoE grouped forms,
// and the MXFP8 variant, for gfx950.
//
// What is computed: D[m][n] = sum_kb (sa[kb][m] * sb[n/128][kb]) *
// sum_{k in kb} qa[m][k] * qb[n][k].  The inner sum over one 128-wide K block
// is one v_mfma_f32_16x16x128_f8f6f4 (FP8 x FP8 -> FP32); the outer sum is an
// FP32 fused multiply-add per K block in registers.  That is the two-level
// accumulation of DeepGEMM (release news, ctol-kr.com, section 1 "FP8": the
// tensor-core FP8 partial sums are promoted into FP32 accumulators on the
// CUDA cores at a fixed interval); here the interval is one scale block, which
// the per-128 scales force.  The MXFP8 path (aitrends.kr B200 article, MXFP8
// section) instead hands each lane's E8M0 byte to
// v_mfma_scale_f32_16x16x128_f8f6f4 and accumulates straight through K.
//
// Work decomposition (one wavefront = 64 lanes, 4 or 8 waves per workgroup):
//   * a workgroup owns a BM x BN output tile; waves split it WAVES_M x WAVES_N;
//     each wave holds its (BM/WAVES_M) x (BN/WAVES_N) FP32 accumulators in
//     VGPRs as 16x16 MFMA tiles;
//   * per 128-wide K block the A and B tiles (BM x 128 and BN x 128 bytes) and
//     their scales are copied from global memory straight into LDS with
//     global_load_lds_dwordx4 / _dword (no staging registers), STAGES blocks
//     in flight;
//   * LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by
//     (r >> 1) & 7, so the MFMA operand reads (ds_read_b128 of one chunk
//     from 16 consecutive rows) hit distinct banks;
//   * a persistent grid walks a linear list of work units: dense tiles
//     (optionally split along K with a deterministic last-arriver reduction),
//     contiguous-layout tiles whose expert comes from block_expert (with an
//     optional gated epilogue that quantizes the activation for the next
//     GEMM; 256-row tiles cover pairs of 128-row blocks, and a pair that
//     straddles two experts runs as two half-height units), masked-layout
//     tiles enumerated from the device-side valid counts, or K-grouped tiles
//     whose K range comes from per-group offsets (the weight gradient, 1x128
//     scales on both operands);
//   * the 256 x 256 tiles are dealt so that each XCD runs a compact block of
//     them (a contiguous run of ids per XCD, walked four tile rows at a time),
//     and their column steps are fenced so that no more than two columns of
//     partial sums are live (the 128 accumulators per lane leave no room).
//
// Lane layout (measured on gfx950 by the probe tests): in the 16x16x128 MFMA
// lane l = i + 16 g holds row i of A (column i of B) with K = 16 g .. 16 g + 15
// in bytes 0-15 and K = 64 + 16 g .. +15 in bytes 16-31; result register v of
// lane l is D[4 (l / 16) + v][l % 16]; with scales, the E8M0 byte of lane
// i + 16 c scales K block c (32 elements) of row i.
#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

#include "fg8_device.h"
#include "fg8_internal.h"

namespace fg8 {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int STAGES_, int OCC_, int KS_ = 1,
          bool SPREAD_ = false>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int WAVES = WAVES_M * WAVES_N, THREADS = 64 * WAVES;
  static constexpr int STAGES = STAGES_, OCC = OCC_;
  static constexpr int KS = KS_;   // 128-wide K blocks per pipeline stage (one barrier each)
  // SPREAD: the next stage's loads are issued between the column tiles of the
  // compute instead of all at once after the barrier
  static constexpr bool SPREAD = SPREAD_;
  // split-K is compiled only into the decode-sized configurations (the large
  // tiles have no registers to spare for the partial sums)
  static constexpr bool SPLITK = WAVES == 4 && BM <= 128 && BN <= 128;
  // PIN: the compute of each column tile is fenced off from the next
  // (sched_barrier), so the scheduler cannot hoist every B fragment read and
  // MFMA of the K block ahead of the promotion: the 256 x 256 tile's
  // 128 accumulators per lane leave no room for more than two columns of
  // partial sums in flight
  static constexpr bool PIN = BM * BN >= 256 * 256;
  // LATE: with two stages, the waves in the second half of the workgroup
  // issue the next stage's loads after column tile LATE of the compute
  // instead of right after the barrier (-1: every wave issues at once).
  // Waves w and w + 4 share a SIMD, and an LDS-DMA instruction holds up its
  // wave until the memory pipeline takes it, so with all waves issuing
  // together both waves of a SIMD stall at once; staggered, one of them is
  // issuing MFMAs while the other waits.  Measured on the MoE W1: after
  // column tile 0, 1, 2 or 3: 1.84, 1.82, 1.80, 1.82 ms (all at once 2.00).
  // The K-grouped kernel issues after column tile 1 (kernel: LATE_AT).
  static constexpr int LATE = PIN && !SPREAD ? 2 : -1;
  static constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  static constexpr int TM = WM / 16, TN = WN / 16;
  // One stage holds KS K blocks, each laid out as: A tile | B tile | A row
  // scales (FP32 sa or E8M0 dwords) | B row scales (E8M0 dwords, MX only) |
  // one B-block scale per wave (FP32).
  static constexpr int A_BYTES = BM * kGroup, B_BYTES = BN * kGroup;
  // SPLITB: a wave's columns may straddle two 128-column B blocks (wave tile
  // width not dividing 128); each wave then keeps both blocks' scales and
  // applies them per 16-column tile
  static constexpr bool SPLITB = (128 % (BN / WAVES_N)) != 0;
  static constexpr int SA_BYTES = BM * 4, SB_BYTES = BN * 4, SBW_BYTES = (SPLITB ? 8 : 4) * WAVES;
  static constexpr int BLOCK_BYTES = A_BYTES + B_BYTES + SA_BYTES + SB_BYTES + SBW_BYTES;
  static constexpr int STAGE_BYTES = KS * BLOCK_BYTES;
  // rows each wave copies per stage; one 16-byte LDS-DMA load covers 8 rows
  static constexpr int A_ROWS = BM / WAVES, B_ROWS = BN / WAVES;
  static constexpr int A_LOADS = A_ROWS / 8, B_LOADS = B_ROWS / 8;
  static_assert(A_ROWS % 8 == 0 && B_ROWS % 8 == 0, "every wave copies whole groups of 8 rows");
  static_assert(WAVES == 4 || WAVES == 8, "four or eight waves per workgroup");
  static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be whole 16x16 MFMA tiles");
  static_assert(WN <= 128 && ((128 % WN) == 0 || SPLITB), "a wave's columns span at most two 128-blocks");
  static_assert(!SPLITB || WN < 128, "two B blocks per wave at most");
  static_assert(A_ROWS <= 64 && B_ROWS <= 64, "one scale load per wave must cover its rows");
  static_assert((BLOCK_BYTES - SBW_BYTES) % 16 == 0 && SBW_BYTES % 16 == 0, "aligned stage parts");
  static_assert(STAGES >= 2, "need at least double buffering");
  static_assert(STAGE_BYTES % 16 == 0, "stages stay 16-byte aligned");
};

template <int L, int MAXN>
__device__ __forceinline__ void wait_stages_after(int pending) {
  // Wait until at most `pending` later stages (L loads each) are outstanding.
  if constexpr (MAXN <= 0) {
    wait_vmcnt<0>();
  } else {
    if (pending >= MAXN) wait_vmcnt<L * MAXN>();
    else wait_stages_after<L, MAXN - 1>(pending);
  }
}

// Fence between the column steps of a pinned configuration: neither the IR
// passes (memory clobber) nor the machine scheduler move LDS reads or MFMAs
// across it.
__device__ __forceinline__ void pin_step() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// An empty asm that reads and rewrites x: the computation of x (an MFMA
// result, a promoted accumulator) must happen before this point and cannot be
// sunk past the branches that follow it.
__device__ __forceinline__ void pin_value(v4f& x) { asm volatile("" : "+v"(x)); }

// x * sigmoid(x) in FP32 from the hardware exp2 and reciprocal (each within
// a few ulp, so silu is within a few FP32 ulp of its correctly rounded
// value); -0 for very negative x (2^(-x log2 e) overflows to inf, whose
// reciprocal is 0).
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// Tile order for the L2s of the eight XCDs.  A persistent grid of G
// workgroups deals unit u to XCD u % 8; within every whole round of G units,
// xcd_block renumbers them so that each XCD takes a contiguous run of G / 8
// ids, and grouped_tile walks those ids down `gm` rows of tiles before moving
// to the next column, so the tiles an XCD runs together share few A row
// blocks and few B column blocks.  Both are bijections on [0, total).
__device__ __forceinline__ int xcd_block(int u, int total, int G) {
  if (G % 8) return u;
  const int base = (u / G) * G;
  if (base + G > total) return u;
  const int b = u - base;
  return base + (b % 8) * (G / 8) + b / 8;
}
__device__ __forceinline__ void grouped_tile(int id, int m_tiles, int n_tiles, int gm, int& mt,
                                             int& nt) {
  const int per = gm * n_tiles;
  const int grp = id / per, first = grp * gm;
  const int rows = min(m_tiles - first, gm);
  const int r = id - grp * per;
  mt = first + r % rows;
  nt = r / rows;
}

struct Unit {
  int g;            // group (expert)
  int64_t m0, n0;   // tile origin inside the group
  int kb0, kb1;     // K-block range
  int split, tile;  // split-K index and flat tile id
  int rows;         // live rows of this group (dense: M)
};

// BS: the B rows of each unit are read by no other tile row of the launch
// (one tile row of M per group), so their copies carry the non-temporal hint.
template <class C, bool MX, int MODE, bool BS>
__global__ __launch_bounds__(C::THREADS, C::OCC) void gemm_kernel(GemmProblem p) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::STAGES * C::STAGE_BYTES];
  // MXG: the E8M0 scales of the two-stage tiles are fetched for four K blocks
  // at a time (16 bytes per tile row) into two alternating group buffers,
  // [row: BM A rows, then BN B rows][4 dwords, one per K block], instead of
  // one dword per row and K block: half the scale loads, each touching 16
  // rows instead of 32, so a quarter of the cache lines.
  constexpr bool MXG = MX && C::STAGES == 2;
  constexpr int GRP_DWORDS = (C::BM + C::BN) * 4;
  static_assert(!MXG || (!C::SPLITK && C::KS == 1 && C::A_ROWS % 16 == 0 && C::B_ROWS % 16 == 0),
                "grouped E8M0 scales: whole K ranges, one K block per stage, 16-row loads");
  __shared__ __attribute__((aligned(16))) uint32_t mx_grp[MXG ? 2 * GRP_DWORDS : 1];
  __shared__ int tile_prefix[MODE == kMasked ? 1025 : 1];
  __shared__ int flag;

  // the wave index is uniform: held in an SGPR, so are the LDS addresses built on it
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int wm0 = wm * C::WM, wn0 = wn * C::WN;
  const int64_t M = p.M, N = p.N, K = p.K;
  // Taking one field of every 32 bytes of the problem struct here issues
  // all its scalar-cache fetches together, one round trip to
  // kernel-argument memory instead of a chain of dependent ones.
  asm volatile("" ::"s"(p.a), "s"(p.d), "s"(N), "s"(p.valid), "s"(p.q_out), "s"(p.ws_counters));
  const int KB = (int)(K / kGroup);
  const int n_tiles = (int)(((uint32_t)N + C::BN - 1) / C::BN);   // N < 2^31 (C ABI)
  const int splits = MODE == kDense ? p.splits : 1;
  const int64_t nb_blocks = (N + kGroup - 1) / kGroup;

  // ---- enumerate work units
  int total;
  if constexpr (MODE == kMasked) {
    // tiles per group from the device-side counts; exclusive prefix in LDS.
    const int G = p.groups;
    constexpr int PER = 1024 / C::THREADS;   // groups per thread (G <= 1024)
    int local[PER];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = tid * PER + j;
      int v = 0;
      if (e < G) {
        const int64_t rows = p.valid ? min(max((int64_t)p.valid[e], (int64_t)0), M) : M;
        v = (int)((rows + C::BM - 1) / C::BM) * n_tiles;
      }
      local[j] = v;
      sum += v;
    }
    // block-wide exclusive scan of the per-thread sums
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    __shared__ int wave_tot[C::WAVES];
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wave_tot[w];
    int run = base + incl - sum;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = tid * PER + j;
      if (e < G) tile_prefix[e] = run;
      run += local[j];
    }
    if (tid == C::THREADS - 1) tile_prefix[G] = run;   // grand total (G <= 1024)
    __syncthreads();
    total = tile_prefix[G];
  } else if constexpr (MODE == kKGrouped) {
    total = p.groups * (int)((M + C::BM - 1) / C::BM) * n_tiles;
  } else if constexpr (MODE == kContiguous && C::BM == 2 * kGroup) {
    total = 2 * (int)((M + C::BM - 1) / C::BM) * n_tiles;   // pair units, then half units
  } else {
    total = (int)((M + C::BM - 1) / C::BM) * n_tiles * splits;
  }

  v4f acc[C::TM][C::TN];
  const uint32_t lds0 = lds_addr(smem);
  const uint32_t mxg0 = lds_addr(mx_grp);

  // The grid size comes in the problem struct: reading gridDim loads the
  // launch's hidden arguments, a scalar-cache miss on the path to each
  // unit's first loads.
  const int G = p.grid;
  for (int u = blockIdx.x; u < total; u += G) {
    // ---- decode the unit
    Unit w;
    if constexpr (MODE == kMasked) {
      // with the XCD-blocked order an XCD runs consecutive tiles, mostly of
      // one expert, so that expert's A rows are fetched into its L2 once
      const int uu = p.raster > 0 ? xcd_block(u, total, G) : u;
      int lo = 0, hi = p.groups - 1;   // last group with prefix <= uu
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_prefix[mid] <= uu) lo = mid; else hi = mid - 1;
      }
      const int t = uu - tile_prefix[lo];
      w.g = lo;
      w.m0 = (int64_t)(t / n_tiles) * C::BM;
      w.n0 = (int64_t)(t % n_tiles) * C::BN;
      w.kb0 = 0; w.kb1 = KB; w.split = 0; w.tile = u;
      w.rows = p.valid ? (int)min(max((int64_t)p.valid[lo], (int64_t)0), M) : (int)M;
    } else if constexpr (MODE == kKGrouped) {
      const int per = (int)((M + C::BM - 1) / C::BM) * n_tiles;
      w.g = u / per;
      const int t = u - w.g * per;
      w.m0 = (int64_t)(t / n_tiles) * C::BM;
      w.n0 = (int64_t)(t % n_tiles) * C::BN;
      // the group's K blocks, range-checked: [k0, k1) inside [0, KB)
      const int k0 = min(max(p.k_offsets[w.g] / kGroup, 0), KB);
      const int k1 = min(max(p.k_offsets[w.g + 1] / kGroup, k0), KB);
      w.kb0 = k0; w.kb1 = k1; w.split = 0; w.tile = u;
      w.rows = (int)M;
    } else if constexpr (MODE == kContiguous && C::BM == 2 * kGroup) {
      // 256-row tiles over pairs of 128-row blocks.  A pair whose blocks
      // belong to one expert is one unit; a pair that straddles two experts
      // (or ends the layout) is done as two half-height units, one per block
      // and expert, enumerated after every pair unit.  The units of the
      // second kind for a one-expert pair are empty.
      const int64_t mblocks = M / kGroup;
      const int pair_units = (int)((mblocks + 1) / 2) * n_tiles;
      const int h = u >= pair_units ? 1 : 0;
      const int t = u - h * pair_units;
      int pr = t / n_tiles, nt = t % n_tiles;
      if (h == 0 && p.raster > 0)
        grouped_tile(xcd_block(t, pair_units, G), (int)((mblocks + 1) / 2), n_tiles,
                     p.raster, pr, nt);
      const int64_t b0 = 2 * (int64_t)pr;
      w.n0 = (int64_t)nt * C::BN;
      const int e0 = p.block_expert[b0];
      const int e1 = b0 + 1 < mblocks ? p.block_expert[b0 + 1] : -1;
      if (e0 == e1 && b0 + 1 < mblocks) {
        w.g = h == 0 ? e0 : -1;
        w.m0 = b0 * kGroup;
        w.rows = (int)M;
      } else {
        const int64_t b = b0 + h;
        w.g = b < mblocks ? (h == 0 ? e0 : e1) : -1;
        w.m0 = b * kGroup;
        w.rows = (int)(w.m0 + kGroup);   // the other half's waves idle
      }
      w.kb0 = 0; w.kb1 = KB; w.split = 0; w.tile = u;
    } else {
      // (32-bit quotients on the wave-uniform unit index: the GPU has no
      // integer divider, and this decode sits on the path to a unit's
      // first loads)
      const uint32_t uu = __builtin_amdgcn_readfirstlane(u);
      uint32_t t = uu, sp = 0;
      if (splits > 1) {
        t = uu / (uint32_t)splits;
        sp = uu - t * (uint32_t)splits;
      }
      w.split = (int)sp;
      w.tile = (int)t;
      int mt = (int)(t / (uint32_t)n_tiles), nt = (int)t - mt * n_tiles;
      // (the XCD-blocked raster is compiled into the 256 x 256 tiles only)
      if (C::PIN && splits == 1 && p.raster > 0)
        grouped_tile(xcd_block(t, total, G), (int)((M + C::BM - 1) / C::BM), n_tiles,
                     p.raster, mt, nt);
      w.m0 = (int64_t)mt * C::BM;
      w.n0 = (int64_t)nt * C::BN;
      // KB < 2^17: the C ABI caps K below 2^24
      w.kb0 = splits > 1 ? (int)(sp * (uint32_t)KB / (uint32_t)splits) : 0;
      w.kb1 = splits > 1 ? (int)((sp + 1) * (uint32_t)KB / (uint32_t)splits) : KB;
      w.rows = (int)M;
      w.g = 0;
      if constexpr (MODE == kContiguous) w.g = p.block_expert[w.m0 / kGroup];
    }
    w.g = uniform(w.g);
    w.m0 = uniform(w.m0);
    w.n0 = uniform(w.n0);
    w.kb0 = uniform(w.kb0);
    w.kb1 = uniform(w.kb1);
    w.rows = uniform(w.rows);
    // a 128-row block whose expert id is out of range is skipped (not written)
    if (MODE == kContiguous && (w.g < 0 || w.g >= p.groups)) continue;

    const uint8_t* ga;
    const uint8_t* gb = p.b;
    const float* gsa = nullptr;
    const float* gsb = nullptr;
    const uint8_t* gea = nullptr;
    const uint8_t* geb = nullptr;
    if constexpr (MODE == kMasked) {
      ga = p.a + (int64_t)w.g * M * K;
      gb = p.b + (int64_t)w.g * N * K;
      if constexpr (MX) {
        gea = (const uint8_t*)p.sa + (int64_t)w.g * M * (K / kMxBlock);
        geb = (const uint8_t*)p.sb + (int64_t)w.g * N * (K / kMxBlock);
      } else {
        gsa = (const float*)p.sa + (int64_t)w.g * KB * M;
        gsb = (const float*)p.sb + (int64_t)w.g * nb_blocks * KB;
      }
    } else if constexpr (MODE == kKGrouped) {
      ga = p.a;
      gsa = (const float*)p.sa;
      gsb = (const float*)p.sb;   // [KB][N]: one scale per B row and K block
    } else {
      ga = p.a;
      gb = p.b + (int64_t)w.g * N * K;
      if constexpr (MX) {
        gea = (const uint8_t*)p.sa;
        geb = (const uint8_t*)p.sb + (int64_t)w.g * N * (K / kMxBlock);
      } else {
        gsa = (const float*)p.sa;
        gsb = (const float*)p.sb + (int64_t)w.g * nb_blocks * KB;
      }
    }

    // every wave must be done with the LDS stages of the previous unit
    __syncthreads();

    const int last_row = w.rows - 1;
    const bool wave_live = (w.m0 + wm0) < w.rows;   // masked: rows past the count are skipped

    // Per-lane byte offsets of the LDS-DMA sources, relative to the tile's
    // first row (fixed for the unit).  Rows past the live count (or past N)
    // are clamped to the last live row: they are read but never stored.
    // (tile-relative rows in 32 bits: a tile row times K stays below 2^32,
    // since K < 2^24; the clamps give the same bits as in 64 bits)
    const int a_last = (int)(last_row - w.m0), b_last = (int)(N - 1 - w.n0);
    const uint32_t Ku = (uint32_t)K;
    uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int r = wave * C::A_ROWS + i * 8 + (lane >> 3);
      a_off[i] = (uint32_t)min(r, a_last) * Ku + (((lane & 7) ^ swz(r)) << 4);
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      const int r = wave * C::B_ROWS + i * 8 + (lane >> 3);
      b_off[i] = (uint32_t)min(r, b_last) * Ku + (((lane & 7) ^ swz(r)) << 4);
    }
    uint32_t sa_off, sb_off = 0;
    {
      sa_off = (uint32_t)min(wave * C::A_ROWS + lane, a_last) * (MX ? Ku / kMxBlock : 4u);
      if constexpr (MX) {
        sb_off = (uint32_t)min(wave * C::B_ROWS + lane, b_last) * (Ku / kMxBlock);
      } else if constexpr (MODE == kKGrouped) {
        sb_off = (uint32_t)min(wave * C::B_ROWS + lane, b_last) * 4u;
      }
    }
    // MXG: lane l fetches dword (l & 3) of row (l >> 2) of each 16-row slice
    // of this wave's A and B rows; the K block index is clamped at the end of
    // the row (a partial last group), so every byte read lies in the row.
    uint32_t ga_off[MXG ? C::A_ROWS / 16 : 1], gb_off[MXG ? C::B_ROWS / 16 : 1];
    if constexpr (MXG) {
#pragma unroll
      for (int c = 0; c < C::A_ROWS / 16; ++c) {
        const int64_t r = w.m0 + wave * C::A_ROWS + 16 * c + (lane >> 2);
        ga_off[c] = (uint32_t)(((r < last_row ? r : last_row) - w.m0) * (K / kMxBlock));
      }
#pragma unroll
      for (int c = 0; c < C::B_ROWS / 16; ++c) {
        const int64_t r = w.n0 + wave * C::B_ROWS + 16 * c + (lane >> 2);
        gb_off[c] = (uint32_t)(((r < N - 1 ? r : N - 1) - w.n0) * (K / kMxBlock));
      }
    }
    // the B-block scale row of this wave's columns (FP32 path)
    const int64_t nbw0 = (w.n0 + wn0) / kGroup;
    const int64_t nbw = nbw0 < nb_blocks - 1 ? nbw0 : nb_blocks - 1;
    const float* sb_row = MX || MODE == kKGrouped ? nullptr : gsb + nbw * KB;
    const uint8_t* a_tile = ga + w.m0 * K;
    const uint8_t* b_tile = gb + w.n0 * K;
    // One LDS-DMA instruction of K block kb into block slot `sub` of stage
    // `stage`: r < A_LOADS copies 8 A rows, then B_LOADS copies of 8 B rows,
    // then the A row scales and the B scales (one dword per row, or the
    // wave's one B-block scale).
    constexpr int PB = C::A_LOADS + C::B_LOADS + 2;   // loads per K block and wave
    auto issue_part = [&](int kb, int stage, int sub, int r) {
      const uint32_t st =
          uniform(lds0 + (uint32_t)(stage * C::STAGE_BYTES + sub * C::BLOCK_BYTES));
      const uint32_t sst = st + C::A_BYTES + C::B_BYTES;
      if (r < C::A_LOADS) {
        const uint8_t* ab = uniform(a_tile + (int64_t)kb * kGroup);
        dma16(ab, a_off[r], uniform(st + (uint32_t)((wave * C::A_ROWS + r * 8) * kGroup)));
      } else if (r < C::A_LOADS + C::B_LOADS) {
        const int i = r - C::A_LOADS;
        const uint8_t* bb = uniform(b_tile + (int64_t)kb * kGroup);
        const uint32_t bl = uniform(st + (uint32_t)(C::A_BYTES + (wave * C::B_ROWS + i * 8) * kGroup));
        if constexpr (BS) dma16_nt(bb, b_off[i], bl);
        else dma16(bb, b_off[i], bl);
      } else if (r == C::A_LOADS + C::B_LOADS) {
        if constexpr (MXG) {
          // the group of K blocks kb .. kb + 3, issued with its first block
          if ((kb & 3) != 0) return;
          const uint32_t kd = (uint32_t)min(kb + (lane & 3), KB - 1) * 4;
          const uint8_t* eab = uniform(gea + w.m0 * (K / kMxBlock));
          const uint32_t gl = uniform(mxg0 + (uint32_t)(((kb >> 2) & 1) * GRP_DWORDS * 4));
#pragma unroll
          for (int c = 0; c < C::A_ROWS / 16; ++c)
            dma4(eab, ga_off[c] + kd, uniform(gl + (uint32_t)((wave * C::A_ROWS + 16 * c) * 16)));
        } else if constexpr (MX) {
          // E8M0 bytes of K block kb for each tile row: one dword per row
          const uint8_t* eab = uniform(gea + w.m0 * (K / kMxBlock) + kb * 4);
          const uint32_t la = uniform(sst + (uint32_t)(wave * C::A_ROWS * 4));
          if (lane < C::A_ROWS) dma4(eab, sa_off, la);
        } else {
          const float* sab = uniform(gsa + (int64_t)kb * M + w.m0);
          const uint32_t la = uniform(sst + (uint32_t)(wave * C::A_ROWS * 4));
          if (lane < C::A_ROWS) dma4(sab, sa_off, la);
        }
      } else {
        if constexpr (MXG) {
          if ((kb & 3) != 0) return;
          const uint32_t kd = (uint32_t)min(kb + (lane & 3), KB - 1) * 4;
          const uint8_t* ebb = uniform(geb + w.n0 * (K / kMxBlock));
          const uint32_t gl = uniform(mxg0 + (uint32_t)(((kb >> 2) & 1) * GRP_DWORDS * 4));
#pragma unroll
          for (int c = 0; c < C::B_ROWS / 16; ++c)
            dma4(ebb, gb_off[c] + kd,
                 uniform(gl + (uint32_t)((C::BM + wave * C::B_ROWS + 16 * c) * 16)));
        } else if constexpr (MX) {
          const uint8_t* ebb = uniform(geb + w.n0 * (K / kMxBlock) + kb * 4);
          const uint32_t lb = uniform(sst + (uint32_t)(C::SA_BYTES + wave * C::B_ROWS * 4));
          if (lane < C::B_ROWS) dma4(ebb, sb_off, lb);
        } else if constexpr (MODE == kKGrouped) {
          // the B row scales of K block kb: one FP32 per row
          const float* sbb = uniform(gsb + (int64_t)kb * N + w.n0);
          const uint32_t lb = uniform(sst + (uint32_t)(C::SA_BYTES + wave * C::B_ROWS * 4));
          if (lane < C::B_ROWS) dma4(sbb, sb_off, lb);
        } else if constexpr (C::SPLITB) {
          // the scales of the two B blocks this wave's columns can touch (the
          // second clamped to the last block): lanes 0 and 1
          const float* sbp = uniform(sb_row + kb);
          const uint32_t lw = uniform(sst + (uint32_t)(C::SA_BYTES + C::SB_BYTES + wave * 8));
          if (lane < 2) dma4(sbp, lane == 1 && nbw < nb_blocks - 1 ? (uint32_t)(KB * 4) : 0u, lw);
        } else {
          // this wave's B-block scale for K block kb, one lane
          const float* sbp = uniform(sb_row + kb);
          const uint32_t lw = uniform(sst + (uint32_t)(C::SA_BYTES + C::SB_BYTES + wave * 4));
          if (lane == 0) dma4(sbp, 0u, lw);
        }
      }
    };
    // loads per stage: every stage issues KS K blocks (past the end of the
    // unit the last K block is fetched again and not used), so that the
    // per-stage count is fixed
    constexpr int LOADS = C::KS * PB;

#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // ---- prologue: STAGES-1 K blocks in flight
    const int nkb = w.kb1 - w.kb0;
    // The K blocks of a unit are walked starting at a unit-dependent offset:
    // tiles that run at the same time and share an operand (the A rows of a
    // skinny GEMM, the A tile of a row of output tiles) then read different
    // K blocks of it instead of all hitting the same L2 lines at once.
    // (compiled into the 256 x 256 tiles only: on the decode tiles its
    // remainder and K-block remapping sat on the path to the first loads)
    const int rot = C::PIN && p.rotate && nkb > 0 && !MXG ? uniform(u % nkb) : 0;   // MXG: groups in order
    auto kb_of = [&](int j) {
      const int x = j + rot;
      return w.kb0 + (x >= nkb ? x - nkb : x);
    };
    const int nst = (nkb + C::KS - 1) / C::KS;   // stages of this unit
    auto issue_range = [&](int si, int stage, int p0, int p1) {
#pragma unroll
      for (int q = 0; q < LOADS; ++q)
        if (q >= p0 && q < p1)
          issue_part(kb_of(min(si * C::KS + q / PB, nkb - 1)), stage, q / PB, q % PB);
    };
    // SAB (masked layout, two-stage 256 x 256 tiles, FP32 block scales):
    // the A part of a K block (A rows and their scales) and its B part (B
    // rows and the B-block scale) are issued separately.  A wave reads its
    // A fragments and the scales into registers when it starts a K block,
    // so once every wave is past column tile MID_AT the block's A region is
    // dead: a barrier there lets the A part of the K block two ahead go
    // into it, giving A two blocks of compute to land while only the B part
    // of the next block must land within one.  The masked GEMM streams each
    // expert's B from HBM once and gains (0.119 -> 0.114 ms); on the other
    // layouts the extra barrier cost more than the slack gained.
    constexpr bool SAB = C::PIN && C::STAGES == 2 && C::KS == 1 && !MX && MODE == kMasked;
    constexpr int NA = C::A_LOADS + 1;   // loads of an A part, per wave
    constexpr int MID_AT = 2, B_LATE_AT = 1, A_LATE_AT = 5;
    static_assert(!SAB || (MID_AT < C::TN && A_LATE_AT < C::TN && B_LATE_AT < MID_AT &&
                           MID_AT < A_LATE_AT), "issue points inside the column steps, B before A");
    auto issue_A = [&](int si, int stage) {
      const int kb = kb_of(min(si, nkb - 1));
#pragma unroll
      for (int r = 0; r < C::A_LOADS; ++r) issue_part(kb, stage, 0, r);
      issue_part(kb, stage, 0, C::A_LOADS + C::B_LOADS);
    };
    auto issue_B = [&](int si, int stage) {
      const int kb = kb_of(min(si, nkb - 1));
#pragma unroll
      for (int r = C::A_LOADS; r < C::A_LOADS + C::B_LOADS; ++r) issue_part(kb, stage, 0, r);
      issue_part(kb, stage, 0, C::A_LOADS + C::B_LOADS + 1);
    };
    if constexpr (SAB) {
      if (nst > 0) {
        issue_A(0, 0);
        issue_B(0, 0);
      }
      if (nst > 1) issue_A(1, 1);
    } else {
      for (int s = 0; s < C::STAGES - 1; ++s)
        if (s < nst) issue_range(s, s, 0, LOADS);
    }

    // ---- main loop.  Where the loads of stage si + STAGES - 1 are issued
    // during the compute of stage si: on the three-stage SPREAD tiles, a
    // share after the MFMAs of each column tile, so that a load instruction
    // that waits for room in the memory pipeline holds up the wave while its
    // MFMAs are already running; on the two-stage 256 x 256 tiles, right
    // after the barrier by the first half of the waves and after column tile
    // LATE_AT by the second half (Cfg::LATE), or split into A and B parts
    // (SAB above); elsewhere all at once after the barrier.
    constexpr int POINTS = C::KS * C::TN;
    // (the K-grouped kernel's per-column scales leave fewer registers: with
    // the issue after column tile 2 it spills more and ran 2.6% slower)
    constexpr int LATE_AT = MODE == kKGrouped && C::LATE >= 0 ? 1 : C::LATE;
    static_assert(LATE_AT < POINTS, "the late issue point lies inside the K block's column steps");
    for (int si = 0; si < nst; ++si) {
      if constexpr (SAB) {
        // stage si's A part (issued two blocks ago) and B part are complete;
        // the A part of block si + 1, issued after them, may stay in flight
        if (si + 1 < nst) wait_vmcnt<NA>();
        else wait_vmcnt<0>();
      } else {
        const int later = min(C::STAGES - 2, nst - 1 - si);   // stages issued after this one
        wait_stages_after<LOADS, C::STAGES - 2>(later);
      }
      __syncthreads();
      const int nsi = si + C::STAGES - 1;
      const bool more = nsi < nst;
      const int nstage = nsi % C::STAGES;
      const bool late = LATE_AT >= 0 && p.stagger && wave >= C::WAVES / 2 && wave_live;
      const bool moreA = si + 2 < nst;   // SAB: the A part two blocks ahead
      auto issue_point = [&](int pt) {
        if constexpr (SAB) {
          // B part of block si + 1 (late waves), the barrier after which this
          // block's A region is free, the A part of block si + 2
          if (pt == B_LATE_AT && late && more) issue_B(nsi, nstage);
          if (pt == MID_AT) {
            __syncthreads();
            if (!late && moreA) issue_A(si + 2, si & 1);
          }
          if (pt == A_LATE_AT && late && moreA) issue_A(si + 2, si & 1);
        } else {
          if (C::SPREAD && more)
            issue_range(nsi, nstage, pt * LOADS / POINTS, (pt + 1) * LOADS / POINTS);
          if (pt == LATE_AT && late && more) issue_range(nsi, nstage, 0, LOADS);
        }
      };
      if constexpr (SAB) {
        if (more && !late) issue_B(nsi, nstage);
        if (!wave_live) {   // (every wave meets the middle barrier)
          __syncthreads();
          if (moreA) issue_A(si + 2, si & 1);
          continue;
        }
      } else if (!C::SPREAD || !wave_live) {
        if (more && !late) issue_range(nsi, nstage, 0, LOADS);
        if (!wave_live) continue;
      }
#pragma unroll
      for (int sub = 0; sub < C::KS; ++sub) {
        const bool active = C::KS == 1 || si * C::KS + sub < nkb;
        const uint8_t* st = smem + (si % C::STAGES) * C::STAGE_BYTES + sub * C::BLOCK_BYTES;
        const uint8_t* As = st;
        const uint8_t* Bs = st + C::A_BYTES;
        const uint8_t* Ss = st + C::A_BYTES + C::B_BYTES;
        if (!active) {
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) issue_point(sub * C::TN + tn);
          continue;
        }
        v8i fa[C::TM];
        fa[0] = load_frag(As, wm0, lane);
        const v8i fb0 = load_frag(Bs, wn0, lane);   // the first MFMA needs only these two
#pragma unroll
        for (int tm = 1; tm < C::TM; ++tm) fa[tm] = load_frag(As, wm0 + tm * 16, lane);
        if constexpr (MX) {
          // the dword of K block kb of each row: per-stage, or in its group buffer
          const int kbc = kb_of(si * C::KS + sub);
          const uint32_t* sa_w = MXG ? mx_grp + ((kbc >> 2) & 1) * GRP_DWORDS + (kbc & 3)
                                     : reinterpret_cast<const uint32_t*>(Ss);
          const uint32_t* sb_w = MXG ? sa_w + C::BM * 4
                                     : reinterpret_cast<const uint32_t*>(Ss + C::SA_BYTES);
          constexpr int RS = MXG ? 4 : 1;   // dwords per row
          int sA[C::TM];
#pragma unroll
          for (int tm = 0; tm < C::TM; ++tm)
            sA[tm] = (int)(sa_w[(wm0 + tm * 16 + (lane & 15)) * RS] >> (8 * (lane >> 4)));
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) {
            const v8i fb = tn == 0 ? fb0 : load_frag(Bs, wn0 + tn * 16, lane);
            const int sB = (int)(sb_w[(wn0 + tn * 16 + (lane & 15)) * RS] >> (8 * (lane >> 4)));
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
              acc[tm][tn] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  fa[tm], fb, acc[tm][tn], 0, 0, 0, sA[tm], 0, sB);
            if constexpr (C::PIN) {
#pragma unroll
              for (int tm = 0; tm < C::TM; ++tm) pin_value(acc[tm][tn]);
            }
            issue_point(sub * C::TN + tn);
            if constexpr (C::PIN) pin_step();
          }
        } else {
          // one B scale per wave (128-row blocks of B), or one per B row
          // (K-grouped: 1x128 scales on both operands, applied per column)
          // (a wave straddling two B blocks applies them per column tile)
          constexpr bool PERCOL = MODE == kKGrouped || C::SPLITB;
          const float sbv =
              PERCOL ? 1.f
                     : *reinterpret_cast<const float*>(Ss + C::SA_BYTES + C::SB_BYTES + wave * 4);
          float sbc[C::TN];
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) {
            if constexpr (MODE == kKGrouped) {
              sbc[tn] = reinterpret_cast<const float*>(Ss + C::SA_BYTES)[wn0 + tn * 16 + (lane & 15)];
            } else if constexpr (C::SPLITB) {
              const int blk = (int)(((w.n0 + wn0 + tn * 16) >> 7) - ((w.n0 + wn0) >> 7));
              sbc[tn] = reinterpret_cast<const float*>(Ss + C::SA_BYTES + C::SB_BYTES + wave * 8)[blk];
            } else {
              sbc[tn] = 1.f;
            }
          }
          v4f sc[C::TM];
#pragma unroll
          for (int tm = 0; tm < C::TM; ++tm) {
            const float4 s4 = *reinterpret_cast<const float4*>(
                Ss + (wm0 + tm * 16 + 4 * (lane >> 4)) * 4);
            sc[tm] = v4f{s4.x * sbv, s4.y * sbv, s4.z * sbv, s4.w * sbv};
          }
          // Two-level accumulation, software-pipelined: the MFMAs of column
          // tile tn (one 128-K partial per 16x16 tile) are issued before the
          // promotion FMAs of column tile tn-1, so the FP32 FMAs run while the
          // matrix core works and no MFMA waits on the previous one's result;
          // the B fragment of column tile tn+1 is read from LDS meanwhile.
          v4f part[2][C::TM];
          v8i fb[2];
          const v4f z = {0.f, 0.f, 0.f, 0.f};
          fb[0] = fb0;
#pragma unroll
          for (int tn = 0; tn < C::TN; ++tn) {
            if (tn + 1 < C::TN) fb[(tn + 1) & 1] = load_frag(Bs, wn0 + (tn + 1) * 16, lane);
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
              part[tn & 1][tm] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                  fa[tm], fb[tn & 1], z, 0, 0, 0, 0, 0, 0);
            if (tn > 0) {
#pragma unroll
              for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  const float f = PERCOL ? sc[tm][v] * sbc[tn - 1] : sc[tm][v];
                  acc[tm][tn - 1][v] = fmaf(part[(tn - 1) & 1][tm][v], f, acc[tm][tn - 1][v]);
                }
            }
            if constexpr (C::PIN) {
#pragma unroll
              for (int tm = 0; tm < C::TM; ++tm) {
                pin_value(part[tn & 1][tm]);
                if (tn > 0) pin_value(acc[tm][tn - 1]);
              }
            }
            issue_point(sub * C::TN + tn);
            if constexpr (C::PIN) pin_step();
          }
#pragma unroll
          for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float f = PERCOL ? sc[tm][v] * sbc[C::TN - 1] : sc[tm][v];
              acc[tm][C::TN - 1][v] =
                  fmaf(part[(C::TN - 1) & 1][tm][v], f, acc[tm][C::TN - 1][v]);
            }
        }
      }
    }

    // ---- split-K: deterministic last-arriver reduction through the workspace
    if (C::SPLITK && MODE == kDense && splits > 1) {
      // (an opaque copy of the split count: the per-split tests below are
      // then formed here instead of being hoisted to the kernel's start,
      // where they had cost SGPR spills on the path to the first loads)
      int nsp = splits;
      asm volatile("" : "+s"(nsp));
      constexpr uint32_t kTileBytes = C::BM * C::BN * 4;
      const __amdgpu_buffer_rsrc_t ws =
          buffer_rsrc(p.ws_partial + (int64_t)w.tile * nsp * (C::BM * C::BN), kTileBytes * nsp);
#pragma unroll
      for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < C::TN; ++tn) {
          const uint32_t idx = ((wave * C::TM + tm) * C::TN + tn) * 64 + lane;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[tm][tn]), ws,
                                                 w.split * kTileBytes + idx * 16, 0, kCoherent);
        }
      wait_all_memory();        // this thread's partials have reached the coherence point
      __syncthreads();          // ... and every other thread's
      if (tid == 0)
        flag = __hip_atomic_fetch_add(p.ws_counters + w.tile, 1, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == nsp - 1;
      __syncthreads();
      if (!flag) continue;
      // All partial loads of a batch of output tiles are issued before the
      // first is used, so their latencies overlap; the sum runs in split
      // order (bitwise reproducible).
      constexpr int NT = C::TM * C::TN;
      // (two-waves-per-SIMD tiles have no registers to spare: one tile at a time)
      constexpr int BATCH = C::WAVES == 8 ? 1 : (NT < 4 ? NT : 4);
#pragma unroll
      for (int t0 = 0; t0 < NT; t0 += BATCH) {
        v4f part[BATCH][kMaxSplits];
#pragma unroll
        for (int b = 0; b < BATCH; ++b)
#pragma unroll
          for (int s = 0; s < kMaxSplits; ++s) {
            const int t = t0 + b;
            const uint32_t idx = (wave * NT + t) * 64 + lane;
            if (t < NT && s < nsp && s != w.split)
              part[b][s] = __builtin_bit_cast(
                  v4f, __builtin_amdgcn_raw_buffer_load_b128(ws, s * kTileBytes + idx * 16, 0,
                                                             kCoherent));
          }
#pragma unroll
        for (int b = 0; b < BATCH; ++b) {
          const int t = t0 + b;
          if (t >= NT) break;
          v4f& a = acc[t / C::TN][t % C::TN];
          v4f sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < kMaxSplits; ++s)
            if (s < nsp) sum += s == w.split ? a : part[b][s];
          a = sum;
        }
      }
      if (tid == 0)
        __hip_atomic_store(p.ws_counters + w.tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    __syncthreads();   // every wave is done with the stage buffers

    // ---- fused gated epilogue (contiguous layout, FP32 scales): the tile's
    // first 128 columns are a gate block and the last 128 the matching up
    // block, so its 128 outputs h = silu(gate) * up of each row form exactly
    // one 1x128 group of the next GEMM's input; they are quantized here
    // (amax, s = amax / 448, codes of h / s) and written as FP8 codes plus a
    // K-block-major scale, instead of the BF16 / FP32 product.
    if constexpr (MODE == kContiguous && !MX) {
      if (p.swiglu) {
        constexpr int ROW = C::BN * 4 + 16;
        static_assert(C::BN == 2 * kGroup, "one gate block and one up block per tile");
        // rows staged at a time: whole wave row blocks that fit in the stage memory
        constexpr int FIT = C::STAGES * C::STAGE_BYTES / ROW;
        constexpr int CR = FIT >= C::BM ? C::BM : (FIT / C::WM) * C::WM;
        static_assert(CR >= C::WM && C::BM % CR == 0, "the FP32 tile stages in whole wave blocks");
        const int64_t NH = N / 2;
        const int64_t hb = w.n0 / C::BN;   // 128-column block of h
        uint8_t* qo = p.q_out + w.m0 * NH + hb * kGroup;
        float* so = p.s_out + hb * M + w.m0;
        const int c = (lane & 31) * 4;
        const int64_t live = min((int64_t)C::BM, (int64_t)w.rows - w.m0);   // rows of this unit
#pragma unroll
        for (int r0 = 0; r0 < C::BM; r0 += CR) {
          if (r0 > 0) __syncthreads();   // the previous rows have left LDS
          if (wave_live && wm0 >= r0 && wm0 < r0 + CR) {
#pragma unroll
            for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
              for (int tn = 0; tn < C::TN; ++tn)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  *reinterpret_cast<float*>(smem + (wm0 - r0 + tm * 16 + 4 * (lane >> 4) + v) * ROW +
                                            (wn0 + tn * 16 + (lane & 15)) * 4) = acc[tm][tn][v];
          }
          __syncthreads();
          // two rows per wave step (lanes 0-31 and 32-63), four columns a lane
          for (int r = wave * 2 + (lane >> 5); r < CR && r0 + r < live; r += 2 * C::WAVES) {
            const float4 g = *reinterpret_cast<const float4*>(smem + r * ROW + c * 4);
            const float4 v = *reinterpret_cast<const float4*>(smem + r * ROW + (kGroup + c) * 4);
            const float4 h = make_float4(silu(g.x) * v.x, silu(g.y) * v.y, silu(g.z) * v.z,
                                         silu(g.w) * v.w);
            const float amax = group_max<32>(abs_max4(h));
            // the 1x128 rule of fp8_quantize: s = amax / 448 and codes of
            // h / s, both correctly rounded FP32 divisions
            const float sc = amax == 0.f ? 1.f : amax / kE4m3Max;
            *reinterpret_cast<uint32_t*>(qo + (r0 + r) * NH + c) =
                pack4_e4m3(make_float4(h.x / sc, h.y / sc, h.z / sc, h.w / sc));
            if ((lane & 31) == 0) so[r0 + r] = sc;
          }
        }
        continue;   // the next unit starts with a barrier before reusing LDS
      }
    }

    // ---- epilogue: the tile is staged in LDS in the output type so that the
    // global stores are 16-byte pieces of rows; FP32 or BF16 (RNE); rows past
    // the live count and columns past N are not written.
    auto store_tile = [&](auto esz_c) {
      constexpr int ESZ = decltype(esz_c)::value;
      constexpr int ROW = C::BN * ESZ + 16;   // padded LDS row: conflict-free writes
      constexpr int CHUNKS = C::BN * ESZ / 16, PER = 16 / ESZ;
      // rows staged at a time: whole wave row blocks that fit in the stage memory
      constexpr int FIT = C::STAGES * C::STAGE_BYTES / ROW;
      constexpr int CR = FIT >= C::BM ? C::BM : (FIT / C::WM) * C::WM;
      static_assert(CR >= C::WM && C::BM % CR == 0, "output rows must stage in whole wave blocks");
      // a whole staged block is CR * CHUNKS 16-byte pieces, ITER per thread
      constexpr bool EVEN = C::THREADS % CHUNKS == 0 && (CR * CHUNKS) % C::THREADS == 0;
      constexpr int ITER = EVEN ? CR * CHUNKS / C::THREADS : 1;
      const int64_t d_off = MODE == kMasked || MODE == kKGrouped ? (int64_t)w.g * M * N : 0;
      const bool vec = (N * ESZ) % 16 == 0;   // every row starts 16-byte aligned
      // the unit's tile lies inside the output and its rows fit 32-bit offsets
      const bool full_cols = vec && w.n0 + C::BN <= N && (int64_t)CR * N * ESZ < (1ll << 31);
#pragma unroll
      for (int r0 = 0; r0 < C::BM; r0 += CR) {
        if (r0 > 0) __syncthreads();   // the previous rows have left LDS
        if (wave_live && wm0 >= r0 && wm0 < r0 + CR) {
#pragma unroll
          for (int tm = 0; tm < C::TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < C::TN; ++tn) {
              // lane (i + 16 g) holds rows 4 g .. 4 g + 3 of column i
              if constexpr (ESZ == 2) {
                uint8_t* q = smem + (wm0 - r0 + tm * 16 + 4 * (lane >> 4)) * ROW +
                             (wn0 + tn * 16 + (lane & 15)) * ESZ;
                const uint32_t lo = bf16x2(acc[tm][tn][0], acc[tm][tn][1]);
                const uint32_t hi = bf16x2(acc[tm][tn][2], acc[tm][tn][3]);
                *reinterpret_cast<uint16_t*>(q) = (uint16_t)lo;
                *reinterpret_cast<uint16_t*>(q + ROW) = (uint16_t)(lo >> 16);
                *reinterpret_cast<uint16_t*>(q + 2 * ROW) = (uint16_t)hi;
                *reinterpret_cast<uint16_t*>(q + 3 * ROW) = (uint16_t)(hi >> 16);
              } else {
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  *reinterpret_cast<float*>(smem + (wm0 - r0 + tm * 16 + 4 * (lane >> 4) + v) * ROW +
                                            (wn0 + tn * 16 + (lane & 15)) * ESZ) = acc[tm][tn][v];
              }
            }
        }
        __syncthreads();
        const int64_t live = min((int64_t)CR, (int64_t)w.rows - w.m0 - r0);
        // rows covered by one pass of all threads over the pieces of a row
        constexpr int RSTEP = EVEN ? C::THREADS / CHUNKS : 1;
        if (EVEN && full_cols && live > 0 && live % RSTEP == 0) {
          // whole passes: all LDS reads first, then the stores (buffer
          // stores with 32-bit offsets from the block's first row); the
          // pass guard i * RSTEP < live is uniform
          uint8_t* dbase = reinterpret_cast<uint8_t*>(p.d) + (d_off + (w.m0 + r0) * N + w.n0) * ESZ;
          const __amdgpu_buffer_rsrc_t out = buffer_rsrc(dbase, (uint32_t)((int64_t)CR * N * ESZ));
          // (an opaque copy of tid: the offsets below are computed here, not
          // hoisted into registers held through the main loop)
          int t = tid;
          asm volatile("" : "+v"(t));
          const int ch = t % CHUNKS, rr = t / CHUNKS;
          const uint32_t off0 = (uint32_t)((rr * N + ch * PER) * ESZ);
          const uint32_t rstep_bytes = (uint32_t)(RSTEP * N * ESZ);
          constexpr int BATCH = ITER < 4 ? ITER : 4;   // pieces in registers at a time
#pragma unroll
          for (int i0 = 0; i0 < ITER; i0 += BATCH) {
            v4i piece[BATCH];
#pragma unroll
            for (int i = i0; i < i0 + BATCH; ++i)
              if (i * RSTEP < live)
                piece[i - i0] = *reinterpret_cast<const v4i*>(smem + (rr + i * RSTEP) * ROW + ch * 16);
#pragma unroll
            for (int i = i0; i < i0 + BATCH; ++i)
              if (i * RSTEP < live)
                __builtin_amdgcn_raw_buffer_store_b128(piece[i - i0], out, off0 + i * rstep_bytes,
                                                       0, kStream);
            asm volatile("" ::: "memory");   // keep the next batch's reads after these stores
          }
        } else {
          for (int idx = tid; idx < live * CHUNKS; idx += C::THREADS) {
            const int r = idx / CHUNKS, ch = idx % CHUNKS;
            const int64_t col = w.n0 + ch * PER;
            const uint8_t* src = smem + r * ROW + ch * 16;
            uint8_t* dst =
                reinterpret_cast<uint8_t*>(p.d) + (d_off + (w.m0 + r0 + r) * N + col) * ESZ;
            if (vec && col + PER <= N) {
              *reinterpret_cast<int4*>(dst) = *reinterpret_cast<const int4*>(src);
            } else {
              for (int e = 0; e < PER && col + e < N; ++e) {
                if constexpr (ESZ == 2)
                  reinterpret_cast<uint16_t*>(dst)[e] = reinterpret_cast<const uint16_t*>(src)[e];
                else
                  reinterpret_cast<float*>(dst)[e] = reinterpret_cast<const float*>(src)[e];
              }
            }
          }
        }
      }
    };
    if (p.out_bf16) store_tile(std::integral_constant<int, 2>{});
    else store_tile(std::integral_constant<int, 4>{});
  }
}

// ------------------------------------------------------------------ configs
// Name                     BM   BN  WAVES  STAGES OCC     wave tile
using CfgBig = Cfg<256, 128, 4, 1, 3, 1, 1, true>;    // 64 x 128
using CfgWide = Cfg<128, 256, 2, 2, 3, 1, 1, true>;   // 64 x 128 (contiguous needs BM <= 128)
using CfgS32 = Cfg<64, 32, 2, 2, 8, 1>;      // 32 x 16, deep pipeline
using CfgS32x2 = Cfg<64, 32, 2, 2, 5, 2>;    // 32 x 16, two workgroups per CU
using CfgS64 = Cfg<64, 64, 1, 4, 6, 1>;      // 64 x 16
using CfgS128 = Cfg<64, 128, 1, 4, 5, 1>;    // 64 x 32
using CfgM64 = Cfg<128, 64, 2, 2, 5, 1>;     // 64 x 32
using CfgM32 = Cfg<128, 32, 4, 1, 6, 1>;     // 32 x 32
using CfgBig8 = Cfg<256, 128, 4, 2, 3, 1, 1, true>;   // 64 x 64, two waves per SIMD
using CfgWide8 = Cfg<128, 256, 2, 4, 3, 1, 1, true>;  // 64 x 64, two waves per SIMD
// several K blocks per stage (one barrier per stage): decode-sized M
using CfgS32k4 = Cfg<64, 32, 2, 2, 3, 1, 4>;   // 32 x 16
using CfgS32k2 = Cfg<64, 32, 2, 2, 5, 1, 2>;   // 32 x 16
using CfgS64k4 = Cfg<64, 64, 1, 4, 2, 1, 4>;   // 64 x 16
using CfgS64k2 = Cfg<64, 64, 1, 4, 4, 1, 2>;   // 64 x 16
using CfgS128k2 = Cfg<64, 128, 1, 4, 3, 1, 2>; // 64 x 32
using CfgM32k2 = Cfg<128, 32, 4, 1, 3, 1, 2>;  // 32 x 32
using CfgS32x2k2 = Cfg<64, 32, 2, 2, 3, 2, 2>; // 32 x 16, two workgroups per CU
using CfgHuge8 = Cfg<256, 256, 4, 2, 2, 1, 1>;  // 64 x 128, two waves per SIMD, loads at once
using CfgS96 = Cfg<64, 96, 2, 2, 4, 1, 1>;     // 32 x 48, B-block scales per column tile

struct CfgInfo {
  int bm, bn, occ;
  bool splitk;
};
#define FG8_CFG_INFO(C) {C::BM, C::BN, C::OCC, C::SPLITK}
static const CfgInfo kCfgs[] = {
    FG8_CFG_INFO(CfgBig),  FG8_CFG_INFO(CfgWide), FG8_CFG_INFO(CfgS32),  FG8_CFG_INFO(CfgS32x2),
    FG8_CFG_INFO(CfgS64),  FG8_CFG_INFO(CfgS128), FG8_CFG_INFO(CfgM64),  FG8_CFG_INFO(CfgM32),
    FG8_CFG_INFO(CfgBig8), FG8_CFG_INFO(CfgWide8), FG8_CFG_INFO(CfgS32k4), FG8_CFG_INFO(CfgS32k2),
    FG8_CFG_INFO(CfgS64k4), FG8_CFG_INFO(CfgS64k2), FG8_CFG_INFO(CfgS128k2), FG8_CFG_INFO(CfgM32k2),
    FG8_CFG_INFO(CfgS32x2k2), FG8_CFG_INFO(CfgHuge8), FG8_CFG_INFO(CfgS96),
};
#undef FG8_CFG_INFO
enum CfgId {
  kCfgBig = 0, kCfgWide, kCfgS32, kCfgS32x2, kCfgS64, kCfgS128, kCfgM64, kCfgM32, kCfgBig8,
  kCfgWide8, kCfgS32k4, kCfgS32k2, kCfgS64k4, kCfgS64k2, kCfgS128k2, kCfgM32k2, kCfgS32x2k2,
  kCfgHuge8, kCfgS96, kNumCfgs
};

int device_cu_count() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

// Split count for a dense problem: enough (tile, split) units to give every
// workgroup slot one, keeping at least two K blocks per split.
static int dense_splits(int64_t tiles, int64_t kb, int slots) {
  if (tiles * 2 > slots || tiles > kSplitKMaxTiles) return 1;
  int64_t s = slots / tiles;
  if (s > kb / 2) s = kb / 2;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  return (int)s;
}

// FG8_TILE_OVERRIDE="cfg[,splits]" forces a compiled tile configuration (and
// split count): a tuning hook, not needed for correctness.  Grouped layouts
// accept only the configurations compiled for them.
static bool tile_override(int* cfg, int* splits) {
  const char* e = getenv("FG8_TILE_OVERRIDE");
  if (!e || !*e) return false;
  int c = -1, s = 0;
  if (sscanf(e, "%d,%d", &c, &s) < 1 || c < 0 || c >= kNumCfgs) return false;
  *cfg = c;
  *splits = s;
  return true;
}

TileChoice choose_tiles(const GemmProblem& p, int num_cus) {
  TileChoice t{};
  int forced_splits = 0;
  bool forced = false;
  int ov = -1;
  if (p.mode != kDense && tile_override(&ov, &forced_splits)) {
    if (p.mode == kContiguous && (ov == kCfgWide || ov == kCfgWide8 || ov == kCfgHuge8)) forced = true;
    if (p.mode == kMasked && (ov == kCfgBig || ov == kCfgBig8 || ov == kCfgHuge8)) forced = true;
    if (p.mode == kKGrouped && (ov == kCfgBig8 || ov == kCfgHuge8)) forced = true;
  }
  if (forced) {
    t.cfg = ov;
  } else if (p.mode == kContiguous) {
    // 256 x 256 tiles over pairs of 128-row blocks once they fill the chip:
    // a third fewer operand bytes per FLOP than 128 x 256
    t.cfg = ((p.M + 255) / 256) * ((p.N + 255) / 256) >= (int64_t)num_cus ? kCfgHuge8 : kCfgWide8;
  } else if (p.mode == kKGrouped || p.mode == kMasked) {
    // (masked: the tile count is an upper bound, every expert at capacity)
    t.cfg = (int64_t)p.groups * ((p.M + 255) / 256) * ((p.N + 255) / 256) >= (int64_t)num_cus
                ? kCfgHuge8
                : kCfgBig8;
  } else if (p.mode == kDense && (forced = tile_override(&t.cfg, &forced_splits))) {
  } else if (p.mode == kDense && p.M <= 64) {
    // decode-sized M: narrow 64 x 32 tiles, two workgroups per CU (the
    // LDS-DMA rate of a CU grows with the waves issuing), two K blocks per
    // stage, split along K; when N alone gives two waves of them, wider
    // tiles without a split: 64 x 96 when those fit in one round and the
    // 64 x 128 ones would leave CUs idle (64 x 24576 x 1536: 13.7 against
    // 14.9 us), else 64 x 128
    if ((p.N + 31) / 32 < 2 * num_cus)
      t.cfg = kCfgS32x2k2;
    else if ((p.N + 95) / 96 <= num_cus && (p.N + 127) / 128 < num_cus)
      t.cfg = kCfgS96;
    else
      t.cfg = kCfgS128;
  } else if (p.mode == kDense && p.M <= 128) {
    t.cfg = kCfgS64k2;
  } else if (p.mode == kDense && (((p.M + 255) / 256) * ((p.N + 255) / 256) >= (int64_t)num_cus ||
                                  ((p.M + 255) / 256) * ((p.N + 127) / 128) > (int64_t)num_cus)) {
    // enough 256 x 256 tiles for every CU: the fewest operand bytes per FLOP.
    // Also when fewer, if the 256 x 128 tiles would need a second round: the
    // one round of 256 x 256 tiles then does the same work per CU at a
    // better rate (4096 x 2112 x 7168: 105 against 125 us)
    t.cfg = kCfgHuge8;
  } else if (p.mode == kDense &&
             ((p.M + 255) / 256) * ((p.N + 127) / 128) * 3 < (int64_t)num_cus) {
    // few 256 x 128 tiles (fewer than a third of the CUs): 128 x 64 tiles
    // keep four times as many CUs busy (measured 1.5-2.6x faster on such
    // shapes; at a third or more the large tiles win)
    t.cfg = kCfgM64;
  } else {
    t.cfg = kCfgBig8;
  }
  t.bm = kCfgs[t.cfg].bm;
  t.bn = kCfgs[t.cfg].bn;
  const int slots = num_cus * kCfgs[t.cfg].occ;
  const int64_t n_tiles = (p.N + t.bn - 1) / t.bn;
  const int64_t KB = p.K / kGroup;
  int64_t units;
  t.splits = 1;
  if (p.mode == kMasked || p.mode == kKGrouped) {
    units = (int64_t)p.groups * ((p.M + t.bm - 1) / t.bm) * n_tiles;   // masked: upper bound
  } else {
    const int64_t tiles = ((p.M + t.bm - 1) / t.bm) * n_tiles;
    if (p.mode == kDense && kCfgs[t.cfg].splitk) {
      t.splits = dense_splits(tiles, KB, slots);
      if (forced && forced_splits > 0 && tiles <= kSplitKMaxTiles)
        t.splits = (int)(forced_splits < KB ? forced_splits : KB);
      if (t.splits > kMaxSplits) t.splits = kMaxSplits;
    }
    units = tiles * t.splits;
    if (p.mode == kContiguous && t.bm == 2 * kGroup) units *= 2;   // pair units, then half units
  }
  t.grid = (int)(units < slots ? units : slots);
  if (t.grid < 1) t.grid = 1;
  // K rotation: off.  Measured on the dense and grouped workloads, tiles that
  // walk K in step are faster: the tiles of one XCD then share the same K
  // block of their common A or B rows, which the L2 serves once.
  t.rotate = 0;
  if (const char* e = getenv("FG8_ROTATE")) t.rotate = atoi(e) != 0;
  // Staggered load issue on the two-stage 256 x 256 tiles: on (W1 of the
  // MoE workload 2.00 -> 1.80 ms, W2 -5%, 4096 x 7168 x 2048 -4%).
  t.stagger = 1;
  if (const char* e = getenv("FG8_STAGGER")) t.stagger = atoi(e) != 0;
  // XCD-blocked tile order, four tile rows per group, for the 256 x 256
  // tiles (measured neutral to 4.5% faster on the dense and contiguous
  // workloads; on the masked one it keeps each XCD on one or two experts at
  // a time, so their A rows stay in its L2: 16% faster with MXFP8); the
  // other configurations keep the plain order.
  t.raster = t.cfg == kCfgHuge8 ? 4 : 0;
  if (const char* e = getenv("FG8_RASTER")) t.raster = atoi(e) > 0 ? atoi(e) : 0;
  return t;
}

size_t splitk_workspace_bytes(int64_t m, int64_t n, int64_t k, int num_cus) {
  GemmProblem p{};
  p.mode = kDense; p.M = m; p.N = n; p.K = k; p.groups = 1;
  const TileChoice t = choose_tiles(p, num_cus);
  if (t.splits <= 1) return 0;
  const int64_t tiles = ((m + t.bm - 1) / t.bm) * ((n + t.bn - 1) / t.bn);
  return kSplitKCounterBytes + (size_t)tiles * t.splits * t.bm * t.bn * sizeof(float);
}

// B copies with the non-temporal hint where no other unit of the launch reads
// the same B rows, or where two tile rows at most do: the dense 64-row tiles,
// which the tile choice takes for M <= 128 only (the tuning override can
// force them on larger M, where the hint stays correct but may cost time),
// and masked experts of one tile row.  Against ordinary copies,
// 64 x 24576 x 1536 12.4-12.8 -> 11.4-11.6 us, 64 x 2112 x 7168 10.8 ->
// 10.6 us, 128 x 7168 x 2048 10.7 -> 10.0 us, the masked MXFP8 GEMM with
// 256-row experts 124 -> 111 us.  Where several tile rows share B
// (4096 x 7168 x 2048, the contiguous layout) the hint cost 5-7%.
template <class C, bool MX, int MODE, bool BS = MODE == kDense && C::BM == 64>
static hipError_t launch(GemmProblem p, int grid, hipStream_t s) {
  p.grid = grid;
  hipLaunchKernelGGL((gemm_kernel<C, MX, MODE, BS>), dim3(grid), dim3(C::THREADS), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gemm(GemmProblem p, const TileChoice& t, hipStream_t s) {
  p.splits = t.splits;
  p.rotate = t.rotate;
  p.stagger = t.stagger;
  p.raster = t.raster;
  switch (p.mode) {
    case kDense:
      switch (t.cfg) {
        case kCfgWide: return launch<CfgWide, false, kDense>(p, t.grid, s);
        case kCfgS32: return launch<CfgS32, false, kDense>(p, t.grid, s);
        case kCfgS32x2: return launch<CfgS32x2, false, kDense>(p, t.grid, s);
        case kCfgS64: return launch<CfgS64, false, kDense>(p, t.grid, s);
        case kCfgS128: return launch<CfgS128, false, kDense>(p, t.grid, s);
        case kCfgM64: return launch<CfgM64, false, kDense>(p, t.grid, s);
        case kCfgM32: return launch<CfgM32, false, kDense>(p, t.grid, s);
        case kCfgBig8: return launch<CfgBig8, false, kDense>(p, t.grid, s);
        case kCfgWide8: return launch<CfgWide8, false, kDense>(p, t.grid, s);
        case kCfgS32k4: return launch<CfgS32k4, false, kDense>(p, t.grid, s);
        case kCfgS32k2: return launch<CfgS32k2, false, kDense>(p, t.grid, s);
        case kCfgS64k4: return launch<CfgS64k4, false, kDense>(p, t.grid, s);
        case kCfgS64k2: return launch<CfgS64k2, false, kDense>(p, t.grid, s);
        case kCfgS128k2: return launch<CfgS128k2, false, kDense>(p, t.grid, s);
        case kCfgM32k2: return launch<CfgM32k2, false, kDense>(p, t.grid, s);
        case kCfgS32x2k2: return launch<CfgS32x2k2, false, kDense>(p, t.grid, s);
        case kCfgHuge8: return launch<CfgHuge8, false, kDense>(p, t.grid, s);
        case kCfgS96: return launch<CfgS96, false, kDense>(p, t.grid, s);
        default: return launch<CfgBig, false, kDense>(p, t.grid, s);
      }
    case kContiguous:
      if (t.cfg == kCfgHuge8) {
        if (p.mx) return launch<CfgHuge8, true, kContiguous>(p, t.grid, s);
        return launch<CfgHuge8, false, kContiguous>(p, t.grid, s);
      }
      if (p.mx) return launch<CfgWide8, true, kContiguous>(p, t.grid, s);
      if (t.cfg == kCfgWide8) return launch<CfgWide8, false, kContiguous>(p, t.grid, s);
      return launch<CfgWide, false, kContiguous>(p, t.grid, s);
    case kKGrouped:
      if (t.cfg == kCfgHuge8) return launch<CfgHuge8, false, kKGrouped>(p, t.grid, s);
      return launch<CfgBig8, false, kKGrouped>(p, t.grid, s);
    default:
      // (masked: one tile row per expert when the capacity fits the 256-row tile)
      if (t.cfg == kCfgHuge8 && p.M <= CfgHuge8::BM) {
        if (p.mx) return launch<CfgHuge8, true, kMasked, true>(p, t.grid, s);
        return launch<CfgHuge8, false, kMasked, true>(p, t.grid, s);
      }
      if (t.cfg == kCfgHuge8) {
        if (p.mx) return launch<CfgHuge8, true, kMasked>(p, t.grid, s);
        return launch<CfgHuge8, false, kMasked>(p, t.grid, s);
      }
      if (t.cfg == kCfgBig8 && p.M <= CfgBig8::BM) {
        if (p.mx) return launch<CfgBig8, true, kMasked, true>(p, t.grid, s);
        return launch<CfgBig8, false, kMasked, true>(p, t.grid, s);
      }
      if (t.cfg == kCfgBig8) {
        if (p.mx) return launch<CfgBig8, true, kMasked>(p, t.grid, s);
        return launch<CfgBig8, false, kMasked>(p, t.grid, s);
      }
      if (p.mx) return launch<CfgBig, true, kMasked>(p, t.grid, s);
      return launch<CfgBig, false, kMasked>(p, t.grid, s);
  }
}

}  // namespace fg8
