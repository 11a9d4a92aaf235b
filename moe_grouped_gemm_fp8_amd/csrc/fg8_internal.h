// Internal interface between the C ABI (api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fg8 {

// kKGrouped: per group g, the K range k_offsets[g] .. k_offsets[g+1] of
// shared A [M][K] and B [N][K], both with 1x128 scales ([K/128][M] and
// [K/128][N]); D [G][M][N].
enum GemmMode : int { kDense = 0, kContiguous = 1, kMasked = 2, kKGrouped = 3 };

// One GEMM problem as the kernels see it.  Per group g (expert or batch
// entry): A rows [M][K], B [N][K], D [M][N].  Scales are FP32 (block-scaled
// path) or E8M0 bytes (MX path); their strides follow fg8.h.
struct GemmProblem {
  const uint8_t* a;
  const void* sa;
  const uint8_t* b;
  const void* sb;
  void* d;
  int out_bf16;
  int mx;                       // 1: E8M0 scales through the scaled MFMA
  int mode;                     // GemmMode
  int64_t M, N, K;              // M = rows per group (dense m, contiguous m_total, masked cap)
  int groups;                   // experts (masked / contiguous) or 1
  const int32_t* block_expert;  // contiguous: expert of each 128-row block
  const int32_t* valid;         // masked: live rows per group (NULL = all M)
  const int32_t* k_offsets;     // K-grouped: K offset of each group [groups + 1]
  int rotate;                   // 1: start each unit's K walk at a unit-dependent block
  int stagger;                  // 1: half the waves issue the next stage's loads late (Cfg::LATE)
  int raster;                   // > 0: XCD-blocked grouped raster of the tiles, this many tile rows per group
  // contiguous only: 1 = fused SiLU-gated epilogue that writes the 1x128
  // quantization of h = silu(gate) * up (W1 rows interleaved in 128-row
  // gate/up blocks) to q_out [M][N/2] and s_out [N/256][M] instead of d
  int swiglu;
  uint8_t* q_out;
  float* s_out;
  // split-K (dense only)
  int splits;
  int grid;                     // workgroups of the launch (set by the launcher)
  float* ws_partial;
  int32_t* ws_counters;
};

// Split-K workspace layout: a fixed header of per-tile arrival counters
// (split-K is only used when there are at most kSplitKMaxTiles tiles), then
// the FP32 partial tiles.  Because the header never moves, a workspace can be
// reused across shapes: every completed call leaves all counters at zero and
// partial sums never land on them.
constexpr int kSplitKMaxTiles = 1024;
constexpr int kMaxSplits = 8;   // K splits per tile
constexpr size_t kSplitKCounterBytes = kSplitKMaxTiles * sizeof(int32_t);

struct TileChoice {
  int cfg;      // index into the compiled tile configurations
  int bm, bn;
  int splits;
  int grid;
  int rotate;
  int stagger;
  int raster;
};

TileChoice choose_tiles(const GemmProblem& p, int num_cus);
size_t splitk_workspace_bytes(int64_t m, int64_t n, int64_t k, int num_cus);
hipError_t launch_gemm(GemmProblem p, const TileChoice& t, hipStream_t stream);

hipError_t launch_quantize(const void* x, bool bf16, int64_t batch, int64_t rows, int64_t cols,
                           int kind, uint8_t* q, void* scales, hipStream_t stream);
// Top-k routing ids -> contiguous layout (counts, offsets, block_expert,
// row_token, token_row) followed by the 1x128 quantize of every token row
// into the rows it owns.
hipError_t launch_route_quantize(const void* x, bool bf16, int64_t tokens, int64_t hidden,
                                 const int32_t* ids, int topk, int num_experts, int64_t m_cap,
                                 uint8_t* q, float* sa, int32_t* block_expert, int32_t* row_token,
                                 int32_t* token_row, int32_t* counts, int32_t* offsets,
                                 hipStream_t stream);

int device_cu_count();

}  // namespace fg8
