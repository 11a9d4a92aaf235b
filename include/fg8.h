/*
 * fg8.h - fine-grained-scaled FP8 GEMM on AMD MI355X (gfx950): the C ABI of
 * libfg8.so.
 *
 * The method (DeepSeek's DeepGEMM as described by the pages this library is
 * built from): FP32 tensors are multiplied by per-group scaling factors and
 * converted to FP8, the GEMM runs on FP8 inputs, and the result is restored to
 * FP32 (cuda-deepseek blog, hrletsgo.me, list item 5 of the custom
 * mixed-precision loop); the FP8 partial sums of the matrix units are promoted
 * at a fixed interval into FP32 accumulators where the scales are applied
 * (DeepGEMM release news, ctol-kr.com, section 1 "FP8": two-level
 * accumulation); besides the dense GEMM there are MoE grouped GEMMs in a
 * contiguous and a masked layout (same article, section 4 "MoE"; DeepGEMM
 * explainer, opsoai.com, MoE section); MXFP8 shares one power-of-two exponent
 * per 32 elements (aitrends.kr article on DeepSeek-V3 MoE training on B200,
 * MXFP8 section and glossary).
 *
 * Formats fixed here (the pages name only "FP8"):
 *   e4m3     OCP FP8 E4M3, no infinities, NaN = 0x7F/0xFF, max 448; stored as
 *            uint8.  Encoding rounds to nearest even, saturates at +-448 and
 *            keeps the sign of zero.
 *   1x128    one FP32 scale per row per 128 consecutive K elements,
 *            s = fl32(amax / 448) (s = 1 for an all-zero group),
 *            q = e4m3(fl32(x / s)).
 *   128x128  one FP32 scale per 128x128 block, same rule; a block cut by the
 *            end of the rows takes its amax over the rows that exist.
 *   MX 1x32  one E8M0 byte per row per 32 consecutive K elements:
 *            E = clamp(floor(log2 amax) - 8, -127, 127), byte = E + 127
 *            (0 for an all-zero block), q = e4m3(x * 2^-E), value 2^(byte-127).
 * A dequantized element is e4m3(q) * scale.  Every GEMM computes
 *   D[m][n] = sum_k A[m][k] * B[n][k]
 * with A [rows][K] and B [N][K] both K-contiguous (B is a Linear weight
 * [out][in]), accumulating in FP32 and storing FP32 or BF16 (round to
 * nearest even).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE memory owned by the caller and must be 16-byte
 *     aligned.  The library allocates nothing, keeps no state between calls,
 *     never synchronizes and never exits the process; work is queued on
 *     `stream` (NULL = the default stream) and the call returns at once.
 *   - Returns FG8_OK, or FG8_EINVAL (NULL or misaligned pointer, a size out
 *     of range), FG8_EUNSUPPORTED (a shape this library does not handle), or
 *     FG8_EHIP (the kernel launch failed).  On FG8_EINVAL and
 *     FG8_EUNSUPPORTED nothing was launched.  fg8_last_error() gives the text
 *     for the calling thread's last failure.  Faults inside a kernel surface
 *     at the caller's next synchronization.
 *   - Device-side index data is range-checked by the kernels: a 128-row
 *     block whose block_expert value lies outside [0, E) is skipped (its
 *     output rows are left as they were), and valid_rows values are clamped
 *     to [0, cap] (gemm_mxfp8: [0, m]).
 *   - Calls may run concurrently on different streams; a split-K workspace
 *     must not be shared by calls that can overlap.
 *   - Every GEMM takes 128 <= k <= 2^24 - 128 with k % 128 == 0 (else
 *     FG8_EUNSUPPORTED): the copies into LDS address a tile of up to 256
 *     rows with 32-bit offsets.
 *   - FP32 inputs to fp8_quantize must be finite.
 */
#ifndef FG8_H
#define FG8_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FG8_OK = 0,
  FG8_EINVAL = 1,
  FG8_EUNSUPPORTED = 2,
  FG8_EHIP = 3
} fg8_status;

typedef enum { FG8_OUT_F32 = 0, FG8_OUT_BF16 = 1 } fg8_out;

typedef enum {
  FG8_SCALE_1x128 = 0,
  FG8_SCALE_128x128 = 1,
  FG8_SCALE_MX1x32 = 2,
  FG8_SCALE_1x128_T = 3
} fg8_scale_kind;

/*
 * fp8_quantize: FP32 -> e4m3 with fine-grained scales (the "multiply by a
 * scaling factor and convert to FP8" step of the cuda-deepseek blog's
 * mixed-precision loop, list item 5, at per-group granularity; MX variant per
 * the aitrends.kr MXFP8 glossary entry).
 *   x       const float [batch][rows][cols], row-major.
 *   q       uint8 [batch][rows][cols] e4m3 codes (output); for
 *           FG8_SCALE_1x128_T the transpose, [batch][cols][rows].
 *   scales  output, layout by kind:
 *             FG8_SCALE_1x128   float   [batch][cols/128][rows]  (K-block major)
 *             FG8_SCALE_128x128 float   [batch][ceil(rows/128)][cols/128]
 *             FG8_SCALE_MX1x32  uint8_t [batch][rows][cols/32]   (E8M0 bytes)
 *             FG8_SCALE_1x128_T float   [batch][rows/128][cols]
 *   FG8_SCALE_1x128_T groups 128 consecutive ROWS of each column: the 1x128
 *   quantization of x^T, written as x^T (the token-axis layout the weight
 *   gradient multiplies, see grouped_gemm_fp8_kgrouped).
 *   batch >= 1, rows >= 1; cols % 128 == 0 (cols % 32 == 0 for MX; for
 *   FG8_SCALE_1x128_T rows % 128 == 0 and cols % 64 == 0), else
 *   FG8_EUNSUPPORTED.  Results are bit-exact with the formats above.
 */
fg8_status fp8_quantize(const float* x, int64_t batch, int64_t rows, int64_t cols,
                        fg8_scale_kind kind, uint8_t* q, void* scales, hipStream_t stream);

/*
 * fp8_quantize_bf16: fp8_quantize for a BF16 source, the BF16 -> MXFP8 step
 * of the MoE training pipeline (aitrends.kr B200 article, MXFP8 section) and
 * its 1x128 / 128x128 counterparts.  BF16 widens exactly to FP32, so the
 * result is bit-identical to fp8_quantize of the widened tensor.
 *   x  const uint16_t [batch][rows][cols] bfloat16 bit patterns, row-major;
 *   every other argument, layout and error as fp8_quantize.
 */
fg8_status fp8_quantize_bf16(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                             fg8_scale_kind kind, uint8_t* q, void* scales, hipStream_t stream);

/*
 * gemm_fp8_blockscaled: dense D = A B^T with 1x128 scales on A and 128x128
 * scales on B, two-level accumulation (DeepGEMM release news, ctol-kr.com,
 * section 1; shapes of the DeepGEMM explainer's speed-up table, opsoai.com).
 *   a  uint8 [m][k]               sa float [k/128][m]
 *   b  uint8 [n][k]               sb float [ceil(n/128)][k/128]
 *   d  [m][n] float (FG8_OUT_F32) or bfloat16 bits (FG8_OUT_BF16), row-major.
 *   m, n >= 1; k % 128 == 0 and k >= 128 (else FG8_EUNSUPPORTED).
 *   workspace: device memory of at least fg8_gemm_workspace_bytes(m, n, k)
 *   bytes (NULL allowed when that is 0).  Its first 4096 bytes are per-tile
 *   arrival counters, the rest FP32 split-K partial sums.  It must be
 *   zero-filled before its first use; every completed call leaves the
 *   counters at zero again, so one workspace serves any sequence of shapes
 *   (of calls that do not overlap).  Too small a workspace is FG8_EINVAL.
 */
fg8_status gemm_fp8_blockscaled(const uint8_t* a, const float* sa, const uint8_t* b,
                                const float* sb, void* d, fg8_out out, int64_t m, int64_t n,
                                int64_t k, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Workspace bytes gemm_fp8_blockscaled needs for this shape (0 if none). */
size_t fg8_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Bytes of the per-GPU scratch array of gemm_fp8_blockscaled_noalloc. */
#define FG8_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * gemm_fp8_blockscaled_noalloc: gemm_fp8_blockscaled without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, layouts, kernels and results as gemm_fp8_blockscaled.
 *   The split-K counters and partial sums live in a static device array of
 *   FG8_NOALLOC_SCRATCH_BYTES (16 MiB), one per GPU the library runs on,
 *   held until the process ends; its address is looked up at the first call
 *   on each device, which also clears its counters on `stream`.  A shape
 *   whose fg8_gemm_workspace_bytes exceeds that size is FG8_EUNSUPPORTED
 *   (nothing launched).  The call allocates nothing.
 *   Every call on one GPU shares that GPU's array: calls that can overlap on
 *   one GPU (other streams, other threads) race and must not be issued;
 *   calls queued on one stream are fine, since each completed call leaves
 *   the counters at zero again.
 */
fg8_status gemm_fp8_blockscaled_noalloc(const uint8_t* a, const float* sa, const uint8_t* b,
                                        const float* sb, void* d, fg8_out out, int64_t m,
                                        int64_t n, int64_t k, hipStream_t stream);

/*
 * grouped_gemm_fp8_contiguous: MoE grouped GEMM, contiguous layout (DeepGEMM
 * release news, ctol-kr.com, section 4; DeepGEMM explainer, MoE section).  The
 * rows routed to each expert are stacked, each expert's run padded to a
 * multiple of 128 rows; block_expert names the expert of every 128-row block.
 *   a  uint8 [m_total][k]         sa float [k/128][m_total]
 *   b  uint8 [E][n][k]            sb float [E][ceil(n/128)][k/128]
 *   block_expert int32 [m_total/128], values in [0, E); others skip the block
 *                (device memory)
 *   d  [m_total][n] float or bfloat16 bits.  Every row is written, padding
 *   rows included (they are zero when the padding rows of a are zero).
 *   m_total % 128 == 0, k % 128 == 0 (else FG8_EUNSUPPORTED); E = num_experts >= 1.
 */
fg8_status grouped_gemm_fp8_contiguous(const uint8_t* a, const float* sa, const uint8_t* b,
                                       const float* sb, const int32_t* block_expert, void* d,
                                       fg8_out out, int64_t m_total, int64_t n, int64_t k,
                                       int32_t num_experts, hipStream_t stream);

/*
 * grouped_gemm_fp8_masked: MoE grouped GEMM, masked layout (DeepGEMM release
 * news, ctol-kr.com, section 4: expert activation may be sparse).  Each expert
 * owns a fixed block of cap rows of which only the first valid_rows[e] are
 * live; the counts stay in device memory (no host synchronization, so the
 * call can be captured in a graph).
 *   a  uint8 [E][cap][k]          sa float [E][k/128][cap]
 *   b  uint8 [E][n][k]            sb float [E][ceil(n/128)][k/128]
 *   valid_rows int32 [E], values in [0, cap]  (device memory)
 *   d  [E][cap][n]: rows r < valid_rows[e] are written; rows at or past the
 *   count are never written (and rows of a and sa there are never read).
 *   cap >= 1, k % 128 == 0 (else FG8_EUNSUPPORTED); E = num_experts >= 1.
 */
fg8_status grouped_gemm_fp8_masked(const uint8_t* a, const float* sa, const uint8_t* b,
                                   const float* sb, const int32_t* valid_rows, void* d,
                                   fg8_out out, int32_t num_experts, int64_t cap, int64_t n,
                                   int64_t k, hipStream_t stream);

/*
 * gemm_mxfp8: MXFP8 grouped GEMM (aitrends.kr article, MXFP8 section: MXFP8
 * grouped GEMM for the MoE experts; glossary: one shared exponent per 32
 * elements).  The E8M0 scales are applied by the gfx950 scaled MFMA, so there
 * is no separate promotion step.
 *   a  uint8 [G][m][k]            sa_e8m0 uint8 [G][m][k/32]
 *   b  uint8 [G][n][k]            sb_e8m0 uint8 [G][n][k/32]
 *   valid_rows NULL (every row of every group) or int32 [G] in [0, m]
 *   (device memory; masked layout as in grouped_gemm_fp8_masked)
 *   d  [G][m][n] float or bfloat16 bits.
 *   k % 128 == 0 (else FG8_EUNSUPPORTED); G = num_groups >= 1, m, n >= 1.
 *   E8M0 byte 0xFF (NaN) is not a valid input.
 */
fg8_status gemm_mxfp8(const uint8_t* a, const uint8_t* sa_e8m0, const uint8_t* b,
                      const uint8_t* sb_e8m0, const int32_t* valid_rows, void* d, fg8_out out,
                      int32_t num_groups, int64_t m_per_group, int64_t n, int64_t k,
                      hipStream_t stream);

/*
 * grouped_gemm_mxfp8_contiguous: MoE grouped GEMM in the contiguous layout
 * with MXFP8 operands (aitrends.kr B200 article, MXFP8 section: MXFP8 grouped
 * GEMM for the experts of a DeepSeek-V3 MoE layer; the contiguous layout of
 * the DeepGEMM release news, ctol-kr.com, section 4).  One E8M0 exponent per
 * 32 consecutive K elements of every row of a and b, applied by the scaled
 * MFMA.
 *   a  uint8 [m_total][k]         sa_e8m0 uint8 [m_total][k/32]
 *   b  uint8 [E][n][k]            sb_e8m0 uint8 [E][n][k/32]
 *   block_expert, d, the skipping of out-of-range expert ids, sizes and errors
 *   as grouped_gemm_fp8_contiguous; k % 128 == 0 (else FG8_EUNSUPPORTED).
 *   E8M0 byte 0xFF (NaN) is not a valid input.
 */
fg8_status grouped_gemm_mxfp8_contiguous(const uint8_t* a, const uint8_t* sa_e8m0,
                                         const uint8_t* b, const uint8_t* sb_e8m0,
                                         const int32_t* block_expert, void* d, fg8_out out,
                                         int64_t m_total, int64_t n, int64_t k,
                                         int32_t num_experts, hipStream_t stream);

/*
 * grouped_gemm_fp8_contiguous_swiglu: the contiguous grouped GEMM of the
 * first expert weight W1 with its activation and the quantization of the
 * second GEMM's input fused into the epilogue, so the W1 product never
 * reaches memory.  The pages give the expert layer as quantize -> grouped
 * GEMM -> restore (aitrends.kr B200 article, MXFP8 pipeline diagram) with a
 * W1 twice as wide as W2's input; the activation between the two GEMMs is
 * not named there, and this library reads it as a SiLU-gated unit:
 *   h[m][128 j + c] = silu(G[m][256 j + c]) * G[m][256 j + 128 + c],
 *   silu(x) = x / (1 + e^-x),   G = the contiguous product A W1^T in FP32,
 * i.e. the rows of W1 (and of its 128x128 scales) interleave in 128-row
 * blocks: gate block j at rows 256 j .. 256 j + 127, up block j at rows
 * 256 j + 128 .. 256 j + 255.  In FP32, silu(g) = g * rcp(1 + exp2(-g log2 e))
 * from the hardware exp2 and reciprocal (within a few FP32 ulp of the exact
 * value), and h = silu(g) * u.  That FP32 h is then quantized 1x128 by the
 * rule of fp8_quantize, bit for bit: s = fl32(amax / 448) (1 when the group
 * is all zero) and q = e4m3(fl32(h / s)), both correctly rounded divisions.
 *   a, sa, b [E][n][k], sb [E][n/128][k/128], block_expert: as
 *            grouped_gemm_fp8_contiguous (b interleaved as above)
 *   q_out    uint8 [m_total][n/2]       s_out  float [n/256][m_total]
 *            (the a / sa operands of the contiguous GEMM with W2, k = n/2)
 * Blocks whose block_expert is out of range are skipped (their rows of q_out
 * and s_out are left as they were); padding rows of a (zeros) give q = 0,
 * s = 1.  n % 256 == 0 and k % 128 == 0 (else FG8_EUNSUPPORTED).
 */
fg8_status grouped_gemm_fp8_contiguous_swiglu(const uint8_t* a, const float* sa,
                                              const uint8_t* b, const float* sb,
                                              const int32_t* block_expert, uint8_t* q_out,
                                              float* s_out, int64_t m_total, int64_t n, int64_t k,
                                              int32_t num_experts, hipStream_t stream);

/*
 * grouped_gemm_fp8_kgrouped: the weight-gradient GEMM of a grouped (MoE)
 * linear layer, dW_e = dY_e^T X_e summed over the tokens routed to expert e.
 * The pages say only that training computes its gradients in the same FP8 /
 * FP32 mixed precision (cuda-deepseek blog, hrletsgo.me, backward-pass step
 * of the training loop; aitrends.kr B200 article: FP8 grouped GEMMs for the
 * DeepSeek-V3 experts in training); this layout is the library's reading.
 * The token axis is K and is shared: group g multiplies the K range
 * k_offsets[g] .. k_offsets[g+1] - 1 of both operands, both quantized 1x128
 * along K (fp8_quantize with FG8_SCALE_1x128_T of dY and X gives them):
 *   D[g][i][j] = sum_{k in group g} A[i][k] * B[j][k],
 *   A[i][k] = e4m3(a[i][k]) * sa[k/128][i],  B[j][k] = e4m3(b[j][k]) * sb[k/128][j]
 *   a  uint8 [m][k_total]      sa float [k_total/128][m]
 *   b  uint8 [n][k_total]      sb float [k_total/128][n]
 *   k_offsets  int32 [num_groups + 1], device memory: multiples of 128,
 *              non-decreasing, in [0, k_total] (the contiguous layout's
 *              expert_offsets); range-checked by the kernel (clamped)
 *   d  [num_groups][m][n] float or bfloat16 bits; an empty group's block is
 *      written with zeros.
 *   k_total % 128 == 0 and 128 <= k_total <= 2^24 - 128 (else
 *   FG8_EUNSUPPORTED); 1 <= num_groups <= 65536; m, n >= 1.
 */
fg8_status grouped_gemm_fp8_kgrouped(const uint8_t* a, const float* sa, const uint8_t* b,
                                     const float* sb, const int32_t* k_offsets, void* d,
                                     fg8_out out, int32_t num_groups, int64_t m, int64_t n,
                                     int64_t k_total, hipStream_t stream);

/*
 * moe_contiguous_layout_fp8: the step before grouped_gemm_fp8_contiguous.
 * From the router's top-k expert ids it builds the contiguous layout of the
 * DeepGEMM release news (ctol-kr.com, section 4 "MoE": the tokens of every
 * expert stacked one expert after another, each expert's run padded to the
 * 128-row M block, one expert index per block) and writes the 1x128
 * quantization of the gathered token rows, all on the device (the counts
 * never visit the host).
 *   x          [tokens][hidden] float (x_is_bf16 = 0) or bfloat16 bits (1)
 *   topk_ids   int32 [tokens][topk]: expert ids; a repeated id in a row
 *              counts once, ids outside [0, num_experts) route nowhere
 *   q          uint8 [m_cap][hidden]       sa float [hidden/128][m_cap]
 *              (the a / sa operands of grouped_gemm_fp8_contiguous)
 *   block_expert   int32 [m_cap/128]: expert of each 128-row block, -1 for
 *              the blocks past the last run (the contiguous GEMM skips them)
 *   row_token  int32 [m_cap]: source token of each row, -1 for padding
 *   token_row  int32 [tokens][topk]: the inverse map, the row holding token
 *              t's copy for its j-th id, -1 where that id routes nowhere or
 *              repeats an earlier id of the token (what the step after the
 *              second expert GEMM needs to bring a token's rows back)
 *   expert_offsets int32 [num_experts + 1]: first row of each expert's run;
 *              expert_offsets[num_experts] = rows in use
 *   expert_counts  int32 [num_experts]: tokens routed to each expert
 * Experts are laid out in id order, an expert's tokens in ascending token
 * order.  Each token row is read and quantized once and written into every
 * row that holds it; padding rows quantize as zeros (code 0, scale 1), so
 * every output is written and the result is the same on every call.  sa
 * doubles as scratch for the per-range counts before the scales are written.
 *   hidden % 128 == 0 (else FG8_EUNSUPPORTED); tokens >= 1;
 *   1 <= topk <= 256; 1 <= num_experts <= 1024; m_cap % 128 == 0 and
 *   m_cap >= fg8_moe_capacity(tokens, topk, num_experts), which holds any
 *   routing (else FG8_EINVAL).
 */
fg8_status moe_contiguous_layout_fp8(const void* x, int32_t x_is_bf16, int64_t tokens,
                                     int64_t hidden, const int32_t* topk_ids, int32_t topk,
                                     int32_t num_experts, int64_t m_cap, uint8_t* q, float* sa,
                                     int32_t* block_expert, int32_t* row_token,
                                     int32_t* token_row, int32_t* expert_offsets,
                                     int32_t* expert_counts, hipStream_t stream);

/* Rows that hold any routing of `tokens` tokens with `topk` ids each over
 * `num_experts` experts: every routed row plus up to 127 padding rows per
 * expert, rounded up to whole 128-row blocks (0 for arguments out of range). */
int64_t fg8_moe_capacity(int64_t tokens, int32_t topk, int32_t num_experts);

/* Diagnostic, host only (no GPU call): the tiling the library picks for a
 * GEMM of this shape on a device with num_cus compute units.  mode: 0 dense
 * (gemm_fp8_blockscaled; m, n, k as there), 1 contiguous (m = m_total),
 * 2 masked (m = cap, groups = experts), 3 K-grouped (m, n as the output,
 * k = total rows, groups = number of groups).  Writes out[0..4] = tile rows,
 * tile columns, K splits, workgroups launched, and the tile-order group size
 * (0: plain order).  FG8_EINVAL for a NULL out, an unknown mode, sizes < 1,
 * k not a positive multiple of 128, or num_cus < 1. */
fg8_status fg8_tile_choice(int32_t mode, int64_t m, int64_t n, int64_t k, int32_t groups,
                           int32_t num_cus, int32_t* out);

/* Text of the calling thread's last non-OK status ("" if none). */
const char* fg8_last_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int fg8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FG8_H */
