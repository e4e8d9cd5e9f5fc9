/*
 * bsg.h -- block-scaled grouped quantize and grouped GEMM for MoE expert products
 * on AMD Instinct MI355X (gfx950).  C ABI of libbsg.so.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers unless the argument comment says [host].
 * - All buffers belong to the caller.  The library keeps no per-call state,
 *   allocates no device memory, never synchronizes and never reads device memory
 *   from the host: each call only enqueues kernels on `stream` (a hipStream_t;
 *   NULL = the legacy default stream), so calls can be captured into a HIP graph.
 * - Return value: 0 (BSG_OK) on success, otherwise a bsg_status code; the
 *   message is in bsg_last_error() (thread-local, valid until the next call on
 *   the same thread).  Argument errors are detected on the host before any HIP
 *   call is made; nothing is enqueued then.
 * - Errors only the device can see (a negative group size, groups that add up
 *   to more rows than the buffers hold, padded offsets that do not fit the
 *   sizes) never cause an out-of-bounds access: offsets are clamped on the
 *   device into [0, capacity] and made non-decreasing, and the bit below is
 *   OR-ed into *dev_status (a device uint32, optional: may be NULL; the caller
 *   clears it).
 * - Row-major everywhere.  "bf16" is IEEE bfloat16 bits (uint16).  E4M3 is
 *   the OCP float8 "fn" variant (max 448, no infinities); E8M0 is a biased
 *   power-of-two exponent byte; E2M1 is the OCP fp4 element.
 */
#ifndef BSG_H
#define BSG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSG_OK = 0,
  BSG_ERR_NULL = 1,        /* a required pointer is NULL */
  BSG_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
  BSG_ERR_ALIGN = 3,       /* a data pointer is not 16-byte aligned */
  BSG_ERR_UNSUPPORTED = 4, /* a mode / dtype / flag value the library does not support */
  BSG_ERR_WORKSPACE = 5,   /* a workspace is smaller than its query function returns */
  BSG_ERR_HIP = 6          /* a HIP launch failed */
} bsg_status;

/* Bits OR-ed into *dev_status by the kernels. */
#define BSG_DEV_NEGATIVE_SIZE 1u   /* a group size < 0 was treated as 0 */
#define BSG_DEV_OVER_CAPACITY 2u   /* offsets ran past the buffer capacity; clamped */
#define BSG_DEV_BAD_PADDING   4u   /* padded offsets not multiples of 128 or smaller than
                                      the live sizes; that group was skipped */

typedef enum {
  BSG_FPROP_TN = 0,
  BSG_WGRAD_NT = 1,
  BSG_DGRAD_NN = 2,
  BSG_WGRAD_NT_E5M2 = 3
} bsg_gemm_mode;
typedef enum { BSG_OUT_BF16 = 0, BSG_OUT_F32 = 1 } bsg_out_dtype;

#define BSG_MAX_GROUPS 256
#define BSG_COLWISE_PAD 128

/* Thread-local message of the last failing call on this thread ("" if none). */
const char* bsg_last_error(void);

/* Library version, (major << 16) | minor. */
int bsg_version(void);

/*
 * group_offsets_i32_to_i64
 *
 * "[JAX] MXFP8 Grouped Quant+GEMM" (Changes list; review thread on
 * cublaslt_grouped_gemm.cu): int32 group sizes become int64 on the device, times
 * a multiplier, and their exclusive prefix sums give G + 1 offsets.  Padding to
 * a multiple (pad_to) gives the offsets of the 128-padded columnwise copies.
 *
 *   sizes      [G] int32, device.  Negative entries count as 0 (status bit 1).
 *   G          1 .. BSG_MAX_GROUPS.
 *   multiplier >= 1.  sizes_i64[g] = sizes[g] * multiplier.
 *   pad_to     >= 1.  offsets[g+1] = offsets[g] + roundup(sizes[g], pad_to) * multiplier.
 *   sizes_i64  [G] int64 output, or NULL.
 *   offsets    [G+1] int64 output; offsets[0] = 0.
 *   capacity   if > 0, offsets[G] > capacity sets status bit 2 (the offsets are
 *              still written unclamped; every consumer clamps them).
 * One wavefront-sized scan kernel; latency bound.
 */
int group_offsets_i32_to_i64(const int32_t* sizes, int64_t G, int64_t multiplier, int64_t pad_to,
                             int64_t* sizes_i64, int64_t* offsets, int64_t capacity,
                             uint32_t* dev_status, void* stream);

/*
 * grouped_quantize_mxfp8
 *
 * Grouped MXFP8 quantize of a bf16 activation split into G consecutive row
 * groups ("[JAX] MXFP8 Grouped Quant+GEMM": V2 grouped quantize with the scale
 * swizzle fused into it; contraction-direction rule of "gemm.py",
 * _quantize_gemm_operands: rowwise when the contraction is the last dim,
 * columnwise/transposed otherwise).  E4M3 elements; one E8M0 scale per 32
 * elements along the contraction dim; scale exponent = floor(log2(block amax))
 * - 8, elements rounded to nearest even and saturated at +-448.
 *
 *   x            [rows_cap, cols] bf16.  Only rows < offsets[G] are read.
 *   rows_cap     >= 0.  cols: multiple of 32, > 0.
 *   offsets      [G+1] int64 live row offsets (from group_offsets_i32_to_i64, pad 1).
 *   Rowwise output (both or neither):
 *     row_data   [rows_cap, cols] E4M3; rows >= offsets[G] untouched.
 *     row_scales E8M0 as [NQ][rows_cap] 4-byte words, NQ = ceil(cols/128): word
 *                (q, r) holds row r's four scale bytes of columns
 *                [128 q, 128 q + 128) in the order b0, b2, b1, b3; bytes past
 *                cols/32 are 0 (rows_cap * 4 * NQ bytes).  This is the order the
 *                grouped GEMM reads: 64 consecutive rows of one K-group are 256
 *                contiguous bytes, and the two bytes each half of a wavefront
 *                needs share one 16-bit half.
 *   Columnwise output (all three or none):
 *     padded_offsets [G+1] int64 (group_offsets_i32_to_i64 with pad_to 128).
 *     col_rows_cap   capacity of the columnwise buffers in padded tokens.
 *     col_data   group g: a [cols, m~_g] block (m~_g = padded_offsets[g+1] -
 *                padded_offsets[g]) at byte padded_offsets[g] * cols; token t of
 *                column c at [c, t]; tokens t >= m_g are 0x00.
 *     col_scales group g: an [m~_g/128][cols] array of words at byte
 *                padded_offsets[g] * cols / 32, word (q, c) holding column c's scale
 *                bytes of tokens [128 q, 128 q + 128) in the b0, b2, b1, b3 order;
 *                padding blocks 0x00.
 * Both directions requested in one call read x once.
 */
int grouped_quantize_mxfp8(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                           const int64_t* offsets, uint8_t* row_data, uint8_t* row_scales,
                           const int64_t* padded_offsets, int64_t col_rows_cap, uint8_t* col_data,
                           uint8_t* col_scales, uint32_t* dev_status, void* stream);

/*
 * grouped_quantize_mxfp8_rowwise_e5m2
 *
 * Rowwise MXFP8 quantize of a gradient with E5M2 elements ("gemm.py",
 * _compatible_fp8_gemm_dtypes: an E5M2 operand pairs with an E4M3 one), for the
 * MoE dgrad.  Same blocks, scale order and arguments as the rowwise part of
 * grouped_quantize_mxfp8; the E8M0 byte is exponent(amax) - 15 (the E5M2
 * maximum 57344 sits in binade 15), elements round to nearest even and
 * saturate at +-57344.
 */
int grouped_quantize_mxfp8_rowwise_e5m2(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                        const int64_t* offsets, uint8_t* row_data,
                                        uint8_t* row_scales, uint32_t* dev_status, void* stream);

/*
 * grouped_quantize_mxfp8_colwise_e5m2
 *
 * Columnwise (transposed) MXFP8 copy of a gradient with E5M2 elements, for the
 * weight gradient's E5M2 x E4M3 product ("gemm.py", _compatible_fp8_gemm_dtypes).
 * Blocks, layout, padding and arguments as the columnwise part of
 * grouped_quantize_mxfp8; the E8M0 byte is exponent(amax) - 15, elements round
 * to nearest even and saturate at +-57344 (as grouped_quantize_mxfp8_rowwise_e5m2).
 */
int grouped_quantize_mxfp8_colwise_e5m2(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                        const int64_t* offsets, const int64_t* padded_offsets,
                                        int64_t col_rows_cap, uint8_t* col_data,
                                        uint8_t* col_scales, uint32_t* dev_status, void* stream);

/*
 * grouped_quantize_nvfp4_rowscaled
 *
 * Row-scaled NVFP4 quantize ("[Common][PyTorch] Add row-scaled NVFP4 support to
 * grouped-tensor GEMM": per-row FP32 outer scale, E4M3 scale per 16 elements,
 * E2M1 elements, amax fused into the cast; outer scale amax / (6 * 448) as the
 * tensor scale of "gemm.py", _get_nvfp4_tensor_scale_inv, taken per row).
 * Float32 steps per row r and 16-element block: S = 2688 / amax_r (1 if
 * amax_r = 0, capped at FLT_MAX); s8 = E4M3((bmax / 6) * S); enc = S / decode(s8)
 * (0 if the scale is 0, capped at FLT_MAX); q = E2M1(x * enc), ties to even,
 * saturated at 6; outer[r] = amax_r / 2688.  Quantize weights with the same
 * call (rows = sum of N_e): the outer scale then is per output column.
 *
 *   x            [rows_cap, cols] bf16; rows >= offsets[G] are not read.
 *   cols         multiple of 32 (rows of more than 16384 elements are read twice).
 *   data         [rows_cap, cols/2]; element 2j in the low nibble of byte j.
 *   block_scales [rows_cap, cols/16] E4M3, row-major (the GEMM reads this order).
 *   outer        [rows_cap] float32.
 */
int grouped_quantize_nvfp4_rowscaled(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                     const int64_t* offsets, uint8_t* data, uint8_t* block_scales,
                                     float* outer, uint32_t* dev_status, void* stream);

/*
 * grouped_quantize_nvfp4_pertensor
 *
 * Per-tensor NVFP4 quantize of grouped rows, each group one tensor ("gemm.py":
 * an NVFP4 operand carries its amax, the GEMM derives the tensor scale
 * amax / (6 * 448) from it, _get_nvfp4_tensor_scale_inv; split per expert,
 * each group has its own amax, as the per-split amax entries of "[Common]
 * [PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM").  The
 * float32 steps of grouped_quantize_nvfp4_rowscaled with the group's amax in
 * place of the row's: S_g = 2688 / amax_g (1 if amax_g = 0, capped at
 * FLT_MAX); s8 = E4M3((bmax / 6) * S_g); enc = S_g / decode(s8) (0 if the
 * scale is 0, capped at FLT_MAX); q = E2M1(x * enc).  Quantize the experts'
 * weights with offsets at the expert boundaries (0, N_0, N_0 + N_1, ...).
 *
 *   x            [rows_cap, cols] bf16; only rows in [offsets[0], offsets[G]) are
 *                read.
 *   cols         multiple of 32 (rows of more than 16384 elements are read twice).
 *   data         [rows_cap, cols/2]; element 2j in the low nibble of byte j.
 *   block_scales [rows_cap, cols/16] E4M3, row-major.  Rows outside
 *                [offsets[0], offsets[G]) (no group owns them) are untouched.
 *   amax         [G] float32 output: each group's largest magnitude (0 for an
 *                empty group).  Three launches: clear amax, group amax (atomic
 *                max per group), cast.
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE, BSG_ERR_ALIGN (x and data 16-byte, amax
 * 4-byte).
 */
int grouped_quantize_nvfp4_pertensor(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                     const int64_t* offsets, uint8_t* data, uint8_t* block_scales,
                                     float* amax, uint32_t* dev_status, void* stream);

/*
 * grouped_quantize_nvfp4_pertensor_rht
 *
 * grouped_quantize_nvfp4_pertensor of the rows' randomized Hadamard transform
 * along the contraction ("gemm.py", _quantize_gemm_operands: with NVFP4 1-D
 * scaling, if one GEMM operand is quantized with RHT the other must be too,
 * so that the transform cancels in the GEMM; quantize both operands with the
 * same mask and multiply them with grouped_gemm_nvfp4_pertensor).  Every
 * 16-element block x of a row becomes y = (1/4) H16 diag(s) x -- H16 the
 * 16 x 16 Sylvester Hadamard matrix, s_i = -1 where bit i of rht_sign_mask is
 * set -- computed in float32 as: sign flips, a butterfly of four stages d = 1,
 * 2, 4, 8 (each replacing (y[i], y[i + d]) by (y[i] + y[i + d], y[i] - y[i + d])
 * for the i with bit d clear), the exact product by 1/4.  amax[g] is the
 * largest transformed magnitude of group g; the cast then follows
 * grouped_quantize_nvfp4_pertensor's float32 steps on the transformed values.
 * (The pages give neither the size nor the signs of the transform: 16, the
 * NVFP4 block, and caller-chosen signs are this library's reading.)
 *
 *   rht_sign_mask  [host] the 16 signs, bits 0..15 (higher bits: BSG_ERR_SHAPE).
 *   Other arguments, outputs and errors as grouped_quantize_nvfp4_pertensor.
 */
int grouped_quantize_nvfp4_pertensor_rht(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                         const int64_t* offsets, uint32_t rht_sign_mask,
                                         uint8_t* data, uint8_t* block_scales, float* amax,
                                         uint32_t* dev_status, void* stream);

/*
 * grouped_quantize_nvfp4_pertensor_2d
 *
 * Per-tensor NVFP4 with 2-D block scales ("gemm.py", _jax_scaled_matmul accepts
 * an NVFP4_2D_SCALING mode): one E4M3 scale per 16 x 16 block -- 16 rows by 16
 * columns, so a tensor and its transpose quantize to transposed codes -- whose
 * maximum is taken over the whole block, with the float32 steps of
 * grouped_quantize_nvfp4_pertensor (S_g from the group's amax).  Block rows
 * start at each group's first row; a group's last block row holds its
 * remaining rows.  block_scales keeps the per-row layout [rows_cap, cols/16]:
 * each row of a block row carries its block's scale byte, so
 * grouped_gemm_nvfp4_pertensor consumes the outputs unchanged.  (The pages give
 * no block shape: 16 x 16 is this library's reading.)
 *
 *   Arguments, outputs and errors as grouped_quantize_nvfp4_pertensor.
 */
int grouped_quantize_nvfp4_pertensor_2d(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                        const int64_t* offsets, uint8_t* data,
                                        uint8_t* block_scales, float* amax, uint32_t* dev_status,
                                        void* stream);

/*
 * grouped_quantize_nvfp4_rowscaled_colwise
 *
 * Columnwise (transposed) row-scaled NVFP4 copies for the weight gradient
 * ("[Common][PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM":
 * columnwise use of row-scaled grouped tensors, the columnwise amax sized per
 * column and split per expert).  Per expert g the block X_g^T [cols, m~_g]
 * (tokens padded with zeros to m~_g) is quantized row by row with the float32
 * steps of grouped_quantize_nvfp4_rowscaled: column c of expert g gets the
 * outer scale amax / 2688 over the expert's tokens, each 16-token block an E4M3
 * scale, each token an E2M1 code.
 *
 *   x              [rows_cap, cols] bf16; rows >= offsets[G] are not read.
 *   cols           multiple of 32.
 *   offsets        [G+1] int64 live token offsets (group_offsets_i32_to_i64, pad 1).
 *   padded_offsets [G+1] int64 (group_offsets_i32_to_i64 with pad_to 128);
 *                  a group whose padded offsets are not multiples of 128 or
 *                  smaller than its size is skipped and flagged (bit 2).
 *   col_rows_cap   capacity of the outputs in padded tokens (>= padded_offsets[G]).
 *   data           expert g: a [cols, m~_g / 2] byte block at byte
 *                  padded_offsets[g] * cols / 2; token 2j of a column in the low
 *                  nibble of byte j; padding tokens encode to 0.
 *   block_scales   expert g: a [cols, m~_g / 16] E4M3 block at byte
 *                  padded_offsets[g] * cols / 16 (padding blocks 0x00).
 *   outer          [G, cols] float32 (0 for an empty expert).
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE, BSG_ERR_ALIGN (x and data 16-byte, outer
 * 4-byte).
 */
int grouped_quantize_nvfp4_rowscaled_colwise(const void* x, int64_t rows_cap, int64_t cols,
                                             int64_t G, const int64_t* offsets,
                                             const int64_t* padded_offsets, int64_t col_rows_cap,
                                             uint8_t* data, uint8_t* block_scales, float* outer,
                                             uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_mxfp8
 *
 * One launch over all groups of a grouped MXFP8 GEMM with FP32 accumulation
 * ("gemm.py", grouped_gemm; "[JAX] MXFP8 Grouped Quant+GEMM": V2 grouped GEMM
 * extended to MXFP8, graph-safe).  Each operand is K-major E4M3 data with E8M0
 * scales per 32 along the contraction in the order grouped_quantize_mxfp8 writes.
 *
 * mode BSG_FPROP_TN (ragged rows; output rows follow the lhs groups):
 *   Y[r, n] = sum_k A[r, k] * B[g, n, k]   for r in [offsets[g], offsets[g+1])
 *   a        [rows_cap, k] E4M3 rowwise,  a_scales [ceil(k/128)][rows_cap] words
 *   b        [G, n, k] E4M3 rowwise,      b_scales [ceil(k/128)][G * n] words (the weights
 *            quantized by grouped_quantize_mxfp8 as G * n rows)
 *   offsets  [G+1] live row offsets; rows_cap = rows of a and out
 *   out      [rows_cap, n]; rows >= offsets[G] untouched.
 * mode BSG_WGRAD_NT (ragged contraction; uniform (G, n, k) output):
 *   dW[g, i, j] = sum_t dY[t, i] * X[t, j] over the tokens t of group g
 *   a        columnwise dY copy (grouped_quantize_mxfp8 col_data with cols = n)
 *   b        columnwise X copy (cols = k); a_scales / b_scales their col_scales
 *   offsets  [G+1] padded (multiple-of-128) token offsets of those copies;
 *            rows_cap = their capacity in padded tokens
 *   out      [G, n, k]; a group with no tokens gets zeros.
 * mode BSG_DGRAD_NN (MoE dgrad, dX = dY W_g; an E5M2 gradient times E4M3
 * weights, a pairing "gemm.py" _compatible_fp8_gemm_dtypes accepts):
 *   dX[r, j] = sum_i dY[r, i] * W[g, i, j]   for r in [offsets[g], offsets[g+1])
 *   a        [rows_cap, k] E5M2 rowwise dY (grouped_quantize_mxfp8_rowwise_e5m2,
 *            cols = k, the contraction), a_scales [ceil(k/128)][rows_cap] words
 *   b        the columnwise copy of the weights W [G, k, n] viewed as G * k rows
 *            of n columns (grouped_quantize_mxfp8 col_data with offsets g * k and
 *            padded offsets g * kp, kp = k rounded up to a multiple of 128):
 *            expert g's [n, kp] block at byte g * n * kp, i.e. W_g transposed,
 *            quantized along k, zero past k; b_scales its col_scales ([kp/128][n]
 *            words per expert, at byte g * n * kp / 32)
 *   offsets, rows_cap, out as in FPROP (out [rows_cap, n]).
 * mode BSG_WGRAD_NT_E5M2: BSG_WGRAD_NT with an E5M2 gradient (dW = dY^T X, an
 *   E5M2 x E4M3 product "gemm.py" _compatible_fp8_gemm_dtypes accepts): a is dY's
 *   columnwise copy from grouped_quantize_mxfp8_colwise_e5m2, b is X's E4M3
 *   columnwise copy; everything else as BSG_WGRAD_NT.
 * k: any positive multiple of 32 (FPROP, DGRAD; "gemm.py",
 * assert_cublas_requirements asks only for the block multiple).  No data byte
 * past k in a row is read; the scale bytes of the last word past k/32 multiply
 * zeros there and may hold any value but 0xFF (grouped_quantize_mxfp8 writes
 * 0x00).  n >= 1.  out_dtype: BSG_OUT_BF16 (round to nearest even) or
 * BSG_OUT_F32.
 */
int grouped_gemm_mxfp8(int mode, int64_t G, const uint8_t* a, const uint8_t* a_scales,
                       const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                       int64_t rows_cap, int64_t n, int64_t k, void* out, int out_dtype,
                       uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_mxfp8_workspace_size / grouped_gemm_mxfp8_ws
 *
 * grouped_gemm_mxfp8 with a workspace that removes most of its last, partly
 * filled round of output tiles (a persistent grid of one workgroup per compute
 * unit takes the tiles in rounds; with T tiles and P workgroups the last round
 * holds T mod P and leaves the rest idle).  FPROP and DGRAD, whose tiles all
 * contract k, split each tile of that round along the contraction into S parts
 * (2 <= S <= 8, at most P / (T mod P), each at least two 64-deep K-steps
 * pairs); the parts' FP32 accumulators go to the workspace and a second kernel
 * on the same stream adds them in a fixed order and stores the tiles.  The
 * result is deterministic, but a split tile's sums are rounded in a different
 * order than grouped_gemm_mxfp8's (differences within FP32 rounding); WGRAD
 * modes never split.  Same arguments and errors as grouped_gemm_mxfp8, plus:
 *   workspace        [device] grouped_gemm_mxfp8_workspace_size() bytes, 256-byte
 *                    aligned, owned by the caller; its contents on entry do not
 *                    matter, and calls that share it must not overlap.
 *   workspace_bytes  its size: less than the query gives BSG_ERR_WORKSPACE; NULL
 *                    workspace BSG_ERR_NULL; misaligned BSG_ERR_ALIGN.
 * The size depends on the current device's compute-unit count: 16 KiB plus
 * 256 KiB per unit (64 MiB on 256 units).
 */
size_t grouped_gemm_mxfp8_workspace_size(void);
int grouped_gemm_mxfp8_ws(int mode, int64_t G, const uint8_t* a, const uint8_t* a_scales,
                          const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                          int64_t rows_cap, int64_t n, int64_t k, void* out, int out_dtype,
                          void* workspace, size_t workspace_bytes, uint32_t* dev_status,
                          void* stream);

/*
 * grouped_gemm_mxfp8_ex
 *
 * grouped_gemm_mxfp8 with the per-group epilogue of "gemm.py" grouped_gemm (a
 * bias of shape (num_gemms, N) over the output columns; per-group float32
 * alpha and beta, defaults 1 and 0) and the copy-or-accumulate output of the
 * row-scaled NVFP4 flow, e.g. accumulating into an FP32 main-grad:
 *   out[r, j] = alpha[g] * S[r, j] + beta[g] * out_previous[r, j] + bias[g, j]
 * combined in float32 and rounded once to out_dtype; out_previous is read only
 * for groups with beta[g] != 0.  S, g, modes and the other arguments as in
 * grouped_gemm_mxfp8 (the output columns are n in FPROP / DGRAD, k in WGRAD).
 *   alpha  [G] float32 or NULL (all 1);  beta [G] float32 or NULL (all 0)
 *   bias   [G, output columns] float32 or NULL; needs a multiple of 4 columns
 * With all three NULL it is grouped_gemm_mxfp8.
 * Errors: those of grouped_gemm_mxfp8, plus BSG_ERR_ALIGN (alpha / beta 4-byte,
 * bias 16-byte) and BSG_ERR_SHAPE (bias with output columns not a multiple of 4).
 */
int grouped_gemm_mxfp8_ex(int mode, int64_t G, const uint8_t* a, const uint8_t* a_scales,
                          const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                          int64_t rows_cap, int64_t n, int64_t k, void* out, int out_dtype,
                          const float* alpha, const float* beta, const float* bias,
                          uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_nvfp4_rowscaled
 *
 * Row-scaled NVFP4 grouped GEMM ("[Common][PyTorch] Add row-scaled NVFP4
 * support to grouped-tensor GEMM": the per-row / per-column FP32 outer scale is
 * neutralized in the GEMM, the product is accumulated in FP32, and the outer
 * scales are applied afterwards over each group's own live rows and its own
 * output width -- the Greptile finding on differing output widths and capacity
 * rows, and its fix):
 *   S[r, n] = sum_k e2m1(A)[r,k] * sA[r, k/16] * e2m1(B_g)[n,k] * sB_g[n, k/16]
 *   Y[r, n] = S[r, n] * a_outer[r] * b_outer_g[n]   for r live in g, n < N_g
 *
 *   a, a_scales, a_outer  grouped_quantize_nvfp4_rowscaled outputs, [rows_cap] rows
 *   offsets               [G+1] live row offsets
 *   b, b_scales, b_outer  the experts' [N_g, k] weights quantized one after
 *                         another (sum N_g rows)
 *   n_per_group           [host] [G] int64 output width of each group, >= 0
 *   out                   [rows_cap, ld_out]; ld_out >= max N_g.  Columns >= N_g of
 *                         group g's rows and rows >= offsets[G] are untouched.
 *   scratch               NULL: the outer scales are applied in the GEMM's
 *                         epilogue.  Otherwise a [rows_cap, ld_out] float32 buffer:
 *                         S is stored there first and a second kernel applies the
 *                         outer scales into out (the pages' two-step flow); rows
 *                         outside [offsets[0], offsets[G]) stay untouched.
 * k: any positive multiple of 32 ("gemm.py", assert_cublas_requirements: the
 * contracting dim of an NVFP4 GEMM needs only that multiple); no byte past k
 * of a row (data or block scales) is read.
 */
int grouped_gemm_nvfp4_rowscaled(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                 const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                                 int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                 const float* b_outer, const int64_t* n_per_group, void* out,
                                 int64_t ld_out, int out_dtype, float* scratch,
                                 uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_nvfp4_rowscaled_ex
 *
 * grouped_gemm_nvfp4_rowscaled with the copy-or-accumulate output of its flow
 * ("[Common][PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM",
 * Greptile flow: apply the outer scales, then copy or accumulate into the
 * output; an accumulate flag rather than a general beta, which that path
 * rejects):
 *   accumulate 0: out = Y (as grouped_gemm_nvfp4_rowscaled)
 *   accumulate 1: out = out_previous + Y, added in float32 and rounded once
 *                 to out_dtype (e.g. accumulating into an FP32 buffer)
 * for the same live rows and columns n < N_g; everything else untouched.  With
 * a scratch the post-scale kernel accumulates.  Other values: BSG_ERR_UNSUPPORTED.
 */
int grouped_gemm_nvfp4_rowscaled_ex(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                    const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                                    int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                    const float* b_outer, const int64_t* n_per_group, void* out,
                                    int64_t ld_out, int out_dtype, float* scratch, int accumulate,
                                    uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_nvfp4_rowscaled_noalloc
 *
 * For callers that cannot allocate device memory -- code under HIP-graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the two-step
 * flow of grouped_gemm_nvfp4_rowscaled (FP32 S first, then a post-scale kernel
 * applies the outer scales) with S in a static device array that the library
 * owns, instead of a caller scratch.  Arguments, results and errors are those
 * of grouped_gemm_nvfp4_rowscaled with a non-NULL scratch; the outputs are
 * bit-identical to it.
 *   Limit: rows_cap * ld_out * 4 <= BSG_NOALLOC_SCRATCH_BYTES (64 MiB), else
 *   BSG_ERR_SHAPE and nothing is enqueued.
 * Each GPU the library runs on holds its own copy of the array until the
 * process ends; its device address is looked up on the first call on that
 * GPU (with it current).  Every call on one GPU shares the array: calls that
 * overlap on one GPU (concurrent streams, or threads) race and must be
 * serialized by the caller.  No hipMalloc, hipFree or allocating library
 * routine is called.
 */
#define BSG_NOALLOC_SCRATCH_BYTES (64u << 20)
int grouped_gemm_nvfp4_rowscaled_noalloc(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                         const float* a_outer, const int64_t* offsets,
                                         int64_t rows_cap, int64_t k, const uint8_t* b,
                                         const uint8_t* b_scales, const float* b_outer,
                                         const int64_t* n_per_group, void* out, int64_t ld_out,
                                         int out_dtype, uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_nvfp4_pertensor
 *
 * Per-tensor NVFP4 grouped GEMM ("gemm.py": for NVFP4 operands alpha is the
 * product of the two tensor scales, alpha = tsi(amax_lhs) * tsi(amax_rhs),
 * tsi(a) = a / (6 * 448), and the product is scaled by it; the graph-safe
 * grouped GEMM takes one float32 alpha per group):
 *   S[r, n]  = sum_k e2m1(A)[r,k] * sA[r, k/16] * e2m1(B_g)[n,k] * sB_g[n, k/16]
 *   alpha_g  = (a_amax[g] / 2688) * (b_amax[g] / 2688)      (float32)
 *   Y[r, n]  = S[r, n] * alpha_g     for r live in g, n < N_g
 *
 *   a, a_scales, a_amax  grouped_quantize_nvfp4_pertensor outputs ([rows_cap] rows)
 *   offsets              [G+1] live row offsets
 *   b, b_scales, b_amax  the experts' [N_g, k] weights quantized one after another
 *                        with one group per expert (b_amax [G])
 *   n_per_group          [host] [G] int64 output width of each group, >= 0
 *   out                  [rows_cap, ld_out]; ld_out >= max N_g.  Columns >= N_g of
 *                        group g's rows and rows >= offsets[G] are untouched.
 * k: any positive multiple of 32.  Errors as grouped_gemm_nvfp4_rowscaled.
 */
int grouped_gemm_nvfp4_pertensor(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                 const float* a_amax, const int64_t* offsets, int64_t rows_cap,
                                 int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                 const float* b_amax, const int64_t* n_per_group, void* out,
                                 int64_t ld_out, int out_dtype, uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_nvfp4_workspace_size / grouped_gemm_nvfp4_rowscaled_ws /
 * grouped_gemm_nvfp4_pertensor_ws
 *
 * The row-scaled NVFP4 GEMM with its fused outer-scale epilogue (and the
 * copy-or-accumulate flag of grouped_gemm_nvfp4_rowscaled_ex), and the
 * per-tensor NVFP4 GEMM, with a workspace that removes most of their last,
 * partly filled round of output tiles, as grouped_gemm_mxfp8_ws does: each
 * tile of that round is split along the contraction into S parts (2 <= S <= 8,
 * at most P / (T mod P) for T tiles on P workgroups, each part at least two
 * 128-deep stages), the parts' FP32 sums go to the workspace, and a second
 * kernel on the same stream adds them in a fixed order, then applies
 * (S * a_outer[r]) * b_outer[n] -- per-tensor: S * alpha_g -- and the store (or
 * accumulate) exactly as the fused epilogue does.  Deterministic; a split
 * tile's S is summed in a different order than without the workspace
 * (differences within FP32 rounding).  Arguments and errors as
 * grouped_gemm_nvfp4_rowscaled_ex (no scratch: the fused epilogue only) and
 * grouped_gemm_nvfp4_pertensor, plus:
 *   workspace        [device] grouped_gemm_nvfp4_workspace_size() bytes, 256-byte
 *                    aligned, owned by the caller; its contents on entry do not
 *                    matter, and calls that share it must not overlap.
 *   workspace_bytes  its size: less than the query gives BSG_ERR_WORKSPACE; NULL
 *                    workspace BSG_ERR_NULL; misaligned BSG_ERR_ALIGN.
 * The size depends on the current device's compute-unit count: 16 KiB plus
 * 256 KiB per unit (64 MiB on 256 units).
 */
size_t grouped_gemm_nvfp4_workspace_size(void);
int grouped_gemm_nvfp4_rowscaled_ws(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                    const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                                    int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                    const float* b_outer, const int64_t* n_per_group, void* out,
                                    int64_t ld_out, int out_dtype, int accumulate, void* workspace,
                                    size_t workspace_bytes, uint32_t* dev_status, void* stream);
int grouped_gemm_nvfp4_pertensor_ws(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                    const float* a_amax, const int64_t* offsets, int64_t rows_cap,
                                    int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                    const float* b_amax, const int64_t* n_per_group, void* out,
                                    int64_t ld_out, int out_dtype, void* workspace,
                                    size_t workspace_bytes, uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_nvfp4_rowscaled_wgrad
 *
 * Row-scaled NVFP4 weight gradient, NT, over each expert's ragged tokens
 * ("[Common][PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM":
 * wgrad consumes the columnwise copies; the outer scales are neutralized in
 * the GEMM and applied afterwards per expert, over its own rows and columns):
 *   S[g, i, j]  = sum_{t < m~_g} (e2m1 * sd)(A_g)[i, t] * (e2m1 * sd)(B_g)[j, t]
 *   dW[g, i, j] = (S * a_outer[g, i]) * b_outer[g, j]       (float32)
 * with A = the columnwise copy of dY ([n, m~_g] per expert) and B that of X
 * ([k, m~_g] per expert), both as written by
 * grouped_quantize_nvfp4_rowscaled_colwise.  One launch for all experts; the
 * outer-scale epilogue is fused (no FP32 scratch).
 *
 *   a, a_scales, a_outer  dY copies: data, E4M3 block scales, f32 [G, n].
 *   b, b_scales, b_outer  X copies: data, E4M3 block scales, f32 [G, k].
 *   padded_offsets [G+1] int64 (pad 128); col_rows_cap as for the quantize.
 *   n, k           dW dims, positive multiples of 32.
 *   out            [G, n, k] bf16 or f32 (out_dtype); an empty expert's block is
 *                  0, as is that of an expert whose padded offsets are not
 *                  multiples of 128 (also flagged, bit 2 of *dev_status).
 * Errors: BSG_ERR_NULL, BSG_ERR_SHAPE, BSG_ERR_UNSUPPORTED (out_dtype),
 * BSG_ERR_ALIGN (a, b 16-byte; scales, outer scales, out 4-byte).
 */
int grouped_gemm_nvfp4_rowscaled_wgrad(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                       const float* a_outer, const uint8_t* b,
                                       const uint8_t* b_scales, const float* b_outer,
                                       const int64_t* padded_offsets, int64_t col_rows_cap,
                                       int64_t n, int64_t k, void* out, int out_dtype,
                                       uint32_t* dev_status, void* stream);

/*
 * grouped_gemm_nvfp4_rowscaled_wgrad_ex
 *
 * grouped_gemm_nvfp4_rowscaled_wgrad with the flow's copy-or-accumulate output:
 * accumulate 1 gives dW[g] = dW_previous[g] + (S * a_outer) * b_outer, added in
 * float32 and rounded once (e.g. into an FP32 main-grad; an empty expert leaves
 * its block as it was); accumulate 0 is grouped_gemm_nvfp4_rowscaled_wgrad.
 */
int grouped_gemm_nvfp4_rowscaled_wgrad_ex(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                          const float* a_outer, const uint8_t* b,
                                          const uint8_t* b_scales, const float* b_outer,
                                          const int64_t* padded_offsets, int64_t col_rows_cap,
                                          int64_t n, int64_t k, void* out, int out_dtype,
                                          int accumulate, uint32_t* dev_status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSG_H */
