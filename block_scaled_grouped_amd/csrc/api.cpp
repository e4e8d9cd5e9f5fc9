// C-ABI entry points of libbsg (declared in include/bsg.h): host-side argument
// validation, then the kernel launchers.  No allocation, no synchronization, no
// device reads from the host.
#include "../../include/bsg.h"

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "bsg_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return BSG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int hip_result(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(BSG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Largest byte span a single GEMM / quantize tile addresses with 32-bit offsets.
constexpr int64_t kMaxTileBytes = (int64_t)1 << 31;

}  // namespace

extern "C" {

const char* bsg_last_error(void) { return g_err; }

int bsg_version(void) { return (0 << 16) | 1; }

int group_offsets_i32_to_i64(const int32_t* sizes, int64_t G, int64_t multiplier, int64_t pad_to,
                             int64_t* sizes_i64, int64_t* offsets, int64_t capacity,
                             uint32_t* dev_status, void* stream) {
  if (sizes == nullptr || offsets == nullptr)
    return fail(BSG_ERR_NULL, "group_offsets_i32_to_i64: sizes and offsets must be non-NULL");
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "group_offsets_i32_to_i64: G=%lld outside [1, %d]", (long long)G,
                BSG_MAX_GROUPS);
  if (multiplier < 1 || pad_to < 1)
    return fail(BSG_ERR_SHAPE, "group_offsets_i32_to_i64: multiplier=%lld and pad_to=%lld must be >= 1",
                (long long)multiplier, (long long)pad_to);
  if (((int64_t)1 << 31) * pad_to > ((int64_t)1 << 62) / multiplier)
    return fail(BSG_ERR_SHAPE, "group_offsets_i32_to_i64: multiplier * pad_to too large");
  return hip_result(bsg::launch_group_offsets(sizes, (int)G, multiplier, pad_to, sizes_i64, offsets,
                                              capacity, dev_status, (hipStream_t)stream),
                    "group_offsets_i32_to_i64");
}

int grouped_quantize_mxfp8(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                           const int64_t* offsets, uint8_t* row_data, uint8_t* row_scales,
                           const int64_t* padded_offsets, int64_t col_rows_cap, uint8_t* col_data,
                           uint8_t* col_scales, uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_quantize_mxfp8";
  if (x == nullptr || offsets == nullptr) return fail(BSG_ERR_NULL, "%s: x and offsets must be non-NULL", fn);
  const bool row = row_data != nullptr || row_scales != nullptr;
  const bool col = padded_offsets != nullptr || col_data != nullptr || col_scales != nullptr;
  if (row && (row_data == nullptr || row_scales == nullptr))
    return fail(BSG_ERR_NULL, "%s: row_data and row_scales go together", fn);
  if (col && (padded_offsets == nullptr || col_data == nullptr || col_scales == nullptr))
    return fail(BSG_ERR_NULL, "%s: padded_offsets, col_data and col_scales go together", fn);
  if (!row && !col) return fail(BSG_ERR_NULL, "%s: no output requested", fn);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || cols <= 0 || cols % 32 != 0)
    return fail(BSG_ERR_SHAPE, "%s: need rows_cap >= 0 and cols a positive multiple of 32 (got %lld, %lld)",
                fn, (long long)rows_cap, (long long)cols);
  if (col && (col_rows_cap < 0 || col_rows_cap * cols >= ((int64_t)1 << 40)))
    return fail(BSG_ERR_SHAPE, "%s: col_rows_cap=%lld out of range", fn, (long long)col_rows_cap);
  if (!aligned16(x) || (row && !aligned16(row_data)) || (col && !aligned16(col_data)))
    return fail(BSG_ERR_ALIGN, "%s: x, row_data and col_data must be 16-byte aligned", fn);
  if (row && !aligned4(row_scales))
    return fail(BSG_ERR_ALIGN, "%s: row_scales must be 4-byte aligned", fn);
  hipStream_t s = (hipStream_t)stream;
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (col) {
    // one pass over x for both directions when both are requested
    return hip_result(bsg::launch_quantize_mxfp8_colwise(xb, rows_cap, cols, (int)G, offsets,
                                                         padded_offsets, col_rows_cap, col_data,
                                                         col_scales, row ? row_data : nullptr,
                                                         row ? row_scales : nullptr, dev_status, s),
                      fn);
  }
  return hip_result(bsg::launch_quantize_mxfp8_rowwise(xb, rows_cap, cols, (int)G, offsets, row_data,
                                                       row_scales, dev_status, s),
                    fn);
}

int grouped_quantize_mxfp8_colwise_e5m2(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                        const int64_t* offsets, const int64_t* padded_offsets,
                                        int64_t col_rows_cap, uint8_t* col_data,
                                        uint8_t* col_scales, uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_quantize_mxfp8_colwise_e5m2";
  if (x == nullptr || offsets == nullptr || padded_offsets == nullptr || col_data == nullptr ||
      col_scales == nullptr)
    return fail(BSG_ERR_NULL, "%s: x, offsets, padded_offsets, col_data and col_scales must be non-NULL",
                fn);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || cols <= 0 || cols % 32 != 0)
    return fail(BSG_ERR_SHAPE, "%s: need rows_cap >= 0 and cols a positive multiple of 32 (got %lld, %lld)",
                fn, (long long)rows_cap, (long long)cols);
  if (col_rows_cap < 0 || col_rows_cap * cols >= ((int64_t)1 << 40))
    return fail(BSG_ERR_SHAPE, "%s: col_rows_cap=%lld out of range", fn, (long long)col_rows_cap);
  if (!aligned16(x) || !aligned16(col_data))
    return fail(BSG_ERR_ALIGN, "%s: x and col_data must be 16-byte aligned", fn);
  return hip_result(bsg::launch_quantize_mxfp8_colwise(static_cast<const uint16_t*>(x), rows_cap,
                                                       cols, (int)G, offsets, padded_offsets,
                                                       col_rows_cap, col_data, col_scales, nullptr,
                                                       nullptr, dev_status, (hipStream_t)stream,
                                                       true),
                    fn);
}

int grouped_quantize_mxfp8_rowwise_e5m2(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                        const int64_t* offsets, uint8_t* row_data,
                                        uint8_t* row_scales, uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_quantize_mxfp8_rowwise_e5m2";
  if (x == nullptr || offsets == nullptr || row_data == nullptr || row_scales == nullptr)
    return fail(BSG_ERR_NULL, "%s: x, offsets, row_data and row_scales must be non-NULL", fn);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || cols <= 0 || cols % 32 != 0)
    return fail(BSG_ERR_SHAPE, "%s: need rows_cap >= 0 and cols a positive multiple of 32 (got %lld, %lld)",
                fn, (long long)rows_cap, (long long)cols);
  if (!aligned16(x) || !aligned16(row_data) || !aligned4(row_scales))
    return fail(BSG_ERR_ALIGN, "%s: x and row_data must be 16-byte aligned, row_scales 4-byte", fn);
  return hip_result(bsg::launch_quantize_mxfp8_rowwise(static_cast<const uint16_t*>(x), rows_cap,
                                                       cols, (int)G, offsets, row_data, row_scales,
                                                       dev_status, (hipStream_t)stream, true),
                    fn);
}

int grouped_quantize_nvfp4_rowscaled(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                     const int64_t* offsets, uint8_t* data, uint8_t* block_scales,
                                     float* outer, uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_quantize_nvfp4_rowscaled";
  if (x == nullptr || offsets == nullptr || data == nullptr || block_scales == nullptr || outer == nullptr)
    return fail(BSG_ERR_NULL, "%s: x, offsets, data, block_scales and outer must be non-NULL", fn);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || cols <= 0 || cols % 32 != 0)
    return fail(BSG_ERR_SHAPE, "%s: need rows_cap >= 0 and cols a positive multiple of 32", fn);
  if (rows_cap > 0x7fffffffLL) return fail(BSG_ERR_SHAPE, "%s: rows_cap too large", fn);
  if (!aligned16(x) || !aligned16(data) || !aligned4(outer))
    return fail(BSG_ERR_ALIGN, "%s: x and data must be 16-byte aligned, outer 4-byte", fn);
  return hip_result(bsg::launch_quantize_nvfp4_rowscaled(static_cast<const uint16_t*>(x), rows_cap,
                                                         cols, (int)G, offsets, data, block_scales,
                                                         outer, dev_status, (hipStream_t)stream),
                    fn);
}

int grouped_quantize_nvfp4_pertensor(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                     const int64_t* offsets, uint8_t* data, uint8_t* block_scales,
                                     float* amax, uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_quantize_nvfp4_pertensor";
  if (x == nullptr || offsets == nullptr || data == nullptr || block_scales == nullptr || amax == nullptr)
    return fail(BSG_ERR_NULL, "%s: x, offsets, data, block_scales and amax must be non-NULL", fn);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || cols <= 0 || cols % 32 != 0)
    return fail(BSG_ERR_SHAPE, "%s: need rows_cap >= 0 and cols a positive multiple of 32", fn);
  if (rows_cap > 0x7fffffffLL) return fail(BSG_ERR_SHAPE, "%s: rows_cap too large", fn);
  if (!aligned16(x) || !aligned16(data) || !aligned4(amax))
    return fail(BSG_ERR_ALIGN, "%s: x and data must be 16-byte aligned, amax 4-byte", fn);
  return hip_result(bsg::launch_quantize_nvfp4_pertensor(static_cast<const uint16_t*>(x), rows_cap,
                                                         cols, (int)G, offsets, data, block_scales,
                                                         amax, dev_status, (hipStream_t)stream),
                    fn);
}

static int pertensor_args(const char* fn, const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                          const int64_t* offsets, const uint8_t* data, const uint8_t* block_scales,
                          const float* amax) {
  if (x == nullptr || offsets == nullptr || data == nullptr || block_scales == nullptr || amax == nullptr)
    return fail(BSG_ERR_NULL, "%s: x, offsets, data, block_scales and amax must be non-NULL", fn);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || cols <= 0 || cols % 32 != 0)
    return fail(BSG_ERR_SHAPE, "%s: need rows_cap >= 0 and cols a positive multiple of 32", fn);
  if (rows_cap > 0x7fffffffLL) return fail(BSG_ERR_SHAPE, "%s: rows_cap too large", fn);
  if (!aligned16(x) || !aligned16(data) || !aligned4(amax))
    return fail(BSG_ERR_ALIGN, "%s: x and data must be 16-byte aligned, amax 4-byte", fn);
  return BSG_OK;
}

int grouped_quantize_nvfp4_pertensor_rht(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                         const int64_t* offsets, uint32_t rht_sign_mask,
                                         uint8_t* data, uint8_t* block_scales, float* amax,
                                         uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_quantize_nvfp4_pertensor_rht";
  const int rc = pertensor_args(fn, x, rows_cap, cols, G, offsets, data, block_scales, amax);
  if (rc != BSG_OK) return rc;
  if (rht_sign_mask > 0xffffu)
    return fail(BSG_ERR_SHAPE, "%s: rht_sign_mask has bits above the 16 signs", fn);
  return hip_result(bsg::launch_quantize_nvfp4_pertensor_rht(static_cast<const uint16_t*>(x),
                                                             rows_cap, cols, (int)G, offsets,
                                                             rht_sign_mask, data, block_scales,
                                                             amax, dev_status, (hipStream_t)stream),
                    fn);
}

int grouped_quantize_nvfp4_pertensor_2d(const void* x, int64_t rows_cap, int64_t cols, int64_t G,
                                        const int64_t* offsets, uint8_t* data,
                                        uint8_t* block_scales, float* amax, uint32_t* dev_status,
                                        void* stream) {
  const char* fn = "grouped_quantize_nvfp4_pertensor_2d";
  const int rc = pertensor_args(fn, x, rows_cap, cols, G, offsets, data, block_scales, amax);
  if (rc != BSG_OK) return rc;
  return hip_result(bsg::launch_quantize_nvfp4_pertensor_2d(static_cast<const uint16_t*>(x),
                                                            rows_cap, cols, (int)G, offsets, data,
                                                            block_scales, amax, dev_status,
                                                            (hipStream_t)stream),
                    fn);
}

int grouped_quantize_nvfp4_rowscaled_colwise(const void* x, int64_t rows_cap, int64_t cols,
                                             int64_t G, const int64_t* offsets,
                                             const int64_t* padded_offsets, int64_t col_rows_cap,
                                             uint8_t* data, uint8_t* block_scales, float* outer,
                                             uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_quantize_nvfp4_rowscaled_colwise";
  if (x == nullptr || offsets == nullptr || padded_offsets == nullptr || data == nullptr ||
      block_scales == nullptr || outer == nullptr)
    return fail(BSG_ERR_NULL,
                "%s: x, offsets, padded_offsets, data, block_scales and outer must be non-NULL", fn);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || col_rows_cap < 0 || cols <= 0 || cols % 32 != 0)
    return fail(BSG_ERR_SHAPE,
                "%s: need rows_cap >= 0, col_rows_cap >= 0 and cols a positive multiple of 32", fn);
  if (rows_cap > 0x7fffffffLL || col_rows_cap > 0x7fffffffLL)
    return fail(BSG_ERR_SHAPE, "%s: rows_cap or col_rows_cap too large", fn);
  if (!aligned16(x) || !aligned16(data) || !aligned4(outer))
    return fail(BSG_ERR_ALIGN, "%s: x and data must be 16-byte aligned, outer 4-byte", fn);
  return hip_result(bsg::launch_quantize_nvfp4_rowscaled_colwise(
                        static_cast<const uint16_t*>(x), rows_cap, cols, (int)G, offsets,
                        padded_offsets, col_rows_cap, data, block_scales, outer, dev_status,
                        (hipStream_t)stream),
                    fn);
}

static int gemm_mxfp8_impl(const char* fn, int mode, int64_t G, const uint8_t* a,
                           const uint8_t* a_scales, const uint8_t* b, const uint8_t* b_scales,
                           const int64_t* offsets, int64_t rows_cap, int64_t n, int64_t k,
                           void* out, int out_dtype, const float* alpha, const float* beta,
                           const float* bias, uint32_t* dev_status, void* stream,
                           void* ws = nullptr) {
  if (a == nullptr || a_scales == nullptr || b == nullptr || b_scales == nullptr || offsets == nullptr ||
      out == nullptr)
    return fail(BSG_ERR_NULL, "%s: operands, scales, offsets and out must be non-NULL", fn);
  if (mode != BSG_FPROP_TN && mode != BSG_WGRAD_NT && mode != BSG_DGRAD_NN &&
      mode != BSG_WGRAD_NT_E5M2)
    return fail(BSG_ERR_UNSUPPORTED, "%s: unknown mode %d", fn, mode);
  if (out_dtype != BSG_OUT_BF16 && out_dtype != BSG_OUT_F32)
    return fail(BSG_ERR_UNSUPPORTED, "%s: unknown out_dtype %d", fn, out_dtype);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || n < 1 || k < 1)
    return fail(BSG_ERR_SHAPE, "%s: need rows_cap >= 0, n >= 1, k >= 1", fn);
  const int64_t esz = out_dtype == BSG_OUT_F32 ? 4 : 2;
  const bool wgrad = mode == BSG_WGRAD_NT || mode == BSG_WGRAD_NT_E5M2;
  if (!wgrad) {
    if (k % 32 != 0)
      return fail(BSG_ERR_SHAPE, "%s: FPROP / DGRAD need k %% 32 == 0 (got %lld)", fn, (long long)k);
    const int64_t nq = (k + 127) / 128;  // scale words per row; DGRAD's B rows hold 128 nq bytes
    if (256 * 128 * nq >= kMaxTileBytes || 256 * n * esz >= kMaxTileBytes || n > 0x7fffffffLL)
      return fail(BSG_ERR_SHAPE, "%s: n or k too large for one tile's 32-bit offsets", fn);
    if (nq * 4 * rows_cap >= kMaxTileBytes || nq * 4 * G * n >= kMaxTileBytes)
      return fail(BSG_ERR_SHAPE, "%s: scale arrays too large for 32-bit offsets", fn);
  } else {
    if (n % 32 != 0 || k % 32 != 0)
      return fail(BSG_ERR_SHAPE, "%s: WGRAD needs n and k multiples of 32", fn);
    if (256 * rows_cap >= kMaxTileBytes || 256 * k * esz >= kMaxTileBytes ||
        (rows_cap / 128) * 4 * (n > k ? n : k) >= kMaxTileBytes)
      return fail(BSG_ERR_SHAPE, "%s: token capacity or k too large for 32-bit tile offsets", fn);
  }
  if (!aligned16(a) || !aligned16(b) || !aligned4(a_scales) || !aligned4(b_scales) || !aligned4(out))
    return fail(BSG_ERR_ALIGN, "%s: a and b must be 16-byte aligned; scales and out 4-byte", fn);
  if (!aligned4(alpha) || !aligned4(beta) || !aligned16(bias))
    return fail(BSG_ERR_ALIGN, "%s: alpha and beta must be 4-byte aligned, bias 16-byte", fn);
  if (bias != nullptr && ((wgrad ? k : n) % 4 != 0))
    return fail(BSG_ERR_SHAPE, "%s: a bias needs a multiple of 4 output columns", fn);
  return hip_result(bsg::launch_gemm_mxfp8(mode, (int)G, a, a_scales, b, b_scales, offsets, rows_cap,
                                           n, k, out, out_dtype == BSG_OUT_F32, dev_status,
                                           (hipStream_t)stream, alpha, beta, bias, ws),
                    fn);
}

int grouped_gemm_mxfp8(int mode, int64_t G, const uint8_t* a, const uint8_t* a_scales,
                       const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                       int64_t rows_cap, int64_t n, int64_t k, void* out, int out_dtype,
                       uint32_t* dev_status, void* stream) {
  return gemm_mxfp8_impl("grouped_gemm_mxfp8", mode, G, a, a_scales, b, b_scales, offsets,
                         rows_cap, n, k, out, out_dtype, nullptr, nullptr, nullptr, dev_status,
                         stream);
}

size_t grouped_gemm_mxfp8_workspace_size(void) { return bsg::gemm_mxfp8_workspace_bytes(); }

int grouped_gemm_mxfp8_ws(int mode, int64_t G, const uint8_t* a, const uint8_t* a_scales,
                          const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                          int64_t rows_cap, int64_t n, int64_t k, void* out, int out_dtype,
                          void* workspace, size_t workspace_bytes, uint32_t* dev_status,
                          void* stream) {
  const char* fn = "grouped_gemm_mxfp8_ws";
  if (workspace == nullptr) return fail(BSG_ERR_NULL, "%s: workspace is NULL", fn);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(BSG_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  const size_t need = bsg::gemm_mxfp8_workspace_bytes();
  if (workspace_bytes < need)
    return fail(BSG_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                need);
  return gemm_mxfp8_impl(fn, mode, G, a, a_scales, b, b_scales, offsets, rows_cap, n, k, out,
                         out_dtype, nullptr, nullptr, nullptr, dev_status, stream, workspace);
}

int grouped_gemm_mxfp8_ex(int mode, int64_t G, const uint8_t* a, const uint8_t* a_scales,
                          const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                          int64_t rows_cap, int64_t n, int64_t k, void* out, int out_dtype,
                          const float* alpha, const float* beta, const float* bias,
                          uint32_t* dev_status, void* stream) {
  return gemm_mxfp8_impl("grouped_gemm_mxfp8_ex", mode, G, a, a_scales, b, b_scales, offsets,
                         rows_cap, n, k, out, out_dtype, alpha, beta, bias, dev_status, stream);
}

static int gemm_nvfp4_impl(const char* fn, bool per_tensor, int64_t G, const uint8_t* a,
                           const uint8_t* a_scales, const float* a_outer, const int64_t* offsets,
                           int64_t rows_cap, int64_t k, const uint8_t* b, const uint8_t* b_scales,
                           const float* b_outer, const int64_t* n_per_group, void* out,
                           int64_t ld_out, int out_dtype, float* scratch, uint32_t* dev_status,
                           void* stream, bool noalloc = false, bool accumulate = false,
                           void* ws = nullptr) {
  if (a == nullptr || a_scales == nullptr || a_outer == nullptr || offsets == nullptr || b == nullptr ||
      b_scales == nullptr || b_outer == nullptr || n_per_group == nullptr || out == nullptr)
    return fail(BSG_ERR_NULL, "%s: operands, scales, offsets, n_per_group and out must be non-NULL", fn);
  if (out_dtype != BSG_OUT_BF16 && out_dtype != BSG_OUT_F32)
    return fail(BSG_ERR_UNSUPPORTED, "%s: unknown out_dtype %d", fn, out_dtype);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (rows_cap < 0 || k < 32 || k % 32 != 0)
    return fail(BSG_ERR_SHAPE, "%s: need rows_cap >= 0 and k a positive multiple of 32 (got %lld)", fn,
                (long long)k);
  bsg::NvGroupTable tab;
  memset(&tab, 0, sizeof tab);
  int64_t max_n = 0, brow = 0;
  for (int64_t g = 0; g < G; ++g) {
    const int64_t ng = n_per_group[g];
    if (ng < 0 || ng > 0x7fffffffLL) return fail(BSG_ERR_SHAPE, "%s: n_per_group[%lld] out of range", fn, (long long)g);
    tab.n[g] = (int32_t)ng;
    tab.brow[g] = (int32_t)brow;
    brow += ng;
    if (brow > 0x7fffffffLL) return fail(BSG_ERR_SHAPE, "%s: sum of n_per_group too large", fn);
    if (ng > max_n) max_n = ng;
  }
  tab.brow[G] = (int32_t)brow;
  if (ld_out < max_n || ld_out < 1)
    return fail(BSG_ERR_SHAPE, "%s: ld_out=%lld below the widest group (%lld)", fn, (long long)ld_out,
                (long long)max_n);
  if (noalloc && rows_cap * ld_out > (int64_t)(bsg::kNoAllocScratchBytes / sizeof(float)))
    return fail(BSG_ERR_SHAPE,
                "%s: rows_cap * ld_out * 4 = %lld bytes exceeds the library's %lld-byte static "
                "scratch; use grouped_gemm_nvfp4_rowscaled with a caller scratch",
                fn, (long long)(rows_cap * ld_out * 4), (long long)bsg::kNoAllocScratchBytes);
  const int64_t esz = (out_dtype == BSG_OUT_F32 || scratch != nullptr || noalloc) ? 4 : 2;
  if (256 * (k / 2) >= kMaxTileBytes || 256 * ld_out * esz >= kMaxTileBytes)
    return fail(BSG_ERR_SHAPE, "%s: k or ld_out too large for 32-bit tile offsets", fn);
  if (!aligned16(a) || !aligned16(b) || !aligned4(a_scales) || !aligned4(b_scales) || !aligned4(out) ||
      (scratch != nullptr && !aligned4(scratch)))
    return fail(BSG_ERR_ALIGN, "%s: a and b must be 16-byte aligned; scales, out and scratch 4-byte", fn);
  if (noalloc)
    return hip_result(bsg::launch_gemm_nvfp4_noalloc((int)G, a, a_scales, a_outer, offsets,
                                                     rows_cap, k, b, b_scales, b_outer, tab,
                                                     (int)max_n, out, ld_out,
                                                     out_dtype == BSG_OUT_F32, dev_status,
                                                     (hipStream_t)stream),
                      fn);
  return hip_result(bsg::launch_gemm_nvfp4((int)G, a, a_scales, a_outer, offsets, rows_cap, k, b,
                                           b_scales, b_outer, tab, (int)max_n, out, ld_out,
                                           out_dtype == BSG_OUT_F32, scratch, dev_status,
                                           (hipStream_t)stream, per_tensor, accumulate, ws),
                    fn);
}

// Checks a split workspace argument; 0 when usable.
static int check_nvfp4_workspace(const char* fn, void* workspace, size_t workspace_bytes) {
  if (workspace == nullptr) return fail(BSG_ERR_NULL, "%s: workspace is NULL", fn);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(BSG_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  const size_t need = bsg::gemm_nvfp4_workspace_bytes();
  if (workspace_bytes < need)
    return fail(BSG_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace_bytes,
                need);
  return BSG_OK;
}

size_t grouped_gemm_nvfp4_workspace_size(void) { return bsg::gemm_nvfp4_workspace_bytes(); }

int grouped_gemm_nvfp4_rowscaled_ws(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                    const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                                    int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                    const float* b_outer, const int64_t* n_per_group, void* out,
                                    int64_t ld_out, int out_dtype, int accumulate, void* workspace,
                                    size_t workspace_bytes, uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_gemm_nvfp4_rowscaled_ws";
  if (accumulate != 0 && accumulate != 1)
    return fail(BSG_ERR_UNSUPPORTED, "%s: accumulate must be 0 or 1", fn);
  const int wc = check_nvfp4_workspace(fn, workspace, workspace_bytes);
  if (wc != BSG_OK) return wc;
  return gemm_nvfp4_impl(fn, false, G, a, a_scales, a_outer, offsets, rows_cap, k, b, b_scales,
                         b_outer, n_per_group, out, ld_out, out_dtype, nullptr, dev_status, stream,
                         false, accumulate == 1, workspace);
}

int grouped_gemm_nvfp4_pertensor_ws(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                    const float* a_amax, const int64_t* offsets, int64_t rows_cap,
                                    int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                    const float* b_amax, const int64_t* n_per_group, void* out,
                                    int64_t ld_out, int out_dtype, void* workspace,
                                    size_t workspace_bytes, uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_gemm_nvfp4_pertensor_ws";
  const int wc = check_nvfp4_workspace(fn, workspace, workspace_bytes);
  if (wc != BSG_OK) return wc;
  return gemm_nvfp4_impl(fn, true, G, a, a_scales, a_amax, offsets, rows_cap, k, b, b_scales,
                         b_amax, n_per_group, out, ld_out, out_dtype, nullptr, dev_status, stream,
                         false, false, workspace);
}

int grouped_gemm_nvfp4_rowscaled(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                 const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                                 int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                 const float* b_outer, const int64_t* n_per_group, void* out,
                                 int64_t ld_out, int out_dtype, float* scratch,
                                 uint32_t* dev_status, void* stream) {
  return gemm_nvfp4_impl("grouped_gemm_nvfp4_rowscaled", false, G, a, a_scales, a_outer, offsets,
                         rows_cap, k, b, b_scales, b_outer, n_per_group, out, ld_out, out_dtype,
                         scratch, dev_status, stream);
}

int grouped_gemm_nvfp4_rowscaled_ex(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                    const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                                    int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                    const float* b_outer, const int64_t* n_per_group, void* out,
                                    int64_t ld_out, int out_dtype, float* scratch, int accumulate,
                                    uint32_t* dev_status, void* stream) {
  if (accumulate != 0 && accumulate != 1)
    return fail(BSG_ERR_UNSUPPORTED, "grouped_gemm_nvfp4_rowscaled_ex: accumulate must be 0 or 1");
  return gemm_nvfp4_impl("grouped_gemm_nvfp4_rowscaled_ex", false, G, a, a_scales, a_outer, offsets,
                         rows_cap, k, b, b_scales, b_outer, n_per_group, out, ld_out, out_dtype,
                         scratch, dev_status, stream, false, accumulate == 1);
}

int grouped_gemm_nvfp4_rowscaled_noalloc(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                         const float* a_outer, const int64_t* offsets,
                                         int64_t rows_cap, int64_t k, const uint8_t* b,
                                         const uint8_t* b_scales, const float* b_outer,
                                         const int64_t* n_per_group, void* out, int64_t ld_out,
                                         int out_dtype, uint32_t* dev_status, void* stream) {
  return gemm_nvfp4_impl("grouped_gemm_nvfp4_rowscaled_noalloc", false, G, a, a_scales, a_outer,
                         offsets, rows_cap, k, b, b_scales, b_outer, n_per_group, out, ld_out,
                         out_dtype, nullptr, dev_status, stream, true);
}

int grouped_gemm_nvfp4_pertensor(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                 const float* a_amax, const int64_t* offsets, int64_t rows_cap,
                                 int64_t k, const uint8_t* b, const uint8_t* b_scales,
                                 const float* b_amax, const int64_t* n_per_group, void* out,
                                 int64_t ld_out, int out_dtype, uint32_t* dev_status, void* stream) {
  return gemm_nvfp4_impl("grouped_gemm_nvfp4_pertensor", true, G, a, a_scales, a_amax, offsets,
                         rows_cap, k, b, b_scales, b_amax, n_per_group, out, ld_out, out_dtype,
                         nullptr, dev_status, stream);
}

static int nv_wgrad_impl(const char* fn, int64_t G, const uint8_t* a, const uint8_t* a_scales,
                         const float* a_outer, const uint8_t* b, const uint8_t* b_scales,
                         const float* b_outer, const int64_t* padded_offsets, int64_t col_rows_cap,
                         int64_t n, int64_t k, void* out, int out_dtype, bool accumulate,
                         uint32_t* dev_status, void* stream) {
  if (a == nullptr || a_scales == nullptr || a_outer == nullptr || b == nullptr ||
      b_scales == nullptr || b_outer == nullptr || padded_offsets == nullptr || out == nullptr)
    return fail(BSG_ERR_NULL, "%s: operands, scales, padded_offsets and out must be non-NULL", fn);
  if (out_dtype != BSG_OUT_BF16 && out_dtype != BSG_OUT_F32)
    return fail(BSG_ERR_UNSUPPORTED, "%s: unknown out_dtype %d", fn, out_dtype);
  if (G < 1 || G > BSG_MAX_GROUPS)
    return fail(BSG_ERR_SHAPE, "%s: G=%lld outside [1, %d]", fn, (long long)G, BSG_MAX_GROUPS);
  if (col_rows_cap < 0 || n < 32 || k < 32 || n % 32 != 0 || k % 32 != 0)
    return fail(BSG_ERR_SHAPE, "%s: need col_rows_cap >= 0 and n, k positive multiples of 32", fn);
  const int64_t esz = out_dtype == BSG_OUT_F32 ? 4 : 2;
  if (256 * (col_rows_cap / 2) >= kMaxTileBytes || 256 * k * esz >= kMaxTileBytes ||
      n > 0x7fffffffLL || k > 0x7fffffffLL)
    return fail(BSG_ERR_SHAPE, "%s: col_rows_cap, n or k too large for 32-bit tile offsets", fn);
  if (!aligned16(a) || !aligned16(b) || !aligned4(a_scales) || !aligned4(b_scales) ||
      !aligned4(a_outer) || !aligned4(b_outer) || !aligned4(out))
    return fail(BSG_ERR_ALIGN, "%s: a and b must be 16-byte aligned; scales, outer and out 4-byte",
                fn);
  return hip_result(bsg::launch_gemm_nvfp4_wgrad((int)G, a, a_scales, a_outer, b, b_scales,
                                                 b_outer, padded_offsets, col_rows_cap, n, k, out,
                                                 out_dtype == BSG_OUT_F32, dev_status,
                                                 (hipStream_t)stream, accumulate),
                    fn);
}

int grouped_gemm_nvfp4_rowscaled_wgrad(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                       const float* a_outer, const uint8_t* b,
                                       const uint8_t* b_scales, const float* b_outer,
                                       const int64_t* padded_offsets, int64_t col_rows_cap,
                                       int64_t n, int64_t k, void* out, int out_dtype,
                                       uint32_t* dev_status, void* stream) {
  return nv_wgrad_impl("grouped_gemm_nvfp4_rowscaled_wgrad", G, a, a_scales, a_outer, b, b_scales,
                       b_outer, padded_offsets, col_rows_cap, n, k, out, out_dtype, false,
                       dev_status, stream);
}

int grouped_gemm_nvfp4_rowscaled_wgrad_ex(int64_t G, const uint8_t* a, const uint8_t* a_scales,
                                          const float* a_outer, const uint8_t* b,
                                          const uint8_t* b_scales, const float* b_outer,
                                          const int64_t* padded_offsets, int64_t col_rows_cap,
                                          int64_t n, int64_t k, void* out, int out_dtype,
                                          int accumulate, uint32_t* dev_status, void* stream) {
  const char* fn = "grouped_gemm_nvfp4_rowscaled_wgrad_ex";
  if (accumulate != 0 && accumulate != 1)
    return fail(BSG_ERR_UNSUPPORTED, "%s: accumulate must be 0 or 1", fn);
  return nv_wgrad_impl(fn, G, a, a_scales, a_outer, b, b_scales, b_outer, padded_offsets,
                       col_rows_cap, n, k, out, out_dtype, accumulate == 1, dev_status, stream);
}

}  // extern "C"
