// Internal declarations of libbsg: device helpers shared by the kernels and the
// launchers called from the C-ABI layer (api.cpp).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsg {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kMaxGroups = 256;
constexpr int kColPad = 128;

constexpr uint32_t kDevNegativeSize = 1u;
constexpr uint32_t kDevOverCapacity = 2u;
constexpr uint32_t kDevBadPadding = 4u;

// ---------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// float32 -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// 16-byte load of an input that is read once (the quantizers' bf16 inputs):
// non-temporal, so the stream does not displace cached lines on its way.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const v4i q = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
  return make_uint4((uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2], (uint32_t)q[3]);
}

__device__ __forceinline__ void dev_status_or(uint32_t* st, uint32_t bits) {
  if (st != nullptr && bits != 0u) atomicOr(st, bits);
}

// Loads offsets[0..G] into LDS, each clamped into [0, cap], so every later
// index stays inside the caller's buffers whatever the device holds.  A group's
// extent is then max(0, s_off[g+1] - s_off[g]).  Flags kDevNegativeSize for a
// negative or decreasing offset and kDevOverCapacity for a value above cap.
// Every thread of the block must call it; it ends with a barrier.
__device__ __forceinline__ void load_offsets_clamped(const int64_t* __restrict__ off, int G,
                                                     int64_t cap, int64_t* s_off,
                                                     uint32_t* status) {
  for (int g = threadIdx.x; g <= G; g += blockDim.x) {
    int64_t v = off[g];
    uint32_t bad = 0;
    if (v < 0) { v = 0; bad |= kDevNegativeSize; }
    if (v > cap) { v = cap; bad |= kDevOverCapacity; }
    s_off[g] = v;
    dev_status_or(status, bad);
  }
  __syncthreads();
  for (int g = threadIdx.x + 1; g <= G; g += blockDim.x)
    if (s_off[g] < s_off[g - 1]) dev_status_or(status, kDevNegativeSize);
}

__device__ __forceinline__ int64_t group_extent(const int64_t* s_off, int g) {
  int64_t d = s_off[g + 1] - s_off[g];
  return d > 0 ? d : 0;
}

// Exclusive prefix sum of s_cnt[0..G-1] into s_pre[0..G] (s_pre[G] = total),
// computed by the first wavefront of the block (G <= kMaxGroups).  The caller
// places a barrier after it.
__device__ __forceinline__ void wave0_exclusive_scan(const int32_t* s_cnt, int G, int32_t* s_pre) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (G + 63) / 64;  // at most 4
    const int base = lane * per;
    int local[4] = {0, 0, 0, 0};
    int sum = 0;
    for (int i = 0; i < per; ++i) {
      int g = base + i;
      int c = g < G ? s_cnt[g] : 0;
      local[i] = c;
      sum += c;
    }
    int incl = sum;
    for (int d = 1; d < 64; d <<= 1) {
      int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    int run = incl - sum;
    for (int i = 0; i < per; ++i) {
      int g = base + i;
      if (g < G) s_pre[g] = run;
      run += local[i];
    }
    if (lane == 63) s_pre[G] = incl;
  }
}

// Index of the group owning item `t` given exclusive prefix s_pre[0..G]:
// the largest g in [0, G-1] with s_pre[g] <= t (empty groups are skipped).
__device__ __forceinline__ int find_group(const int32_t* s_pre, int G, int t) {
  int lo = 0, hi = G - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_pre[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Workgroup b of a launch runs on XCD b % kXcds, and each XCD has its own L2.
constexpr int kXcds = 8;

// Position of workgroup b in the tile order: with a grid that is a multiple of
// kXcds, the workgroups of one XCD take consecutive tiles of each round of
// gridDim.x tiles, so tiles that share operand rows share that XCD's L2.
__device__ __forceinline__ int xcd_slot() {
  const int nxcd = gridDim.x % kXcds == 0 ? kXcds : 1;
  return (blockIdx.x % nxcd) * (gridDim.x / nxcd) + blockIdx.x / nxcd;
}

// Position (mt, nt) of local tile u of a group with mtiles x ntiles tiles,
// enumerated in blocks of SM x SN tiles (row of blocks by row of blocks, m
// fastest inside a block); only the last block row / column can be partial,
// so the block of u follows from two divisions.
template <int SM, int SN>
__device__ __forceinline__ void super_tile(int u, int mtiles, int ntiles, int& mt, int& nt) {
  const int full_rows = mtiles / SM;
  int br, hgt, u2;
  if (u < full_rows * SM * ntiles) {
    br = u / (SM * ntiles);
    hgt = SM;
    u2 = u - br * SM * ntiles;
  } else {
    br = full_rows;
    hgt = mtiles - full_rows * SM;
    u2 = u - full_rows * SM * ntiles;
  }
  const int bc = u2 / (SN * hgt);
  const int u3 = u2 - bc * SN * hgt;
  mt = br * SM + u3 % hgt;
  nt = bc * SN + u3 / hgt;
}

// ---------------------------------------------------------------- launchers

struct NvGroupTable {
  int32_t n[kMaxGroups];        // output width of each group
  int32_t brow[kMaxGroups + 1]; // first weight row of each group (prefix sum of n)
};

hipError_t launch_group_offsets(const int32_t* sizes, int G, int64_t multiplier, int64_t pad_to,
                                int64_t* sizes_i64, int64_t* offsets, int64_t capacity,
                                uint32_t* status, hipStream_t stream);

hipError_t launch_quantize_mxfp8_rowwise(const uint16_t* x, int64_t rows_cap, int64_t cols, int G,
                                         const int64_t* offsets, uint8_t* data, uint8_t* scales,
                                         uint32_t* status, hipStream_t stream, bool e5m2 = false);

// Columnwise (and, if row_data != nullptr, the rowwise output in the same pass);
// e5m2: E5M2 elements, columnwise only.
hipError_t launch_quantize_mxfp8_colwise(const uint16_t* x, int64_t rows_cap, int64_t cols, int G,
                                         const int64_t* offsets, const int64_t* padded_offsets,
                                         int64_t col_rows_cap, uint8_t* col_data,
                                         uint8_t* col_scales, uint8_t* row_data,
                                         uint8_t* row_scales, uint32_t* status,
                                         hipStream_t stream, bool e5m2 = false);

hipError_t launch_quantize_nvfp4_rowscaled(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                           int G, const int64_t* offsets, uint8_t* data,
                                           uint8_t* block_scales, float* outer, uint32_t* status,
                                           hipStream_t stream);

hipError_t launch_quantize_nvfp4_pertensor(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                           int G, const int64_t* offsets, uint8_t* data,
                                           uint8_t* block_scales, float* amax, uint32_t* status,
                                           hipStream_t stream);

hipError_t launch_quantize_nvfp4_pertensor_rht(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                               int G, const int64_t* offsets, uint32_t sign_mask,
                                               uint8_t* data, uint8_t* block_scales, float* amax,
                                               uint32_t* status, hipStream_t stream);

hipError_t launch_quantize_nvfp4_pertensor_2d(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                              int G, const int64_t* offsets, uint8_t* data,
                                              uint8_t* block_scales, float* amax, uint32_t* status,
                                              hipStream_t stream);

hipError_t launch_quantize_nvfp4_rowscaled_colwise(const uint16_t* x, int64_t rows_cap,
                                                   int64_t cols, int G, const int64_t* offsets,
                                                   const int64_t* padded_offsets,
                                                   int64_t col_rows_cap, uint8_t* data,
                                                   uint8_t* block_scales, float* outer,
                                                   uint32_t* status, hipStream_t stream);

hipError_t launch_gemm_mxfp8(int mode, int G, const uint8_t* a, const uint8_t* a_scales,
                             const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                             int64_t rows_cap, int64_t n, int64_t k, void* out, int out_f32,
                             uint32_t* status, hipStream_t stream,
                             const float* alpha = nullptr, const float* beta = nullptr,
                             const float* bias = nullptr, void* ws = nullptr);

// Bytes of the workspace that lets launch_gemm_mxfp8 split its last round of
// tiles along the contraction (on the current device).
size_t gemm_mxfp8_workspace_bytes();

hipError_t launch_gemm_nvfp4(int G, const uint8_t* a, const uint8_t* a_scales,
                             const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                             int64_t k, const uint8_t* b, const uint8_t* b_scales,
                             const float* b_outer, const NvGroupTable& table, int max_n,
                             void* out, int64_t ld_out, int out_f32, float* s_buf,
                             uint32_t* status, hipStream_t stream, bool per_tensor = false,
                             bool accumulate = false, void* ws = nullptr);

// Bytes of the workspace that lets launch_gemm_nvfp4 split its last round of
// tiles along the contraction (on the current device).
size_t gemm_nvfp4_workspace_bytes();

// The FP32 S of grouped_gemm_nvfp4_rowscaled_noalloc lives in a static device
// array of this many bytes (per GPU).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;

hipError_t noalloc_scratch_ptr(float** ptr);

hipError_t launch_gemm_nvfp4_noalloc(int G, const uint8_t* a, const uint8_t* a_scales,
                                     const float* a_outer, const int64_t* offsets,
                                     int64_t rows_cap, int64_t k, const uint8_t* b,
                                     const uint8_t* b_scales, const float* b_outer,
                                     const NvGroupTable& table, int max_n, void* out,
                                     int64_t ld_out, int out_f32, uint32_t* status,
                                     hipStream_t stream);

hipError_t launch_gemm_nvfp4_wgrad(int G, const uint8_t* a, const uint8_t* a_scales,
                                   const float* a_outer, const uint8_t* b, const uint8_t* b_scales,
                                   const float* b_outer, const int64_t* padded_offsets,
                                   int64_t col_rows_cap, int64_t n, int64_t k, void* out,
                                   int out_f32, uint32_t* status, hipStream_t stream,
                                   bool accumulate = false);

int device_cu_count();

}  // namespace bsg
