// Row-scaled NVFP4 quantize: bf16 -> E2M1 elements, one E4M3 scale per 16
// elements, one FP32 outer scale per row, with the row amax fused into the cast.
//
// "[Common][PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM":
// row-scaled grouped NVFP4 cast with a per-row outer scale; the amax pass is
// fused into the same single launch.  Outer scale = amax / (6 * 448), the
// tensor-scale formula of "gemm.py" (_get_nvfp4_tensor_scale_inv) taken per
// row.  Float32 steps, each rounded to nearest (IEEE division):
//   S   = 2688 / amax_r   (1 if amax_r == 0, capped at FLT_MAX)
//   s8  = E4M3((bmax / 6) * S)        saturating, ties to even
//   enc = S / decode(s8)  (0 if the scale is 0, capped at FLT_MAX)
//   q   = E2M1(x * enc)               saturating at 6, ties to even
// The E4M3 convert is exact round-to-nearest-even below 464, so the scale is
// clamped to 448 first; the E2M1 convert (unit scale) rounds to nearest even
// and saturates by itself.
//
// One 256-thread block per live row, each thread holding up to four 16-element
// blocks in registers (cols <= 16384): the row is read from HBM once.
#include "bsg_internal.h"

#pragma clang fp contract(off)

namespace bsg {

constexpr int kNvThreads = 256;
constexpr int kNvMaxBlocksPerThread = 4;

namespace {

__device__ __forceinline__ float e4m3_decode_pos(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
}

__device__ __forceinline__ uint32_t mag_bits(uint32_t w) {
  return max(w & 0x7fffu, (w >> 16) & 0x7fffu);
}

// Four packed bf16 pairs (8 elements) times enc -> 8 E2M1 nibbles in one dword,
// element 2j in the low nibble of byte j.
__device__ __forceinline__ uint32_t fp4_pack8(uint4 v, float enc) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_to_f32(v.x & 0xffffu) * enc,
                                               __uint_as_float(v.x & 0xffff0000u) * enc, 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_to_f32(v.y & 0xffffu) * enc,
                                               __uint_as_float(v.y & 0xffff0000u) * enc, 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_to_f32(v.z & 0xffffu) * enc,
                                               __uint_as_float(v.z & 0xffff0000u) * enc, 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_to_f32(v.w & 0xffffu) * enc,
                                               __uint_as_float(v.w & 0xffff0000u) * enc, 1.0f, 3);
  return r;
}

}  // namespace

__global__ __launch_bounds__(kNvThreads) void nvfp4_rowscaled_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, uint8_t* __restrict__ data, uint8_t* __restrict__ bscales,
    float* __restrict__ outer, uint32_t* status) {
  __shared__ uint32_t s_wmax[kNvThreads / 64];
  int64_t live = offsets[G];
  if (live < 0) live = 0;
  if (live > rows_cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0) dev_status_or(status, kDevOverCapacity);
    live = rows_cap;
  }
  const int64_t row = blockIdx.x;
  if (row >= live) return;
  const int tid = threadIdx.x;
  const int64_t nblk = cols / 16;
  const uint16_t* xr = x + row * cols;

  uint4 v[kNvMaxBlocksPerThread][2];
  uint32_t bm[kNvMaxBlocksPerThread];
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < kNvMaxBlocksPerThread; ++i) {
    const int64_t j = tid + (int64_t)kNvThreads * i;
    bm[i] = 0;
    if (j < nblk) {
      v[i][0] = reinterpret_cast<const uint4*>(xr + 16 * j)[0];
      v[i][1] = reinterpret_cast<const uint4*>(xr + 16 * j)[1];
      bm[i] = max(max(max(mag_bits(v[i][0].x), mag_bits(v[i][0].y)),
                      max(mag_bits(v[i][0].z), mag_bits(v[i][0].w))),
                  max(max(mag_bits(v[i][1].x), mag_bits(v[i][1].y)),
                      max(mag_bits(v[i][1].z), mag_bits(v[i][1].w))));
      am = max(am, bm[i]);
    }
  }
  for (int d = 32; d >= 1; d >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, d, 64));
  if ((tid & 63) == 0) s_wmax[tid >> 6] = am;
  __syncthreads();
  am = max(max(s_wmax[0], s_wmax[1]), max(s_wmax[2], s_wmax[3]));

  const float amax = bf16_to_f32(am);
  float S = amax > 0.0f ? 2688.0f / amax : 1.0f;
  S = __builtin_fminf(S, 3.40282346638528859812e+38f);
  if (tid == 0) outer[row] = amax / 2688.0f;

#pragma unroll
  for (int i = 0; i < kNvMaxBlocksPerThread; ++i) {
    const int64_t j = tid + (int64_t)kNvThreads * i;
    if (j < nblk) {
      const float bmax = bf16_to_f32(bm[i]);
      float sf = (bmax / 6.0f) * S;
      sf = __builtin_fminf(sf, 448.0f);
      const uint32_t s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sf, 0.0f, 0, false) & 0xffu;
      const float sd = e4m3_decode_pos(s8);
      float enc = 0.0f;
      if (sd != 0.0f) enc = __builtin_fminf(S / sd, 3.40282346638528859812e+38f);
      const uint32_t lo = fp4_pack8(v[i][0], enc);
      const uint32_t hi = fp4_pack8(v[i][1], enc);
      *reinterpret_cast<uint2*>(data + row * (cols / 2) + 8 * j) = make_uint2(lo, hi);
      bscales[row * nblk + j] = (uint8_t)s8;
    }
  }
}

hipError_t launch_quantize_nvfp4_rowscaled(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                           int G, const int64_t* offsets, uint8_t* data,
                                           uint8_t* block_scales, float* outer, uint32_t* status,
                                           hipStream_t stream) {
  if (rows_cap == 0) return hipSuccess;
  hipLaunchKernelGGL(nvfp4_rowscaled_kernel, dim3((unsigned)rows_cap), dim3(kNvThreads), 0, stream,
                     x, rows_cap, cols, G, offsets, data, block_scales, outer, status);
  return hipGetLastError();
}

}  // namespace bsg
