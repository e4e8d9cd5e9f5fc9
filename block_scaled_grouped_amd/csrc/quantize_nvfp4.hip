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
// blocks in registers: a row of up to 16384 elements is read from HBM once;
// longer rows read their remaining blocks a second time, from the L2.
//
// The file also holds the per-tensor form (one outer scale per group from the
// group's amax: a group-amax pass, then the same cast), its randomized-Hadamard
// and 2-D (16 x 16 block scale) variants, and the columnwise (transposed,
// per-expert) form for the weight gradient; each is described where it starts
// below.
#include "bsg_internal.h"

#pragma clang fp contract(off)

namespace bsg {

constexpr int kNvThreads = 256;
constexpr int kNvMaxBlocksPerThread = 4;
static_assert(kMaxGroups <= kNvThreads, "the per-tensor cast gives each group one thread");

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

// Largest bf16 magnitude bits of a 16-element block (two 16-byte halves).
__device__ __forceinline__ uint32_t block_mag(const uint4& a, const uint4& b) {
  return max(max(max(mag_bits(a.x), mag_bits(a.y)), max(mag_bits(a.z), mag_bits(a.w))),
             max(max(mag_bits(b.x), mag_bits(b.y)), max(mag_bits(b.z), mag_bits(b.w))));
}

// Block j of a row: the E4M3 scale from its largest magnitude bits and the
// row's (or group's) S, then the 16 E2M1 codes, stored.
__device__ __forceinline__ void nv_cast_block(const uint4& a, const uint4& b, uint32_t bm, float S,
                                              uint8_t* __restrict__ drow,
                                              uint8_t* __restrict__ srow, int64_t j) {
  const float bmax = bf16_to_f32(bm);
  float sf = (bmax / 6.0f) * S;
  sf = __builtin_fminf(sf, 448.0f);
  const uint32_t s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sf, 0.0f, 0, false) & 0xffu;
  const float sd = e4m3_decode_pos(s8);
  float enc = 0.0f;
  if (sd != 0.0f) enc = __builtin_fminf(S / sd, 3.40282346638528859812e+38f);
  *reinterpret_cast<uint2*>(drow + 8 * j) = make_uint2(fp4_pack8(a, enc), fp4_pack8(b, enc));
  srow[j] = (uint8_t)s8;
}

// PER_TENSOR: the row's outer scale comes from its group's amax (computed by
// nvfp4_group_amax_kernel into group_amax), no per-row outer scale is written,
// and a row that no group owns (before offsets[0]) is left untouched;
// otherwise the row's own amax is reduced here and amax / 2688 stored.
// LONG: rows of more than kNvMaxBlocksPerThread blocks per thread; the blocks
// past the first kNvMaxBlocksPerThread * 256 are read again for the cast (the
// row, at least 64 KiB, is still in the L2 then).
template <bool PER_TENSOR, bool LONG>
__global__ __launch_bounds__(kNvThreads) void nvfp4_rowscaled_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, uint8_t* __restrict__ data, uint8_t* __restrict__ bscales,
    float* __restrict__ outer, const float* __restrict__ group_amax, uint32_t* status) {
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
  uint8_t* drow = data + row * (cols / 2);
  uint8_t* srow = bscales + row * nblk;
  constexpr int64_t kRegBlocks = (int64_t)kNvMaxBlocksPerThread * kNvThreads;

  uint4 v[kNvMaxBlocksPerThread][2];
  uint32_t bm[kNvMaxBlocksPerThread];
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < kNvMaxBlocksPerThread; ++i) {
    const int64_t j = tid + (int64_t)kNvThreads * i;
    bm[i] = 0;
    if (j < nblk) {
      if constexpr (PER_TENSOR) {  // the second read of the rows: do not re-allocate them
        v[i][0] = load_stream16(xr + 16 * j);
        v[i][1] = load_stream16(xr + 16 * j + 8);
      } else {
        v[i][0] = reinterpret_cast<const uint4*>(xr + 16 * j)[0];
        v[i][1] = reinterpret_cast<const uint4*>(xr + 16 * j)[1];
      }
      bm[i] = block_mag(v[i][0], v[i][1]);
      am = max(am, bm[i]);
    }
  }
  if constexpr (LONG && !PER_TENSOR) {
    for (int64_t j = kRegBlocks + tid; j < nblk; j += kNvThreads) {
      const uint4* p = reinterpret_cast<const uint4*>(xr + 16 * j);
      am = max(am, block_mag(p[0], p[1]));
    }
  }
  float amax;
  if constexpr (PER_TENSOR) {
    // the row's group amax in one round trip: thread t (G <= 256) loads group
    // t's offsets and amax together and publishes the amax if the row is
    // group t's; word 1 says whether any group owns the row
    bool mine = false;
    uint32_t val = 0u;
    if (tid < G) {
      const int64_t lo = offsets[tid], hi = offsets[tid + 1];
      val = __float_as_uint(group_amax[tid]);
      mine = lo <= row && row < hi;
    }
    if (tid == 0) {
      s_wmax[0] = 0u;
      s_wmax[1] = 0u;
    }
    __syncthreads();
    if (mine) {
      s_wmax[0] = val;
      s_wmax[1] = 1u;
    }
    __syncthreads();
    if (s_wmax[1] == 0u) return;  // uniform: no group owns this row
    amax = __uint_as_float(s_wmax[0]);
  } else {
    for (int d = 32; d >= 1; d >>= 1) am = max(am, (uint32_t)__shfl_xor((int)am, d, 64));
    if ((tid & 63) == 0) s_wmax[tid >> 6] = am;
    __syncthreads();
    am = max(max(s_wmax[0], s_wmax[1]), max(s_wmax[2], s_wmax[3]));
    amax = bf16_to_f32(am);
  }
  float S = amax > 0.0f ? 2688.0f / amax : 1.0f;
  S = __builtin_fminf(S, 3.40282346638528859812e+38f);
  if (!PER_TENSOR && tid == 0) outer[row] = amax / 2688.0f;

#pragma unroll
  for (int i = 0; i < kNvMaxBlocksPerThread; ++i) {
    const int64_t j = tid + (int64_t)kNvThreads * i;
    if (j < nblk) nv_cast_block(v[i][0], v[i][1], bm[i], S, drow, srow, j);
  }
  if constexpr (LONG) {
    for (int64_t j = kRegBlocks + tid; j < nblk; j += kNvThreads) {
      const uint4* p = reinterpret_cast<const uint4*>(xr + 16 * j);
      const uint4 a = p[0], b = p[1];
      nv_cast_block(a, b, block_mag(a, b), S, drow, srow, j);
    }
  }
}

// Rows with more blocks than a thread keeps in registers take the LONG form.
__host__ __forceinline__ bool nv_long_rows(int64_t cols) {
  return cols / 16 > (int64_t)kNvMaxBlocksPerThread * kNvThreads;
}

hipError_t launch_quantize_nvfp4_rowscaled(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                           int G, const int64_t* offsets, uint8_t* data,
                                           uint8_t* block_scales, float* outer, uint32_t* status,
                                           hipStream_t stream) {
  if (rows_cap == 0) return hipSuccess;
  if (nv_long_rows(cols))
    hipLaunchKernelGGL((nvfp4_rowscaled_kernel<false, true>), dim3((unsigned)rows_cap),
                       dim3(kNvThreads), 0, stream, x, rows_cap, cols, G, offsets, data,
                       block_scales, outer, nullptr, status);
  else
    hipLaunchKernelGGL((nvfp4_rowscaled_kernel<false, false>), dim3((unsigned)rows_cap),
                       dim3(kNvThreads), 0, stream, x, rows_cap, cols, G, offsets, data,
                       block_scales, outer, nullptr, status);
  return hipGetLastError();
}

// A 64-bit value as the first lane holds it (for values the same in every
// lane, so the compiler can keep them in scalar registers).
__device__ __forceinline__ int64_t first_lane64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// ---------------------------------------------------------------- per tensor
//
// Per-tensor NVFP4 of grouped rows: each group (an expert's rows, or an
// expert's weight) is one tensor whose outer scale is amax_g / 2688 ("gemm.py",
// _get_nvfp4_tensor_scale_inv; the GEMM's alpha is the product of the two
// operands' outer scales).  The group amax must be complete before any of the
// group's blocks is encoded, so it is its own pass: a small kernel clears the
// G amax words, nvfp4_group_amax_kernel reduces the live rows to one maximum
// per group (16-byte loads, integer max of the bf16 magnitudes, per-group
// maxima in LDS, then one atomic max per group and workgroup: atomics on one
// address from every XCD serialize, so their count is kept to a few hundred;
// non-negative floats order as their bit patterns), then the cast above runs
// with the group's amax, reading the rows a second time.
constexpr int kAmaxThreads = 512;
constexpr int kAmaxBlocksPerCu = 2;
constexpr int kAmaxBatch = 8;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(256) void nvfp4_amax_clear_kernel(uint32_t* __restrict__ amax_bits,
                                                               int G) {
  for (int g = threadIdx.x; g < G; g += blockDim.x) amax_bits[g] = 0u;
}

// The live rows are one contiguous run of 16-byte chunks; workgroup b takes the
// b-th contiguous share of it, thread t every 512th chunk from t.  A thread
// keeps the running max of its current group and folds it into the
// workgroup's per-group maxima in LDS when its chunks cross into the next
// group; at the end the workgroup issues one global atomic max per group it
// saw, so a group receives one atomic from each workgroup that touches it.
__global__ __launch_bounds__(kAmaxThreads) void nvfp4_group_amax_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, uint32_t* __restrict__ amax_bits, uint32_t* status) {
  __shared__ int64_t s_off[kMaxGroups + 1];
  __shared__ uint32_t s_max[kMaxGroups];
  const int tid = threadIdx.x;
  for (int g = tid; g < G; g += kAmaxThreads) s_max[g] = 0u;
  load_offsets_clamped(offsets, G, rows_cap, s_off, blockIdx.x == 0 ? status : nullptr);
  const int64_t cpr = cols / 8;  // 16-byte chunks per row
  // the groups' rows: [offsets[0], offsets[G]) (rows before offsets[0] belong to no group)
  const int64_t first = s_off[0] * cpr, total = s_off[G] * cpr;
  const int64_t span = total > first ? total - first : 0;
  const int64_t per = (span + gridDim.x - 1) / gridDim.x;
  const int64_t c0 = first + (int64_t)blockIdx.x * per;
  const int64_t c1 = c0 + per < total ? c0 + per : total;
  // every thread runs the same number of batches (chunks past the share read
  // zeros), so the loop and its waits are uniform
  {
    int64_t c = c0 + tid;
    const int64_t row = c / cpr;
    int g = 0, hi = G - 1;  // the largest g with s_off[g] <= row
    while (g < hi) {
      const int mid = (g + hi + 1) >> 1;
      if (s_off[mid] <= row) g = mid; else hi = mid - 1;
    }
    int64_t bound = s_off[g + 1] * cpr;  // first chunk past group g
    // the workgroup's share as one buffer range: loads past it read zeros, so
    // every load is issued unconditionally and the wait for a batch counts
    // only the loads issued before it
    const uint64_t xb = reinterpret_cast<uint64_t>(x + c0 * 8);
    const uint32_t xlo = __builtin_amdgcn_readfirstlane((uint32_t)xb);
    const uint32_t xhi = __builtin_amdgcn_readfirstlane((uint32_t)(xb >> 32));
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(((uint64_t)xhi << 32) | xlo), (short)0,
        __builtin_amdgcn_readfirstlane((int)(c1 > c0 ? (c1 - c0) * 16 : 0)), 0x00020000);
    uint32_t m = 0;
    constexpr int64_t kStep = (int64_t)kAmaxBatch * kAmaxThreads;
    // two batches in flight: the next batch's loads are issued before the
    // current one is folded
    auto load = [&](uint4 (&v)[kAmaxBatch], int64_t cb) {
#pragma unroll
      for (int k = 0; k < kAmaxBatch; ++k) {
        const int64_t ck = cb + (int64_t)k * kAmaxThreads;
        const v4i q = __builtin_amdgcn_raw_buffer_load_b128(
            rx, ck < c1 ? (int)((ck - c0) * 16) : 0x7ffffff0, 0, 0);
        v[k] = make_uint4((uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2], (uint32_t)q[3]);
      }
    };
    auto fold = [&](const uint4 (&v)[kAmaxBatch], int64_t cb) {
#pragma unroll
      for (int k = 0; k < kAmaxBatch; ++k) {
        // chunks past the share read zeros, which leave every maximum as it is
        const int64_t ck = cb + (int64_t)k * kAmaxThreads;
        if (ck >= bound) {
          atomicMax(&s_max[g], m);
          m = 0;
          while (g < G - 1 && s_off[g + 1] * cpr <= ck) ++g;
          bound = s_off[g + 1] * cpr;
        }
        m = max(m, max(max(mag_bits(v[k].x), mag_bits(v[k].y)),
                       max(mag_bits(v[k].z), mag_bits(v[k].w))));
      }
    };
    const int64_t nb = first_lane64(c1 > c0 ? (c1 - c0 + kStep - 1) / kStep : 0);
    uint4 va[kAmaxBatch], vb[kAmaxBatch];
    if (nb > 0) load(va, c);
    for (int64_t b = 0; b < nb; b += 2, c += 2 * kStep) {
      load(vb, c + kStep);
      fold(va, c);
      if (b + 1 >= nb) break;
      load(va, c + 2 * kStep);
      fold(vb, c + kStep);
    }
    atomicMax(&s_max[g], m);
  }
  __syncthreads();
  for (int g = tid; g < G; g += kAmaxThreads)
    if (s_max[g] != 0u) atomicMax(&amax_bits[g], s_max[g] << 16);
}

hipError_t launch_quantize_nvfp4_pertensor(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                           int G, const int64_t* offsets, uint8_t* data,
                                           uint8_t* block_scales, float* amax, uint32_t* status,
                                           hipStream_t stream) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
  hipLaunchKernelGGL(nvfp4_amax_clear_kernel, dim3(1), dim3(256), 0, stream, bits, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows_cap == 0) return e;
  const int64_t chunks = rows_cap * (cols / 8);
  int64_t blocks = (chunks + kAmaxBatch * kAmaxThreads - 1) / (kAmaxBatch * kAmaxThreads);
  const int64_t most = (int64_t)device_cu_count() * kAmaxBlocksPerCu;
  if (blocks > most) blocks = most;
  hipLaunchKernelGGL(nvfp4_group_amax_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream,
                     x, rows_cap, cols, G, offsets, bits, status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nv_long_rows(cols))
    hipLaunchKernelGGL((nvfp4_rowscaled_kernel<true, true>), dim3((unsigned)rows_cap),
                       dim3(kNvThreads), 0, stream, x, rows_cap, cols, G, offsets, data,
                       block_scales, nullptr, amax, nullptr);
  else
    hipLaunchKernelGGL((nvfp4_rowscaled_kernel<true, false>), dim3((unsigned)rows_cap),
                       dim3(kNvThreads), 0, stream, x, rows_cap, cols, G, offsets, data,
                       block_scales, nullptr, amax, nullptr);
  return hipGetLastError();
}

// ---------------------------------------------------------------- per tensor, RHT
//
// Per-tensor NVFP4 of the randomized Hadamard transform of the rows ("gemm.py",
// _quantize_gemm_operands: with NVFP4 1-D scaling both GEMM operands carry the
// RHT, so that it cancels in the product).  Each 16-element block x along the
// contraction becomes y = (1/4) H16 diag(s) x, H16 the Sylvester Hadamard
// matrix and s the caller's 16 signs (bit i of the mask set: s_i = -1), in
// float32: the sign flips, a four-stage butterfly (stage d = 1, 2, 4, 8 replaces
// (y[i], y[i + d]) by (y[i] + y[i + d], y[i] - y[i + d]) for the i with bit d
// clear), then the exact product by 1/4.  The group amax is taken over the
// transformed values (their float32 magnitude bits, an order-preserving key for
// non-negative floats), and the cast quantizes the transformed values with the
// per-tensor float32 steps.  Both passes transform each block in registers from
// its 32 bytes; nothing transformed is written back.

namespace {

__device__ __forceinline__ void rht16(const uint4& a, const uint4& b, uint32_t mask,
                                      float (&y)[16]) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    y[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    y[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i)  // sign flip: exact
    y[i] = __uint_as_float(__float_as_uint(y[i]) ^ (((mask >> i) & 1u) << 31));
#pragma unroll
  for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & d) == 0) {
        const float u = y[i], v = y[i + d];
        y[i] = u + v;
        y[i + d] = u - v;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] *= 0.25f;
}

// Largest magnitude of 16 floats, as the float32 bits of it.
__device__ __forceinline__ uint32_t fmag_bits(const float (&y)[16]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = max(m, __float_as_uint(y[i]) & 0x7fffffffu);
  return m;
}

// 8 floats times enc -> 8 E2M1 nibbles in one dword (element 2j low nibble of byte j).
__device__ __forceinline__ uint32_t fp4_pack8f(const float* y, float enc) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[0] * enc, y[1] * enc, 1.0f, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[2] * enc, y[3] * enc, 1.0f, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[4] * enc, y[5] * enc, 1.0f, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[6] * enc, y[7] * enc, 1.0f, 3);
  return r;
}

// E4M3 scale code and encode factor of a block with largest magnitude bmax
// under the group's S (the per-tensor float32 steps).
__device__ __forceinline__ void nv_scale_enc(float bmax, float S, uint32_t& s8, float& enc) {
  float sf = (bmax / 6.0f) * S;
  sf = __builtin_fminf(sf, 448.0f);
  s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sf, 0.0f, 0, false) & 0xffu;
  const float sd = e4m3_decode_pos(s8);
  enc = 0.0f;
  if (sd != 0.0f) enc = __builtin_fminf(S / sd, 3.40282346638528859812e+38f);
}

constexpr int kRhtBatch = 4;  // blocks (32 bytes each) in flight per thread

}  // namespace

// The group amax pass over transformed blocks: as nvfp4_group_amax_kernel, with
// 16-element blocks (two 16-byte loads) in place of 16-byte chunks.
__global__ __launch_bounds__(kAmaxThreads) void nvfp4_group_amax_rht_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, uint32_t mask, uint32_t* __restrict__ amax_bits,
    uint32_t* status) {
  __shared__ int64_t s_off[kMaxGroups + 1];
  __shared__ uint32_t s_max[kMaxGroups];
  const int tid = threadIdx.x;
  for (int g = tid; g < G; g += kAmaxThreads) s_max[g] = 0u;
  load_offsets_clamped(offsets, G, rows_cap, s_off, blockIdx.x == 0 ? status : nullptr);
  const int64_t bpr = cols / 16;  // 16-element blocks per row
  const int64_t first = s_off[0] * bpr, total = s_off[G] * bpr;
  const int64_t span = total > first ? total - first : 0;
  const int64_t per = (span + gridDim.x - 1) / gridDim.x;
  const int64_t c0 = first + (int64_t)blockIdx.x * per;
  const int64_t c1 = c0 + per < total ? c0 + per : total;
  int64_t c = c0 + tid;
  if (c < c1) {
    const int64_t row = c / bpr;
    int g = 0, hi = G - 1;  // the largest g with s_off[g] <= row
    while (g < hi) {
      const int mid = (g + hi + 1) >> 1;
      if (s_off[mid] <= row) g = mid; else hi = mid - 1;
    }
    int64_t bound = s_off[g + 1] * bpr;  // first block past group g
    const uint4* __restrict__ xv = reinterpret_cast<const uint4*>(x);
    uint32_t m = 0;
    for (; c < c1; c += kRhtBatch * kAmaxThreads) {
      uint4 v[kRhtBatch][2];  // the batch's loads are all issued before any is used
#pragma unroll
      for (int k = 0; k < kRhtBatch; ++k) {
        const int64_t ck = c + (int64_t)k * kAmaxThreads;
        v[k][0] = ck < c1 ? xv[2 * ck] : make_uint4(0, 0, 0, 0);
        v[k][1] = ck < c1 ? xv[2 * ck + 1] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < kRhtBatch; ++k) {
        const int64_t ck = c + (int64_t)k * kAmaxThreads;
        if (ck >= c1) break;
        if (ck >= bound) {
          atomicMax(&s_max[g], m);
          m = 0;
          while (g < G - 1 && s_off[g + 1] * bpr <= ck) ++g;
          bound = s_off[g + 1] * bpr;
        }
        float y[16];
        rht16(v[k][0], v[k][1], mask, y);
        m = max(m, fmag_bits(y));
      }
    }
    atomicMax(&s_max[g], m);
  }
  __syncthreads();
  for (int g = tid; g < G; g += kAmaxThreads)
    if (s_max[g] != 0u) atomicMax(&amax_bits[g], s_max[g]);
}

// The cast of transformed rows: one 256-thread block per live row, each thread
// transforming up to four 16-element blocks in registers (LONG: the blocks past
// them are read and transformed again); the row's group amax as in the plain
// per-tensor cast; rows that no group owns are left untouched.
template <bool LONG>
__global__ __launch_bounds__(kNvThreads) void nvfp4_pertensor_rht_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, uint32_t mask, uint8_t* __restrict__ data,
    uint8_t* __restrict__ bscales, const float* __restrict__ group_amax) {
  __shared__ uint32_t s_grp[2];
  int64_t live = offsets[G];
  if (live < 0) live = 0;
  if (live > rows_cap) live = rows_cap;
  const int64_t row = blockIdx.x;
  if (row >= live) return;
  const int tid = threadIdx.x;
  const int64_t nblk = cols / 16;
  const uint16_t* xr = x + row * cols;
  uint8_t* drow = data + row * (cols / 2);
  uint8_t* srow = bscales + row * nblk;
  constexpr int64_t kRegBlocks = (int64_t)kNvMaxBlocksPerThread * kNvThreads;

  float y[kNvMaxBlocksPerThread][16];
  uint32_t bm[kNvMaxBlocksPerThread];
#pragma unroll
  for (int i = 0; i < kNvMaxBlocksPerThread; ++i) {
    const int64_t j = tid + (int64_t)kNvThreads * i;
    bm[i] = 0;
    if (j < nblk) {
      const uint4 a = load_stream16(xr + 16 * j), b = load_stream16(xr + 16 * j + 8);
      rht16(a, b, mask, y[i]);
      bm[i] = fmag_bits(y[i]);
    }
  }
  // the row's group amax in one round trip (see nvfp4_rowscaled_kernel)
  bool mine = false;
  uint32_t val = 0u;
  if (tid < G) {
    const int64_t lo = offsets[tid], hi = offsets[tid + 1];
    val = __float_as_uint(group_amax[tid]);
    mine = lo <= row && row < hi;
  }
  if (tid == 0) {
    s_grp[0] = 0u;
    s_grp[1] = 0u;
  }
  __syncthreads();
  if (mine) {
    s_grp[0] = val;
    s_grp[1] = 1u;
  }
  __syncthreads();
  if (s_grp[1] == 0u) return;  // uniform: no group owns this row
  const float amax = __uint_as_float(s_grp[0]);
  float S = amax > 0.0f ? 2688.0f / amax : 1.0f;
  S = __builtin_fminf(S, 3.40282346638528859812e+38f);
#pragma unroll
  for (int i = 0; i < kNvMaxBlocksPerThread; ++i) {
    const int64_t j = tid + (int64_t)kNvThreads * i;
    if (j < nblk) {
      uint32_t s8;
      float enc;
      nv_scale_enc(__uint_as_float(bm[i]), S, s8, enc);
      *reinterpret_cast<uint2*>(drow + 8 * j) =
          make_uint2(fp4_pack8f(&y[i][0], enc), fp4_pack8f(&y[i][8], enc));
      srow[j] = (uint8_t)s8;
    }
  }
  if constexpr (LONG) {
    for (int64_t j = kRegBlocks + tid; j < nblk; j += kNvThreads) {
      const uint4* p = reinterpret_cast<const uint4*>(xr + 16 * j);
      float t[16];
      rht16(p[0], p[1], mask, t);
      uint32_t s8;
      float enc;
      nv_scale_enc(__uint_as_float(fmag_bits(t)), S, s8, enc);
      *reinterpret_cast<uint2*>(drow + 8 * j) = make_uint2(fp4_pack8f(&t[0], enc),
                                                           fp4_pack8f(&t[8], enc));
      srow[j] = (uint8_t)s8;
    }
  }
}

hipError_t launch_quantize_nvfp4_pertensor_rht(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                               int G, const int64_t* offsets, uint32_t sign_mask,
                                               uint8_t* data, uint8_t* block_scales, float* amax,
                                               uint32_t* status, hipStream_t stream) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
  hipLaunchKernelGGL(nvfp4_amax_clear_kernel, dim3(1), dim3(256), 0, stream, bits, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows_cap == 0) return e;
  const int64_t nb = rows_cap * (cols / 16);
  int64_t blocks = (nb + kRhtBatch * kAmaxThreads - 1) / (kRhtBatch * kAmaxThreads);
  const int64_t most = (int64_t)device_cu_count() * kAmaxBlocksPerCu;
  if (blocks > most) blocks = most;
  hipLaunchKernelGGL(nvfp4_group_amax_rht_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0,
                     stream, x, rows_cap, cols, G, offsets, sign_mask, bits, status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nv_long_rows(cols))
    hipLaunchKernelGGL(nvfp4_pertensor_rht_kernel<true>, dim3((unsigned)rows_cap),
                       dim3(kNvThreads), 0, stream, x, rows_cap, cols, G, offsets, sign_mask,
                       data, block_scales, amax);
  else
    hipLaunchKernelGGL(nvfp4_pertensor_rht_kernel<false>, dim3((unsigned)rows_cap),
                       dim3(kNvThreads), 0, stream, x, rows_cap, cols, G, offsets, sign_mask,
                       data, block_scales, amax);
  return hipGetLastError();
}

// ---------------------------------------------------------------- per tensor, 2-D scales
//
// Per-tensor NVFP4 with one E4M3 scale per 16 x 16 block ("gemm.py",
// _jax_scaled_matmul: the NVFP4_2D_SCALING mode; 16 rows by 16 columns, the
// NVFP4 block in both directions, so a tensor and its transpose quantize to
// transposed codes).  Block rows start at each group's first row (a group's
// last one holds its remaining rows).  The group amax comes from the same pass
// as the 1-D per-tensor quantize; then one workgroup per (group, block row):
// thread t takes block columns t, t + 256, ..., holds the block's 16 rows of 32
// bytes in registers, takes the block maximum, and writes the 16 rows' codes
// and the block's scale byte in every row of it (the GEMM's per-row layout).

__global__ __launch_bounds__(kNvThreads) void nvfp4_pertensor_2d_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, uint8_t* __restrict__ data,
    uint8_t* __restrict__ bscales, const float* __restrict__ group_amax) {
  __shared__ int64_t s_off[kMaxGroups + 1];
  __shared__ int32_t s_cnt[kMaxGroups];
  __shared__ int32_t s_pre[kMaxGroups + 1];
  load_offsets_clamped(offsets, G, rows_cap, s_off, nullptr);
  for (int g = threadIdx.x; g < G; g += blockDim.x)
    s_cnt[g] = (int32_t)((group_extent(s_off, g) + 15) / 16);
  __syncthreads();
  wave0_exclusive_scan(s_cnt, G, s_pre);
  __syncthreads();
  const int unit = blockIdx.x;
  if (unit >= s_pre[G]) return;
  const int g = find_group(s_pre, G, unit);
  const int64_t r0 = s_off[g] + 16 * (int64_t)(unit - s_pre[g]);
  const int64_t rest = s_off[g + 1] - r0;
  const int nr = (int)(rest < 16 ? rest : 16);
  const float amax = group_amax[g];
  float S = amax > 0.0f ? 2688.0f / amax : 1.0f;
  S = __builtin_fminf(S, 3.40282346638528859812e+38f);
  const int64_t nblk = cols / 16;
  for (int64_t j = threadIdx.x; j < nblk; j += kNvThreads) {
    uint4 v[16][2];
    uint32_t bm = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      v[r][0] = v[r][1] = make_uint4(0, 0, 0, 0);
      if (r < nr) {
        const uint16_t* p = x + (r0 + r) * cols + 16 * j;
        v[r][0] = load_stream16(p);
        v[r][1] = load_stream16(p + 8);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) bm = max(bm, block_mag(v[r][0], v[r][1]));
    uint32_t s8;
    float enc;
    nv_scale_enc(bf16_to_f32(bm), S, s8, enc);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (r < nr) {
        *reinterpret_cast<uint2*>(data + (r0 + r) * (cols / 2) + 8 * j) =
            make_uint2(fp4_pack8(v[r][0], enc), fp4_pack8(v[r][1], enc));
        bscales[(r0 + r) * nblk + j] = (uint8_t)s8;
      }
    }
  }
}

hipError_t launch_quantize_nvfp4_pertensor_2d(const uint16_t* x, int64_t rows_cap, int64_t cols,
                                              int G, const int64_t* offsets, uint8_t* data,
                                              uint8_t* block_scales, float* amax, uint32_t* status,
                                              hipStream_t stream) {
  uint32_t* bits = reinterpret_cast<uint32_t*>(amax);
  hipLaunchKernelGGL(nvfp4_amax_clear_kernel, dim3(1), dim3(256), 0, stream, bits, G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || rows_cap == 0) return e;
  const int64_t chunks = rows_cap * (cols / 8);
  int64_t blocks = (chunks + kAmaxBatch * kAmaxThreads - 1) / (kAmaxBatch * kAmaxThreads);
  const int64_t most = (int64_t)device_cu_count() * kAmaxBlocksPerCu;
  if (blocks > most) blocks = most;
  hipLaunchKernelGGL(nvfp4_group_amax_kernel, dim3((unsigned)blocks), dim3(kAmaxThreads), 0, stream,
                     x, rows_cap, cols, G, offsets, bits, status);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // upper bound of the block rows: every group adds at most one partial one
  const int64_t units = rows_cap / 16 + G;
  hipLaunchKernelGGL(nvfp4_pertensor_2d_kernel, dim3((unsigned)units), dim3(kNvThreads), 0, stream,
                     x, rows_cap, cols, G, offsets, data, block_scales, amax);
  return hipGetLastError();
}

// ---------------------------------------------------------------- columnwise
//
// Columnwise (transposed) copies for the weight gradient: "[Common][PyTorch]
// Add row-scaled NVFP4 support to grouped-tensor GEMM" lets wgrad consume the
// transpose of row-scaled grouped tensors, with the columnwise amax sized per
// column and split per expert.  Per expert g the block X_g^T [C, m~_g] (tokens
// padded with zeros to m~_g, a multiple of 128) is quantized row by row exactly
// as the rowwise kernel above quantizes rows: column c of expert g gets the
// outer scale amax / 2688 over the expert's tokens, 16-token blocks an E4M3
// scale, tokens E2M1 codes.  Output: the packed [C, m~_g / 2] block at byte
// padded_offsets[g] * C / 2, the E4M3 [C, m~_g / 16] block at
// padded_offsets[g] * C / 16, outer scales [G, C].
//
// One workgroup per (expert, 64-column slab) owns its columns' amax outright,
// so the whole quantize is one launch without atomics or workspace: a first
// pass over the expert's tokens takes the column maxima, a second pass reads
// the same tokens again (mostly from the L2 / last-level cache) and converts
// them.  The workgroup is four 256-thread sub-groups, each taking every fourth
// 128-token tile in both passes, so an expert's tokens are walked in a quarter
// of the memory round trips.  The second pass stages each sub-group's
// 128-token x 64-column tile (16 KiB) in LDS from registers loaded one tile
// ahead; thread (column pair p, 16-token block b) reads its 16 tokens of the
// two columns as 4-byte words and writes 8 packed bytes and one scale byte per
// column, so the 8 threads of a column write its 64 bytes contiguously.
constexpr int kNvColCols = 64;
constexpr int kNvColTokens = 128;
constexpr int kNvColSubs = 4;                      // sub-groups of 256 threads
constexpr int kNvColThreads = 256 * kNvColSubs;

namespace {

typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// LDS byte offset of 16-byte chunk q (columns 8 q .. 8 q + 7) of tile row r:
// the XOR with (r / 16) % 8 puts the 4-byte column-pair reads of one token of
// eight 16-token blocks on different banks.
__device__ __forceinline__ uint32_t nvcol_slot(int r, int q) {
  return (uint32_t)(r * 128 + ((q ^ ((r >> 4) & 7)) << 4));
}

// Thread u's (u < 256, its index in the sub-group) four 16-byte loads of a
// tile (token rows u / 8 + 32 i, columns 8 (u % 8) ..), zeros past the
// expert's tokens or the last column.
__device__ __forceinline__ void nvcol_load(const uint16_t* __restrict__ x, int64_t cols,
                                           int64_t row0, int live_rows, int64_t c0, int u,
                                           uint4 (&v)[4]) {
  const int tid = u;
  const int64_t c = c0 + 8 * (tid & 7);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    v[i] = make_uint4(0, 0, 0, 0);
    if (r < live_rows && c < cols)
      v[i] = *reinterpret_cast<const uint4*>(x + (row0 + r) * cols + c);
  }
}

__device__ __forceinline__ uint32_t pk_mag_max(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_elementwise_max(__builtin_bit_cast(v2u16, a & 0x7fff7fffu),
                                                      __builtin_bit_cast(v2u16, b & 0x7fff7fffu)));
}

// E2M1 codes of 16 tokens of one column (the bf16 in the low (HI = 0) or high
// half of w[i]) times enc, token 2j in the low nibble of byte j.
template <int HI, int J>
__device__ __forceinline__ uint32_t fp4_col_pair(uint32_t r, const uint32_t (&w)[16], float enc) {
  const float a = HI ? __uint_as_float(w[2 * J] & 0xffff0000u) : bf16_to_f32(w[2 * J] & 0xffffu);
  const float b =
      HI ? __uint_as_float(w[2 * J + 1] & 0xffff0000u) : bf16_to_f32(w[2 * J + 1] & 0xffffu);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, a * enc, b * enc, 1.0f, J & 3);
}

template <int HI>
__device__ __forceinline__ uint2 fp4_pack_col16(const uint32_t (&w)[16], float enc) {
  uint32_t lo = 0, hi = 0;
  lo = fp4_col_pair<HI, 0>(lo, w, enc);
  lo = fp4_col_pair<HI, 1>(lo, w, enc);
  lo = fp4_col_pair<HI, 2>(lo, w, enc);
  lo = fp4_col_pair<HI, 3>(lo, w, enc);
  hi = fp4_col_pair<HI, 4>(hi, w, enc);
  hi = fp4_col_pair<HI, 5>(hi, w, enc);
  hi = fp4_col_pair<HI, 6>(hi, w, enc);
  hi = fp4_col_pair<HI, 7>(hi, w, enc);
  return make_uint2(lo, hi);
}

// Block scale byte and encode factor of a 16-token block with largest
// magnitude bits `bm`, in the rowwise kernel's float32 steps.
__device__ __forceinline__ void nv_block_scale(uint32_t bm, float S, uint32_t& s8, float& enc) {
  const float bmax = bf16_to_f32(bm);
  float sf = (bmax / 6.0f) * S;
  sf = __builtin_fminf(sf, 448.0f);
  s8 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sf, 0.0f, 0, false) & 0xffu;
  const float sd = e4m3_decode_pos(s8);
  enc = 0.0f;
  if (sd != 0.0f) enc = __builtin_fminf(S / sd, 3.40282346638528859812e+38f);
}

}  // namespace

__global__ __launch_bounds__(kNvColThreads) void nvfp4_colwise_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ poffsets, int64_t col_cap,
    uint8_t* __restrict__ data, uint8_t* __restrict__ bscales, float* __restrict__ outer,
    uint32_t* status) {
  __shared__ int64_t s_off[kMaxGroups + 1];
  __shared__ int64_t s_poff[kMaxGroups + 1];
  __shared__ uint32_t s_amax[kNvColThreads / 64][kNvColCols / 2];
  __shared__ int s_order[kMaxGroups];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kNvColSubs][kNvColTokens * kNvColCols * 2];
  const bool report = blockIdx.x == 0;
  load_offsets_clamped(offsets, G, rows_cap, s_off, report ? status : nullptr);
  load_offsets_clamped(poffsets, G, col_cap, s_poff, report ? status : nullptr);
  // experts in decreasing padded size (ties by index), so that the longest
  // slabs start first and the short ones fill in behind them
  for (int h = threadIdx.x; h < G; h += blockDim.x) {
    const int64_t mh = group_extent(s_poff, h);
    int rank = 0;
    for (int j = 0; j < G; ++j) {
      const int64_t mj = group_extent(s_poff, j);
      rank += (mj > mh || (mj == mh && j < h)) ? 1 : 0;
    }
    s_order[rank] = h;
  }
  __syncthreads();
  const int64_t nslab = (cols + kNvColCols - 1) / kNvColCols;
  if ((int64_t)blockIdx.x >= (int64_t)G * nslab) return;
  const int g = s_order[blockIdx.x / nslab];
  const int64_t c0 = (blockIdx.x % nslab) * kNvColCols;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int sub = tid >> 8, u = tid & 255;  // sub-group, thread within it
  const int64_t m = group_extent(s_off, g), mp = group_extent(s_poff, g);
  const bool ok = s_poff[g] % kNvColTokens == 0 && mp % kNvColTokens == 0 && mp >= m;
  if (!ok) {
    if (tid == 0 && c0 == 0) dev_status_or(status, kDevBadPadding);
    return;
  }
  const int64_t row0 = s_off[g];

  // pass 1: column maxima (bf16 magnitude bits) over the expert's tokens; this
  // thread sees columns c0 + 8 (tid % 8) .. + 7 as four packed pairs
  uint32_t am[4] = {0, 0, 0, 0};
  for (int64_t t0 = (int64_t)sub * kNvColTokens; t0 < m; t0 += kNvColSubs * kNvColTokens) {
    uint4 v[4];
    nvcol_load(x, cols, row0 + t0, (int)(m - t0 < kNvColTokens ? m - t0 : kNvColTokens), c0, u, v);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      am[0] = pk_mag_max(am[0], v[i].x);
      am[1] = pk_mag_max(am[1], v[i].y);
      am[2] = pk_mag_max(am[2], v[i].z);
      am[3] = pk_mag_max(am[3], v[i].w);
    }
  }
  // lanes l, l ^ 8, l ^ 16, ... of a wave hold the same columns
#pragma unroll
  for (int d = 8; d < 64; d <<= 1)
#pragma unroll
    for (int q = 0; q < 4; ++q) am[q] = pk_mag_max(am[q], (uint32_t)__shfl_xor((int)am[q], d, 64));
  if (lane < 8) {
#pragma unroll
    for (int q = 0; q < 4; ++q) s_amax[w][4 * lane + q] = am[q];
  }
  __syncthreads();
  // thread (p, b) of a sub-group: column pair p = u / 8 (columns c0 + 2 p, + 1),
  // block b = u % 8
  const int p = u >> 3, b = u & 7;
  uint32_t pm = 0;
#pragma unroll
  for (int i = 0; i < kNvColThreads / 64; ++i) pm = pk_mag_max(pm, s_amax[i][p]);
  float S[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const float amax = bf16_to_f32(e ? pm >> 16 : pm & 0xffffu);
    S[e] = amax > 0.0f ? 2688.0f / amax : 1.0f;
    S[e] = __builtin_fminf(S[e], 3.40282346638528859812e+38f);
    const int64_t c = c0 + 2 * p + e;
    if (sub == 0 && b == 0 && c < cols) outer[(int64_t)g * cols + c] = amax / 2688.0f;
  }
  if (mp == 0) return;

  // pass 2: convert, each sub-group one 128-token tile at a time (padding
  // tokens load as zeros); every sub-group runs the same number of rounds
  const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)tile[sub];
  uint8_t* dg = data + s_poff[g] * cols / 2;       // expert g's [C, mp / 2] block
  uint8_t* sg = bscales + s_poff[g] * cols / 16;   // and its [C, mp / 16] scales
  const auto live_in = [&](int64_t t) {            // live tokens in the tile at t
    const int64_t rest = m - t;
    return (int)(rest < 0 ? 0 : (rest > kNvColTokens ? kNvColTokens : rest));
  };
  uint4 v[4];
  nvcol_load(x, cols, row0 + (int64_t)sub * kNvColTokens, live_in((int64_t)sub * kNvColTokens), c0,
             u, v);
  for (int64_t base = 0; base < mp; base += kNvColSubs * kNvColTokens) {
    const int64_t t0 = base + (int64_t)sub * kNvColTokens;
    const bool has = t0 < mp;
    __syncthreads();
    if (has) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 q = v[i];
        *reinterpret_cast<__attribute__((address_space(3))) v4i*>(
            (size_t)(lds + nvcol_slot((u >> 3) + 32 * i, u & 7))) =
            v4i{(int)q.x, (int)q.y, (int)q.z, (int)q.w};
      }
    }
    __syncthreads();
    const int64_t tn = t0 + kNvColSubs * kNvColTokens;
    if (tn < mp) nvcol_load(x, cols, row0 + tn, live_in(tn), c0, u, v);
    if (!has) continue;
    // tokens 16 b .. 16 b + 15 of columns 2 p, 2 p + 1 as bf16 pairs
    uint32_t wv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 16 * b + i;
      wv[i] = *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>(
          (size_t)(lds + nvcol_slot(r, p >> 2) + 4 * (p & 3)));
    }
    uint32_t bm2 = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) bm2 = pk_mag_max(bm2, wv[i]);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      uint32_t s8;
      float enc;
      nv_block_scale(e ? bm2 >> 16 : bm2 & 0xffffu, S[e], s8, enc);
      const uint2 q = e ? fp4_pack_col16<1>(wv, enc) : fp4_pack_col16<0>(wv, enc);
      const int64_t c = c0 + 2 * p + e;
      if (c < cols) {
        *reinterpret_cast<uint2*>(dg + c * (mp / 2) + t0 / 2 + 8 * b) = q;
        sg[c * (mp / 16) + t0 / 16 + b] = (uint8_t)s8;
      }
    }
  }
}

hipError_t launch_quantize_nvfp4_rowscaled_colwise(const uint16_t* x, int64_t rows_cap,
                                                   int64_t cols, int G, const int64_t* offsets,
                                                   const int64_t* padded_offsets,
                                                   int64_t col_rows_cap, uint8_t* data,
                                                   uint8_t* block_scales, float* outer,
                                                   uint32_t* status, hipStream_t stream) {
  const int64_t blocks = (int64_t)G * ((cols + kNvColCols - 1) / kNvColCols);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(nvfp4_colwise_kernel, dim3((unsigned)blocks), dim3(kNvColThreads), 0, stream, x,
                     rows_cap, cols, G, offsets, padded_offsets, col_rows_cap, data, block_scales,
                     outer, status);
  return hipGetLastError();
}

}  // namespace bsg
