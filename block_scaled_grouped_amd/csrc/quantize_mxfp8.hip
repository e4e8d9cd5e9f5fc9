// Grouped MXFP8 quantize: bf16 -> E4M3 elements + one E8M0 scale per 32
// elements along the contraction dim, rowwise and columnwise (transposed).
//
// "[JAX] MXFP8 Grouped Quant+GEMM": grouped quantize over ragged row groups,
// with the scale order the GEMM consumes written by the quantize itself (no
// separate swizzle pass).  "gemm.py", _quantize_gemm_operands: an operand is
// quantized along its contraction dim -- rowwise for fprop (contraction =
// last dim), columnwise/transposed for wgrad (contraction = token rows).
//
// Per 32-element block: amax = largest |x| (integer max of the bf16 magnitude
// bits), scale byte = max(exponent(amax) - 8, 0) (the E4M3 maximum 448 sits in
// binade 8), element = E4M3(x * 2^(127 - byte)), ties to even, saturated at
// 448.  The multiply by a power of two is exact in fp32; the values are
// clamped to +-448 before the hardware convert, which rounds to nearest even
// but would give NaN from 464 up.
#include "bsg_internal.h"

namespace bsg {

namespace {

__device__ __forceinline__ float clamp448(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
}

// E8M0 byte from the largest bf16 magnitude bits of a block.
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
  const uint32_t e = amax_bits >> 7;  // biased exponent of the bf16 magnitude
  return e > 8u ? e - 8u : 0u;
}

// 2^(127 - byte) as float; byte <= 247 for finite input, so always normal.
__device__ __forceinline__ float inv_scale(uint32_t byte) {
  return __uint_as_float((254u - byte) << 23);
}

__device__ __forceinline__ uint32_t amax_bits_of(uint32_t w) {
  return max(w & 0x7fffu, (w >> 16) & 0x7fffu);
}

// Two packed bf16 (low element first) times f -> two E4M3 bytes in the low
// (HI = false) or high half of `old`.
template <bool HI>
__device__ __forceinline__ int cvt2(uint32_t w, float f, int old) {
  float a = clamp448(bf16_to_f32(w & 0xffffu) * f);
  float b = clamp448(__uint_as_float(w & 0xffff0000u) * f);
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// 8 bf16 (4 dwords) -> 8 E4M3 bytes (2 dwords).
__device__ __forceinline__ uint2 cvt8(uint4 v, float f) {
  int lo = cvt2<false>(v.x, f, 0);
  lo = cvt2<true>(v.y, f, lo);
  int hi = cvt2<false>(v.z, f, 0);
  hi = cvt2<true>(v.w, f, hi);
  return make_uint2((uint32_t)lo, (uint32_t)hi);
}

// Position of logical scale byte j of a row in the GEMM-ready order: within
// every 4 bytes the stored order is b0, b2, b1, b3.
__device__ __forceinline__ int64_t scale_pos(int64_t j) {
  return (j & ~int64_t(3)) + ((j & 1) << 1) + ((j >> 1) & 1);
}

}  // namespace

// ---------------------------------------------------------------- rowwise
//
// One wavefront per (row, 1024-element chunk).  Lane l converts elements
// [8l, 8l+8) and [512+8l, 512+8l+8) of the chunk: every load and store
// instruction of the wave covers 1 KiB (512 B) of contiguous memory.  Four
// lanes form one 32-element block (amax by two xor-shuffles); sixteen lanes
// form one 128-element stretch whose four scale bytes are written as one
// dword in the b0, b2, b1, b3 order.
constexpr int kRowChunk = 1024;

__global__ __launch_bounds__(256) void mx_rowwise_kernel(const uint16_t* __restrict__ x,
                                                         int64_t rows_cap, int64_t cols, int G,
                                                         const int64_t* __restrict__ offsets,
                                                         uint8_t* __restrict__ data,
                                                         uint8_t* __restrict__ scales,
                                                         uint32_t* status) {
  int64_t live = offsets[G];
  if (live < 0) live = 0;
  if (live > rows_cap) {
    if (blockIdx.x == 0 && threadIdx.x == 0) dev_status_or(status, kDevOverCapacity);
    live = rows_cap;
  }
  const int lane = threadIdx.x & 63;
  const int64_t chunks = (cols + kRowChunk - 1) / kRowChunk;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t row = unit / chunks;
  if (row >= live) return;
  const int64_t base = (unit % chunks) * kRowChunk;

  const uint16_t* xr = x + row * cols;
  int64_t e[2] = {base + 8 * lane, base + 512 + 8 * lane};
  uint4 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    v[h] = e[h] < cols ? *reinterpret_cast<const uint4*>(xr + e[h]) : make_uint4(0, 0, 0, 0);

#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t am = max(max(amax_bits_of(v[h].x), amax_bits_of(v[h].y)),
                      max(amax_bits_of(v[h].z), amax_bits_of(v[h].w)));
    am = max(am, (uint32_t)__shfl_xor((int)am, 1, 64));
    am = max(am, (uint32_t)__shfl_xor((int)am, 2, 64));
    const uint32_t byte = e8m0_from_amax_bits(am);
    // gather the four block bytes of this lane's 128-element stretch
    const uint32_t b1 = (uint32_t)__shfl_down((int)byte, 4, 16);
    const uint32_t b2 = (uint32_t)__shfl_down((int)byte, 8, 16);
    const uint32_t b3 = (uint32_t)__shfl_down((int)byte, 12, 16);
    if (e[h] < cols) {
      uint2 q = cvt8(v[h], inv_scale(byte));
      *reinterpret_cast<uint2*>(data + row * cols + e[h]) = q;
      if ((lane & 15) == 0) {
        const uint32_t dw = byte | (b2 << 8) | (b1 << 16) | (b3 << 24);
        // word (q, row) of the [NQ][rows_cap] scale array, q = 128-element stretch
        *reinterpret_cast<uint32_t*>(scales + 4 * ((e[h] / 128) * rows_cap + row)) = dw;
      }
    }
  }
}

hipError_t launch_quantize_mxfp8_rowwise(const uint16_t* x, int64_t rows_cap, int64_t cols, int G,
                                         const int64_t* offsets, uint8_t* data, uint8_t* scales,
                                         uint32_t* status, hipStream_t stream) {
  if (rows_cap == 0) return hipSuccess;
  const int64_t chunks = (cols + kRowChunk - 1) / kRowChunk;
  const int64_t units = rows_cap * chunks;
  const int64_t blocks = (units + 3) / 4;
  hipLaunchKernelGGL(mx_rowwise_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows_cap,
                     cols, G, offsets, data, scales, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------- columnwise
//
// One 256-thread block per (128-token tile of a group, 64-column slab).  The
// bf16 tile is staged in LDS (128 rows x 128 B).  Columnwise: wave w takes the
// 32-token block w and lane l the column l, so LDS reads are conflict-free row
// reads; each lane writes its column's 32 E4M3 bytes (two 16-byte stores) and
// one scale byte.  Rowwise (when requested): thread t takes row t/2 and the
// 32-column block t%2 of the same LDS tile, so the input is read from HBM once
// for both outputs.  Tokens past the group's size are zeros (pad bytes 0x00,
// all-padding blocks get scale 0x00).
constexpr int kColTokens = 128;
constexpr int kColCols = 64;

__global__ __launch_bounds__(256) void mx_colwise_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ poffsets, int64_t col_cap,
    uint8_t* __restrict__ col_data, uint8_t* __restrict__ col_scales, uint8_t* __restrict__ row_data,
    uint8_t* __restrict__ row_scales, uint32_t* status) {
  __shared__ int64_t s_off[kMaxGroups + 1];
  __shared__ int64_t s_poff[kMaxGroups + 1];
  __shared__ uint16_t tile[kColTokens][kColCols];

  const int64_t nslab = (cols + kColCols - 1) / kColCols;
  const int64_t ttile = blockIdx.x / nslab;
  const int64_t c0 = (blockIdx.x % nslab) * kColCols;
  const bool report = blockIdx.x == 0;
  load_offsets_clamped(offsets, G, rows_cap, s_off, report ? status : nullptr);
  load_offsets_clamped(poffsets, G, col_cap, s_poff, report ? status : nullptr);

  const int64_t t0 = ttile * kColTokens;  // padded token index of the tile
  if (t0 >= s_poff[G]) return;
  int lo = 0, hi = G - 1;  // group: largest g with s_poff[g] <= t0
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_poff[mid] <= t0) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int64_t m = group_extent(s_off, g);
  const int64_t mp = group_extent(s_poff, g);
  if (s_poff[g] % kColPad != 0 || mp % kColPad != 0 || mp < m) {
    if (threadIdx.x == 0 && t0 == s_poff[g] && c0 == 0) dev_status_or(status, kDevBadPadding);
    return;
  }
  const int64_t tt = t0 - s_poff[g];           // token offset of the tile inside the group
  if (tt >= mp) return;                        // only with invalid (decreasing) padded offsets
  int64_t nv = m - tt;                         // live tokens in this tile
  nv = nv < 0 ? 0 : (nv > kColTokens ? kColTokens : nv);
  const int64_t row0 = s_off[g] + tt;

  // stage the bf16 tile (zeros past the live tokens and past the last column)
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = (tid >> 3) + 32 * p;
    const int ch = tid & 7;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < nv && c0 + ch * 8 < cols)
      v = *reinterpret_cast<const uint4*>(x + (row0 + r) * cols + c0 + ch * 8);
    *reinterpret_cast<uint4*>(&tile[r][ch * 8]) = v;
  }
  __syncthreads();

  // columnwise
  {
    const int w = tid >> 6;     // 32-token block
    const int c = tid & 63;     // column within the slab
    if (c0 + c < cols) {
      uint32_t wv[16];
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t lo16 = tile[32 * w + 2 * i][c];
        uint32_t hi16 = tile[32 * w + 2 * i + 1][c];
        wv[i] = lo16 | (hi16 << 16);
        am = max(am, max(lo16 & 0x7fffu, hi16 & 0x7fffu));
      }
      const uint32_t byte = e8m0_from_amax_bits(am);
      const float f = inv_scale(byte);
      uint32_t q[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint2 r = cvt8(make_uint4(wv[4 * i], wv[4 * i + 1], wv[4 * i + 2], wv[4 * i + 3]), f);
        q[2 * i] = r.x;
        q[2 * i + 1] = r.y;
      }
      uint8_t* dst = col_data + s_poff[g] * cols + (c0 + c) * mp + tt + 32 * w;
      reinterpret_cast<uint4*>(dst)[0] = make_uint4(q[0], q[1], q[2], q[3]);
      reinterpret_cast<uint4*>(dst)[1] = make_uint4(q[4], q[5], q[6], q[7]);
      // word (tt / 128, column) of the group's [m~/128][cols] scale array; byte w
      // in the b0, b2, b1, b3 order
      col_scales[s_poff[g] * cols / 32 + 4 * ((tt / 128) * cols + c0 + c) + scale_pos(w)] =
          (uint8_t)byte;
    }
  }

  // rowwise from the same tile
  if (row_data != nullptr) {
    const int r = tid >> 1;
    const int hb = tid & 1;
    const int64_t col = c0 + 32 * hb;
    if (r < nv && col < cols) {
      uint4 v[4];
      uint32_t am = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = *reinterpret_cast<const uint4*>(&tile[r][32 * hb + 8 * i]);
        am = max(am, max(max(amax_bits_of(v[i].x), amax_bits_of(v[i].y)),
                         max(amax_bits_of(v[i].z), amax_bits_of(v[i].w))));
      }
      const uint32_t byte = e8m0_from_amax_bits(am);
      const float f = inv_scale(byte);
      uint2 q0 = cvt8(v[0], f), q1 = cvt8(v[1], f), q2 = cvt8(v[2], f), q3 = cvt8(v[3], f);
      const int64_t row = row0 + r;
      uint8_t* dst = row_data + row * cols + col;
      reinterpret_cast<uint4*>(dst)[0] = make_uint4(q0.x, q0.y, q1.x, q1.y);
      reinterpret_cast<uint4*>(dst)[1] = make_uint4(q2.x, q2.y, q3.x, q3.y);
      // word (q, row) of the [NQ][rows_cap] scale array, byte of block col / 32
      const int64_t jb = col / 32;
      row_scales[4 * ((jb / 4) * rows_cap + row) + scale_pos(jb & 3)] = (uint8_t)byte;
      // a row whose last 128-element stretch is short gets zero pad bytes
      if (col + 32 >= cols) {
        const int64_t nblk = cols / 32;
        const int64_t srow = ((nblk + 3) / 4) * 4;
        for (int64_t j = nblk; j < srow; ++j)
          row_scales[4 * ((j / 4) * rows_cap + row) + scale_pos(j & 3)] = 0;
      }
    }
  }
}

hipError_t launch_quantize_mxfp8_colwise(const uint16_t* x, int64_t rows_cap, int64_t cols, int G,
                                         const int64_t* offsets, const int64_t* padded_offsets,
                                         int64_t col_rows_cap, uint8_t* col_data,
                                         uint8_t* col_scales, uint8_t* row_data,
                                         uint8_t* row_scales, uint32_t* status,
                                         hipStream_t stream) {
  const int64_t ttiles = (col_rows_cap + kColTokens - 1) / kColTokens;
  const int64_t nslab = (cols + kColCols - 1) / kColCols;
  const int64_t blocks = ttiles * nslab;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_colwise_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, rows_cap,
                     cols, G, offsets, padded_offsets, col_rows_cap, col_data, col_scales, row_data,
                     row_scales, status);
  return hipGetLastError();
}

}  // namespace bsg
