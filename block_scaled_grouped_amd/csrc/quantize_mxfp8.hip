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
// 448.  gfx950's v_cvt_scalef32_pk_fp8_bf16 converts two bf16 directly, divided
// by the power of two whose exponent field is the scale byte, rounding to
// nearest even -- exactly this -- except that magnitudes above 464 come out as
// the NaN code S.1111.111 instead of saturating; finite input never yields NaN
// otherwise, so those bytes are mapped to S.1111.110 (448) afterwards.
#include "bsg_internal.h"

namespace bsg {

namespace {

// E8M0 byte from the largest bf16 magnitude bits of a block: the OCP rule,
// exponent(amax) - emax of the element format (8 for E4M3, 15 for E5M2).
template <bool E5M2 = false>
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
  constexpr uint32_t emax = E5M2 ? 15u : 8u;
  const uint32_t e = amax_bits >> 7;  // biased exponent of the bf16 magnitude
  return e > emax ? e - emax : 0u;
}

// The scale operand of the scaled converts: a float whose exponent field is the
// E8M0 byte (the instruction reads only the exponent field).
__device__ __forceinline__ float e8m0_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));

// Lane moves inside 16-lane rows (DPP): the value of lane l ^ 1, and of lane
// l + N (only read where l + N stays inside the row).
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
}
template <int N>
__device__ __forceinline__ uint32_t dpp_down(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + N, 0xF, 0xF, false);  // row_shl N
}

// Largest of the two bf16 magnitudes in each 16-bit half of a and b.
__device__ __forceinline__ uint32_t amax2(uint32_t a, uint32_t b) {
  const v2u16 x = __builtin_bit_cast(v2u16, a & 0x7fff7fffu);
  const v2u16 y = __builtin_bit_cast(v2u16, b & 0x7fff7fffu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Combines the two halves of an amax2 result.
__device__ __forceinline__ uint32_t amax_fold(uint32_t m) { return max(m & 0xffffu, m >> 16); }

// Overflowed codes become the largest finite code, in each byte of a word:
// E4M3 S.1111.111 (only produced for magnitudes above 464) -> S.1111.110;
// E5M2 S.11111.00 (the infinity the E5M2 convert gives past 57344, the only
// exponent-31 code finite input produces) -> S.11110.11.
template <bool E5M2 = false>
__device__ __forceinline__ uint32_t fp8_saturate(uint32_t x) {
  constexpr uint32_t gap = E5M2 ? 0x04040404u : 0x01010101u;  // 0x80 - first overflow code
  const uint32_t t = (((x & 0x7f7f7f7fu) + gap) >> 7) & 0x01010101u;
  // E4M3: S.1111.111 -> S.1111.110 flips bit 0 (one bitwise op with the mask)
  return E5M2 ? x - t : x ^ t;
}

// Two packed bf16 (low element first), scaled -> two E4M3 (or E5M2) bytes in
// the low (HI = false) or high half of `old`.  Both converts are exact
// round-to-nearest-even of x / 2^scale up to the overflow handled above.
template <bool HI, bool E5M2 = false>
__device__ __forceinline__ uint32_t cvt2(uint32_t w, float scale, uint32_t old) {
  v2s r;
  if constexpr (E5M2)
    r = __builtin_amdgcn_cvt_scalef32_pk_bf8_bf16(__builtin_bit_cast(v2s, old),
                                                  __builtin_bit_cast(v2bf, w), scale, HI);
  else
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(v2s, old),
                                                  __builtin_bit_cast(v2bf, w), scale, HI);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 bf16 (4 dwords) -> 8 E4M3 (or E5M2) bytes (2 dwords).
template <bool E5M2 = false>
__device__ __forceinline__ uint2 cvt8(uint4 v, float scale) {
  // The first convert's other half is written by the second, so its prior
  // contents do not matter: passing the source word lets the result take the
  // source's register (no copy into a zeroed one).
  const uint32_t lo = cvt2<true, E5M2>(v.y, scale, cvt2<false, E5M2>(v.x, scale, v.x));
  const uint32_t hi = cvt2<true, E5M2>(v.w, scale, cvt2<false, E5M2>(v.z, scale, v.z));
  return make_uint2(fp8_saturate<E5M2>(lo), fp8_saturate<E5M2>(hi));
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
//
// The scale words of 32 consecutive rows share one 128-byte line of the
// [NQ][rows_cap] array, and workgroup b runs on XCD b % 8, each XCD with its
// own L2.  Workgroups are renumbered so that every XCD takes runs of 32 whole
// rows: each scale line is then completed in a single L2 and written back
// once, not as up to 8 partial lines.
// The bf16 input is read once, with non-temporal loads (load_stream16): on
// the 940 MB weight quantize that took 248 -> 227 us, and the columnwise
// quantize of the [8 x 14336, 4096] weights 304 -> 275 us.
constexpr int kRowChunk = 1024;

template <bool E5M2>
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
  const int64_t run = 8 * chunks;  // workgroups (4 units each) per 32 rows
  const int64_t full = (int64_t)gridDim.x / (kXcds * run) * (kXcds * run);
  int64_t wg = blockIdx.x;
  if (wg < full) {  // a permutation of [0, full); the tail keeps its order
    const int64_t xcd = wg % kXcds, idx = wg / kXcds;
    wg = ((idx / run) * kXcds + xcd) * run + idx % run;
  }
  const int64_t unit = wg * 4 + (threadIdx.x >> 6);
  const int64_t row = unit / chunks;
  if (row >= live) return;
  const int64_t base = (unit % chunks) * kRowChunk;

  const uint16_t* xr = x + row * cols;
  int64_t e[2] = {base + 8 * lane, base + 512 + 8 * lane};
  uint4 v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    v[h] = e[h] < cols ? load_stream16(xr + e[h]) : make_uint4(0, 0, 0, 0);

#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t am = amax_fold(amax2(amax2(v[h].x, v[h].y), amax2(v[h].z, v[h].w)));
    am = max(am, (uint32_t)__shfl_xor((int)am, 1, 64));
    am = max(am, (uint32_t)__shfl_xor((int)am, 2, 64));
    const uint32_t byte = e8m0_from_amax_bits<E5M2>(am);
    // gather the four block bytes of this lane's 128-element stretch
    const uint32_t b1 = (uint32_t)__shfl_down((int)byte, 4, 16);
    const uint32_t b2 = (uint32_t)__shfl_down((int)byte, 8, 16);
    const uint32_t b3 = (uint32_t)__shfl_down((int)byte, 12, 16);
    if (e[h] < cols) {
      uint2 q = cvt8<E5M2>(v[h], e8m0_scale(byte));
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
                                         uint32_t* status, hipStream_t stream, bool e5m2) {
  if (rows_cap == 0) return hipSuccess;
  const int64_t chunks = (cols + kRowChunk - 1) / kRowChunk;
  const int64_t units = rows_cap * chunks;
  const int64_t blocks = (units + 3) / 4;
  if (e5m2)
    hipLaunchKernelGGL(mx_rowwise_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       rows_cap, cols, G, offsets, data, scales, status);
  else
    hipLaunchKernelGGL(mx_rowwise_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       rows_cap, cols, G, offsets, data, scales, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------- columnwise
//
// Three blocks of 4 waves per CU loop over tiles of (128 tokens of a group) x
// (128 columns).  A block stages a tile's bf16 values in LDS from registers
// loaded one tile ahead (rows past the group's live tokens and columns past the
// end are zeros), so the next tile's loads are in flight while the current one
// is converted: columnwise, then rowwise (when requested), so the input is read
// from HBM once for both outputs.  Each 32-element block's E4M3 bytes and scale
// are produced as described at the top of this file.
// Tokens past the group's size are zeros (pad bytes 0x00, all-padding blocks
// get scale 0x00).  In LDS, 16-byte chunk c of tile row r sits in slot
// c ^ ((r % 8) ^ ((r / 16) % 8)), which keeps the row-major stores and both
// read patterns (nearly) free of bank conflicts.
constexpr int kColTokens = 128;
constexpr int kColCols = 128;
constexpr int kColTileBytes = kColTokens * kColCols * 2;   // 32 KiB
constexpr int kColBlocksPerCu = 3;

__device__ __forceinline__ uint32_t col_tile_slot(int r, int c16) {
  return (uint32_t)(r * 256 + ((c16 ^ ((r & 7) ^ ((r >> 4) & 7))) << 4));
}

typedef __attribute__((address_space(3))) v4i lds_v4i;

__device__ __forceinline__ uint4 lds_ld16(uint32_t a) {
  const v4i v = *reinterpret_cast<const lds_v4i*>((size_t)a);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}
__device__ __forceinline__ uint32_t lds_ld4(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((size_t)a);
}

// 16 E4M3 (or E5M2) bytes from 16 values given as bf16 bits (element i in
// halves of w[i/2]).
template <bool E5M2 = false>
__device__ __forceinline__ uint4 cvt16(const uint32_t (&w)[8], float f) {
  const uint2 a = cvt8<E5M2>(make_uint4(w[0], w[1], w[2], w[3]), f);
  const uint2 b = cvt8<E5M2>(make_uint4(w[4], w[5], w[6], w[7]), f);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// Where tile `id` sits: its group, token offset, live tokens, first row.
struct ColTile {
  int64_t t0, c0, tt, row0, mp;
  int g, nv;
  bool ok;
};

__device__ __forceinline__ ColTile col_tile_info(int64_t id, int64_t nslab, int G,
                                                 const int64_t* s_off, const int64_t* s_poff) {
  ColTile t;
  t.t0 = (id / nslab) * kColTokens;
  t.c0 = (id % nslab) * kColCols;
  int lo = 0, hi = G - 1;  // group: largest g with s_poff[g] <= t0
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_poff[mid] <= t.t0) lo = mid; else hi = mid - 1;
  }
  t.g = lo;
  const int64_t m = group_extent(s_off, t.g);
  t.mp = group_extent(s_poff, t.g);
  t.tt = t.t0 - s_poff[t.g];
  t.ok = s_poff[t.g] % kColPad == 0 && t.mp % kColPad == 0 && t.mp >= m && t.tt < t.mp;
  const int64_t nv = m - t.tt;  // live tokens in this tile
  t.nv = (int)(nv < 0 ? 0 : (nv > kColTokens ? kColTokens : nv));
  t.row0 = s_off[t.g] + t.tt;
  return t;
}

// Columnwise part of a staged tile, NW waves: per pass, lane (k, q) of wave w
// takes a column pair 2 pc, 2 pc + 1 (pc = 8 w + q + the pass's base) and
// tokens [16 k, 16 k + 16) (4-byte LDS reads), so a column's 32-token block is split over lanes k, k ^ 1 and its 128
// output bytes are written by 8 neighbouring lanes, 16 bytes each; the column's
// four block scales become one word of the GEMM order.  E5M2: gradient elements
// (scale byte exponent(amax) - 15).
template <int NW, bool E5M2>
__device__ __forceinline__ void col_convert_columns(uint32_t lds, const ColTile& t, int64_t cols,
                                                    int64_t poff, int w, int lane,
                                                    uint8_t* __restrict__ col_data,
                                                    uint8_t* __restrict__ col_scales) {
  const int k = lane & 7;               // tokens [16 k, 16 k + 16)
#pragma unroll
  for (int pass = 0; pass < 8 / NW; ++pass) {
  const int pc = 64 / (8 / NW) * pass + 8 * w + (lane >> 3);   // columns 2 pc, 2 pc + 1
  uint32_t cw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i)
    cw[i] = lds_ld4(lds + col_tile_slot(16 * k + i, pc >> 2) + 4 * (pc & 3));
  const int64_t scale_base = poff * cols / 32 + 4 * ((t.tt / 128) * cols);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)  // tokens 2 i, 2 i + 1 of the column, as one bf16 pair
      pk[i] = __builtin_amdgcn_perm(cw[2 * i + 1], cw[2 * i], e ? 0x07060302u : 0x05040100u);
    uint32_t am = amax_fold(amax2(amax2(amax2(pk[0], pk[1]), amax2(pk[2], pk[3])),
                                  amax2(amax2(pk[4], pk[5]), amax2(pk[6], pk[7]))));
    am = max(am, dpp_xor1(am));   // the block's other 16 tokens
    const uint32_t byte = e8m0_from_amax_bits<E5M2>(am);
    const uint4 q = cvt16<E5M2>(pk, e8m0_scale(byte));
    // block bytes of tokens [0, 32), [32, 64), ... sit in lanes k = 0, 2, 4, 6
    const uint32_t b1 = dpp_down<2>(byte), b2 = dpp_down<4>(byte), b3 = dpp_down<6>(byte);
    const int64_t c = t.c0 + 2 * pc + e;
    if (c < cols) {
      *reinterpret_cast<uint4*>(col_data + poff * cols + c * t.mp + t.tt + 16 * k) = q;
      if (k == 0)
        *reinterpret_cast<uint32_t*>(col_scales + scale_base + 4 * c) =
            byte | (b2 << 8) | (b1 << 16) | (b3 << 24);
    }
  }
  }
}

// Rowwise part, NW waves: per pass, 8 lanes per row, 16 columns each; the
// row's four block scales become one word.
template <int NW>
__device__ __forceinline__ void col_convert_rows(uint32_t lds, const ColTile& t, int64_t cols,
                                                 int64_t rows_cap, int w, int lane,
                                                 uint8_t* __restrict__ row_data,
                                                 uint8_t* __restrict__ row_scales) {
  const int j = lane & 7;
#pragma unroll
  for (int pass = 0; pass < 16 / NW; ++pass) {
    const int r = 8 * NW * pass + 8 * w + (lane >> 3);
    const uint4 a = lds_ld16(lds + col_tile_slot(r, 2 * j));
    const uint4 b = lds_ld16(lds + col_tile_slot(r, 2 * j + 1));
    uint32_t am = amax_fold(amax2(amax2(amax2(a.x, a.y), amax2(a.z, a.w)),
                                  amax2(amax2(b.x, b.y), amax2(b.z, b.w))));
    am = max(am, dpp_xor1(am));   // the block's other 16 columns
    const uint32_t byte = e8m0_from_amax_bits(am);
    const float f = e8m0_scale(byte);
    const uint2 qa = cvt8(a, f), qb = cvt8(b, f);
    const uint32_t b1 = dpp_down<2>(byte), b2 = dpp_down<4>(byte), b3 = dpp_down<6>(byte);
    if (r < t.nv) {
      const int64_t row = t.row0 + r;
      const int64_t col = t.c0 + 16 * j;
      if (col < cols)
        *reinterpret_cast<uint4*>(row_data + row * cols + col) = make_uint4(qa.x, qa.y, qb.x, qb.y);
      // word (c0 / 128, row) of the [NQ][rows_cap] scale array, b0, b2, b1, b3
      // (blocks past the last column read zeros: byte 0)
      if (j == 0)
        *reinterpret_cast<uint32_t*>(row_scales + 4 * ((t.c0 / 128) * rows_cap + row)) =
            byte | (b2 << 8) | (b1 << 16) | (b3 << 24);
    }
  }
}


__device__ __forceinline__ void col_tile_load(const uint16_t* __restrict__ x, int64_t cols,
                                              const ColTile& t, uint4 (&v)[8]) {
  const int tid = threadIdx.x;
  const int c16 = tid & 15;
  const bool colok = t.ok && t.c0 + 8 * c16 < cols;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = (tid >> 4) + 16 * p;
    v[p] = make_uint4(0, 0, 0, 0);
    if (r < t.nv && colok)
      v[p] = load_stream16(x + (t.row0 + r) * cols + t.c0 + 8 * c16);
  }
}

__device__ __forceinline__ void lds_st16(uint32_t a, uint4 v) {
  *reinterpret_cast<lds_v4i*>((size_t)a) = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
}

template <bool E5M2>
__global__ __launch_bounds__(256) void mx_colwise_kernel(
    const uint16_t* __restrict__ x, int64_t rows_cap, int64_t cols, int G,
    const int64_t* __restrict__ offsets, const int64_t* __restrict__ poffsets, int64_t col_cap,
    uint8_t* __restrict__ col_data, uint8_t* __restrict__ col_scales, uint8_t* __restrict__ row_data,
    uint8_t* __restrict__ row_scales, uint32_t* status) {
  __shared__ int64_t s_off[kMaxGroups + 1];
  __shared__ int64_t s_poff[kMaxGroups + 1];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kColTileBytes];
  const bool report = blockIdx.x == 0;
  {
    // both offset arrays in one round trip (clamped and checked as
    // load_offsets_clamped does)
    uint32_t* st = report ? status : nullptr;
    for (int g = threadIdx.x; g <= G; g += blockDim.x) {
      int64_t v = offsets[g], pv = poffsets[g];
      uint32_t bad = 0;
      if (v < 0) { v = 0; bad |= kDevNegativeSize; }
      if (v > rows_cap) { v = rows_cap; bad |= kDevOverCapacity; }
      if (pv < 0) { pv = 0; bad |= kDevNegativeSize; }
      if (pv > col_cap) { pv = col_cap; bad |= kDevOverCapacity; }
      s_off[g] = v;
      s_poff[g] = pv;
      dev_status_or(st, bad);
    }
    __syncthreads();
    for (int g = threadIdx.x + 1; g <= G; g += blockDim.x)
      if (s_off[g] < s_off[g - 1] || s_poff[g] < s_poff[g - 1]) dev_status_or(st, kDevNegativeSize);
  }
  const uint32_t lds = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)tile;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane((int)(tid >> 6));
  const int64_t nslab = (cols + kColCols - 1) / kColCols;
  const int64_t ntiles = ((s_poff[G] + kColTokens - 1) / kColTokens) * nslab;
  int64_t id = blockIdx.x;
  if (id >= ntiles) return;
  ColTile cur = col_tile_info(id, nslab, G, s_off, s_poff);
  uint4 v[8];
  col_tile_load(x, cols, cur, v);
  for (; id < ntiles; id += gridDim.x) {
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 8; ++p) lds_st16(lds + col_tile_slot((tid >> 4) + 16 * p, tid & 15), v[p]);
    __syncthreads();
    const ColTile t = cur;
    if (id + gridDim.x < ntiles) {
      cur = col_tile_info(id + gridDim.x, nslab, G, s_off, s_poff);
      col_tile_load(x, cols, cur, v);
    }
    if (!t.ok) {
      if (tid == 0 && t.t0 == s_poff[t.g] && t.c0 == 0) dev_status_or(status, kDevBadPadding);
      continue;
    }
    col_convert_columns<4, E5M2>(lds, t, cols, s_poff[t.g], w, lane, col_data, col_scales);
    if (!E5M2 && row_data != nullptr)
      col_convert_rows<4>(lds, t, cols, rows_cap, w, lane, row_data, row_scales);
  }
}

hipError_t launch_quantize_mxfp8_colwise(const uint16_t* x, int64_t rows_cap, int64_t cols, int G,
                                         const int64_t* offsets, const int64_t* padded_offsets,
                                         int64_t col_rows_cap, uint8_t* col_data,
                                         uint8_t* col_scales, uint8_t* row_data,
                                         uint8_t* row_scales, uint32_t* status,
                                         hipStream_t stream, bool e5m2) {
  // upper bound of the tile count from the host-known capacity
  const int64_t bound = ((col_rows_cap + kColTokens - 1) / kColTokens) * ((cols + kColCols - 1) / kColCols);
  int64_t blocks = (int64_t)device_cu_count() * kColBlocksPerCu;
  if (bound < blocks) blocks = bound;
  if (blocks <= 0) return hipSuccess;
  if (e5m2)  // the gradient's columnwise copy only (no rowwise output)
    hipLaunchKernelGGL(mx_colwise_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       rows_cap, cols, G, offsets, padded_offsets, col_rows_cap, col_data,
                       col_scales, nullptr, nullptr, status);
  else
    hipLaunchKernelGGL(mx_colwise_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, x,
                       rows_cap, cols, G, offsets, padded_offsets, col_rows_cap, col_data,
                       col_scales, row_data, row_scales, status);
  return hipGetLastError();
}

}  // namespace bsg
