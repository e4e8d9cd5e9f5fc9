// Output stores of a 256 x 256 tile held as 4 x 4 transposed 32 x 32 MFMA
// accumulator blocks per wavefront (shared by the grouped GEMMs).
#ifndef BSG_STORE_TILE_H
#define BSG_STORE_TILE_H

#include "bsg_internal.h"

namespace bsg {

// Stores one 32 x 32 accumulator block: this lane's row `row`, columns
// col0 + 8 q + [0, 4) in registers 4 q .. 4 q + 3 (col0 = 32 j + 4 h).  `ro`
// covers the tile's valid rows, so stores to rows past them are dropped by the
// buffer range check; a column past out_cols gets an offset past every range
// (kDropped), which drops it the same way, without a branch.
//   WIDE, bf16 (row stride and out_cols multiples of 8): the two lanes of a row
//     trade halves with v_permlane32_swap so that lane h holds columns
//     16 h .. 16 h + 15 of the block as two 16-byte pieces; v_permlane16_swap
//     then regroups the pieces so that each of the two stores covers 16 whole
//     64-byte block rows (lane L: row L % 16, columns 8 (L / 16) .. + 7, and
//     the same 16 rows further) rather than half of each of the 32 rows,
//     which halves the cache lines every store instruction touches.
//   WIDE, f32 (multiples of 4): each run of four columns is one 16-byte store.
//   Otherwise: one store per element.
constexpr uint32_t kDropped = 0xfffffff0u;

template <bool WIDE, bool F32>
__device__ __forceinline__ void store_block(const v16f& acc, __amdgpu_buffer_rsrc_t ro, int ldc,
                                            int row, int col0, int h, int out_cols) {
  constexpr int esz = F32 ? 4 : 2;
  if constexpr (WIDE && !F32) {
    // d[2 q + e] = columns col0 + 8 q + 2 e, + 1 (bf16 pairs)
    int d[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
        d[2 * q + e] = __builtin_bit_cast(
            int, __builtin_convertvector((v2f){acc[4 * q + 2 * e], acc[4 * q + 2 * e + 1]}, v2bf));
    }
    // lane (r, 0) keeps d[0..3] and receives lane (r, 1)'s d[0..3] as d[4..7];
    // lane (r, 1) receives lane (r, 0)'s d[4..7] as d[0..3] and keeps d[4..7]
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto sw = __builtin_amdgcn_permlane32_swap(d[k], d[4 + k], false, false);
      d[k] = sw[0];
      d[4 + k] = sw[1];
    }
    // x: columns 16 h .. + 7 of row r, y: 16 h + 8 .. + 15.  After the swap of
    // x's odd 16-lane groups with y's even ones, lane L holds in x piece L / 16
    // of block row L % 16, in y the same piece of block row 16 + L % 16.
    int x[4] = {d[0], d[1], d[4], d[5]}, y[4] = {d[2], d[3], d[6], d[7]};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto sw = __builtin_amdgcn_permlane16_swap(x[k], y[k], false, false);
      x[k] = sw[0];
      y[k] = sw[1];
    }
    const int lane = threadIdx.x & 63;
    const int rowx = row - (lane & 31) + (lane & 15);
    const int col = col0 - 4 * h + 8 * (lane >> 4);
    const int base = rowx * ldc + col;
    const bool live = col < out_cols;
    const int offx = live ? base * esz : (int)kDropped;
    const int offy = live ? (base + 16 * ldc) * esz : (int)kDropped;
    __builtin_amdgcn_raw_buffer_store_b128((v4i){x[0], x[1], x[2], x[3]}, ro, offx, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128((v4i){y[0], y[1], y[2], y[3]}, ro, offy, 0, 0);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = col0 + 8 * q;
      const int idx = row * ldc + col;
      if constexpr (WIDE) {
        const int off = col < out_cols ? idx * esz : (int)kDropped;
        const v4i v = {__float_as_int(acc[4 * q]), __float_as_int(acc[4 * q + 1]),
                       __float_as_int(acc[4 * q + 2]), __float_as_int(acc[4 * q + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, ro, off, 0, 0);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int off = col + e < out_cols ? (idx + e) * esz : (int)kDropped;
          if constexpr (F32)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(acc[4 * q + e]), ro, off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16(
                (unsigned short)f32_to_bf16_rne(acc[4 * q + e]), ro, off, 0, 0);
        }
      }
    }
  }
}

template <bool WIDE, bool F32>
__device__ __forceinline__ void store_tile(const v16f (&acc)[4][4], __amdgpu_buffer_rsrc_t ro,
                                           int ldc, int row, int col, int h, int out_cols) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_block<WIDE, F32>(acc[i][j], ro, ldc, row + 32 * i, col + 32 * j, h, out_cols);
}

// Per-group epilogue terms: Y = alpha * S + beta * C + bias[column], C the
// output's previous contents (read only when beta != 0), bias float32 over the
// tile's columns (its descriptor covers them, so columns past them read 0).
struct EpiTerms {
  float alpha, beta;
  __amdgpu_buffer_rsrc_t bias;
  bool has_bias;
};

// One 32 x 32 accumulator block through the epilogue terms: this lane's row
// `row`, columns col0 + 8 q + [0, 4) in registers 4 q .. 4 q + 3.  WIDE (row
// stride and out_cols multiples of 4): each run of four columns is one vector
// load of C, one of the bias and one store; otherwise one element at a time.
// The three terms are combined in float32, then rounded once to the output.
// All of the block's loads are issued before its first store, so their
// latencies overlap (no store of the block writes a position one of its loads
// reads).
template <bool WIDE, bool F32>
__device__ __forceinline__ void store_block_ex(const v16f& acc, __amdgpu_buffer_rsrc_t ro, int ldc,
                                               int row, int col0, int out_cols, const EpiTerms& ep) {
  constexpr int esz = F32 ? 4 : 2;
  const bool read_c = ep.beta != 0.0f;
  float c[16], bs[16];
  int off[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int col = col0 + 8 * q;
    if constexpr (WIDE) {
      const int o = col < out_cols ? (row * ldc + col) * esz : (int)kDropped;
      off[4 * q] = o;
      if (read_c) {
        if constexpr (F32) {
          const v4i cv = __builtin_amdgcn_raw_buffer_load_b128(ro, o, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) c[4 * q + e] = __int_as_float(cv[e]);
        } else {
          const v2i cv = __builtin_amdgcn_raw_buffer_load_b64(ro, o, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w = (uint32_t)cv[e >> 1];
            c[4 * q + e] = __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) c[4 * q + e] = 0.0f;
      }
      if (ep.has_bias) {
        const v4i bv = __builtin_amdgcn_raw_buffer_load_b128(ep.bias, col * 4, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e) bs[4 * q + e] = __int_as_float(bv[e]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) bs[4 * q + e] = 0.0f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int cc = col + e;
        const int o = cc < out_cols ? (row * ldc + cc) * esz : (int)kDropped;
        off[4 * q + e] = o;
        c[4 * q + e] = 0.0f;
        if (read_c) {
          if constexpr (F32)
            c[4 * q + e] = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(ro, o, 0, 0));
          else
            c[4 * q + e] = __uint_as_float(
                (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(ro, o, 0, 0) << 16);
        }
        bs[4 * q + e] =
            ep.has_bias ? __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(ep.bias, cc * 4, 0, 0))
                        : 0.0f;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      y[e] = ep.alpha * acc[4 * q + e] + ep.beta * c[4 * q + e] + bs[4 * q + e];
    if constexpr (WIDE) {
      if constexpr (F32) {
        __builtin_amdgcn_raw_buffer_store_b128(
            (v4i){__float_as_int(y[0]), __float_as_int(y[1]), __float_as_int(y[2]),
                  __float_as_int(y[3])},
            ro, off[4 * q], 0, 0);
      } else {
        const int lo = __builtin_bit_cast(int, __builtin_convertvector((v2f){y[0], y[1]}, v2bf));
        const int hi = __builtin_bit_cast(int, __builtin_convertvector((v2f){y[2], y[3]}, v2bf));
        __builtin_amdgcn_raw_buffer_store_b64((v2i){lo, hi}, ro, off[4 * q], 0, 0);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if constexpr (F32)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(y[e]), ro, off[4 * q + e], 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_rne(y[e]), ro,
                                                off[4 * q + e], 0, 0);
      }
    }
  }
}

// One block at a time: each block's accumulators are copied out right before
// its loads and stores (scheduling fences keep the compiler from copying the
// whole tile out of the accumulators at once).
template <bool WIDE, bool F32>
__device__ __forceinline__ void store_tile_ex(const v16f (&acc)[4][4], __amdgpu_buffer_rsrc_t ro,
                                              int ldc, int row, int col, int out_cols,
                                              const EpiTerms& ep) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      v16f y = acc[i][j];
      asm volatile("" : "+v"(y));
      store_block_ex<WIDE, F32>(y, ro, ldc, row + 32 * i, col + 32 * j, out_cols, ep);
      __builtin_amdgcn_sched_barrier(0);
    }
}

}  // namespace bsg

#endif  // BSG_STORE_TILE_H
