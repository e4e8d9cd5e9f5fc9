// Row-scaled NVFP4 grouped GEMM with the outer-scale epilogue.
//
// "[Common][PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM": the
// per-row (activation) and per-column (weight) FP32 outer scales are
// neutralized in the GEMM, the product is accumulated in FP32 (the "FP32
// scratch"), and the outer scales are applied afterwards over each group's own
// live rows and own output width (the Greptile finding on differing widths and
// capacity rows, and the commits that fix it).
//
//   S[r, n] = sum_k e2m1(A)[r,k] sA[r,k/16] * e2m1(B_g)[n,k] sB_g[n,k/16]
//   Y[r, n] = (S[r, n] * a_outer[r]) * b_outer_g[n]
//
// gfx950's scaled MFMA takes only power-of-two (E8M0) scales per 32 elements,
// and E2M1 x E4M3 needs up to 6 significant bits, so no FP8/FP6/FP4 MFMA input
// holds it exactly.  Each element is instead decoded while it is staged into
// LDS: E2M1 -> fp32 (hardware convert, unit scale), times its decoded E4M3 block
// scale (exact in fp32), truncated to bf16 (exact: at most 6 significant bits,
// magnitudes in [2^-10, 2688]).  The product then runs on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with FP32 accumulation: exact products, FP32 sums.
//
// Tile 256 x 256 x 64, 4 wavefronts (2 x 2), 128 x 128 per wavefront; LDS holds
// bf16 rows of 128 bytes with the same XOR chunk swizzle as the MXFP8 GEMM.
#include "bsg_internal.h"

namespace bsg {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;          // elements per K-step (32 bytes of E2M1 per row)
constexpr int kThreads = 256;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));


struct NvArgs {
  const uint8_t* a;
  const uint8_t* as;
  const float* aout;
  const int64_t* offsets;
  int64_t rows_cap;
  int64_t k;
  const uint8_t* b;
  const uint8_t* bs;
  const float* bout;
  void* out;
  int64_t ld_out;
  float* scratch;
  uint32_t* status;
  int G;
  int out_f32;
  NvGroupTable tab;
};

struct Smem {
  uint8_t a[2][BM * 128];
  uint8_t b[2][BN * 128];
  float aout[BM];
  float bout[BN];
  int64_t off[kMaxGroups + 1];
  int32_t cnt[kMaxGroups];
  int32_t pre[kMaxGroups + 1];
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (c & 0x80u) ? -mag : mag;
}

// One byte (two E2M1 nibbles, low nibble first) of dword w, times sd, as a
// packed bf16 pair (low element in the low half).
template <int SEL>
__device__ __forceinline__ uint32_t dq_pair(uint32_t w, float sd) {
  const v2f f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
  const uint32_t lo = __float_as_uint(f[0] * sd);
  const uint32_t hi = __float_as_uint(f[1] * sd);
  return __builtin_amdgcn_perm(hi, lo, 0x07060302u);
}

// 16 bytes (32 elements, two 16-element blocks with scales s0, s1) -> 32 bf16.
__device__ __forceinline__ void dq32(const v4i& d, float s0, float s1, v4i (&o)[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = (uint32_t)d[q];
    const float sd = q < 2 ? s0 : s1;
    o[q][0] = (int)dq_pair<0>(w, sd);
    o[q][1] = (int)dq_pair<1>(w, sd);
    o[q][2] = (int)dq_pair<2>(w, sd);
    o[q][3] = (int)dq_pair<3>(w, sd);
  }
}

struct Raw {
  v4i a[2], b[2];
  int sa, sb;
};

struct TileDesc {
  const uint8_t* a;
  const uint8_t* as;
  const uint8_t* b;
  const uint8_t* bs;
  int64_t lda, ldas;  // bytes per row: k/2 and k/16
  int a_rows, b_rows;
  int64_t kl;
};

// Thread t loads row t of both operand tiles for one K-step: 32 bytes of E2M1
// and 4 scale bytes each.  Rows past the valid ones read as zeros.
__device__ __forceinline__ void load_raw(const TileDesc& t, __amdgpu_buffer_rsrc_t ra,
                                         __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rsa,
                                         __amdgpu_buffer_rsrc_t rsb, int64_t kt, int tid, Raw& x) {
  const int od = tid * (int)t.lda + (int)kt * (BK / 2);
  x.a[0] = __builtin_amdgcn_raw_buffer_load_b128(ra, od, 0, 0);
  x.a[1] = __builtin_amdgcn_raw_buffer_load_b128(ra, od + 16, 0, 0);
  x.b[0] = __builtin_amdgcn_raw_buffer_load_b128(rb, od, 0, 0);
  x.b[1] = __builtin_amdgcn_raw_buffer_load_b128(rb, od + 16, 0, 0);
  const int os = tid * (int)t.ldas + (int)kt * (BK / 16);
  x.sa = __builtin_amdgcn_raw_buffer_load_b32(rsa, os, 0, 0);
  x.sb = __builtin_amdgcn_raw_buffer_load_b32(rsb, os, 0, 0);
}

__device__ __forceinline__ void dequant_store(uint8_t* lds, int row, const v4i (&d)[2], int s) {
  const uint32_t sc = (uint32_t)s;
  v4i o[4];
  dq32(d[0], e4m3_decode(sc & 0xffu), e4m3_decode((sc >> 8) & 0xffu), o);
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<v4i*>(lds + swz(row, q)) = o[q];
  dq32(d[1], e4m3_decode((sc >> 16) & 0xffu), e4m3_decode(sc >> 24), o);
#pragma unroll
  for (int q = 0; q < 4; ++q) *reinterpret_cast<v4i*>(lds + swz(row, 4 + q)) = o[q];
}

template <int S>
__device__ __forceinline__ void mfma_substep(const Smem& sm, int st, int wm, int wn, int r, int h,
                                             v16f (&acc)[4][4]) {
  v8bf af[4], bf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    af[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(
                                         sm.a[st] + swz(wm * 128 + 32 * i + r, 2 * S + h)));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    bf[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4i*>(
                                         sm.b[st] + swz(wn * 128 + 32 * j + r, 2 * S + h)));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

__global__ __launch_bounds__(kThreads) void nv_gemm_kernel(NvArgs p) {
  __shared__ Smem sm;
  const int G = p.G;
  const int tid = threadIdx.x;
  uint32_t* status = blockIdx.x == 0 ? p.status : nullptr;
  load_offsets_clamped(p.offsets, G, p.rows_cap, sm.off, status);
  for (int g = tid; g < G; g += kThreads) {
    const int64_t m = group_extent(sm.off, g);
    const int64_t ng = p.tab.n[g];
    sm.cnt[g] = (int32_t)(((m + BM - 1) / BM) * ((ng + BN - 1) / BN));
  }
  __syncthreads();
  wave0_exclusive_scan(sm.cnt, G, sm.pre);
  __syncthreads();
  const int total = sm.pre[G];

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    // opaque per-tile copy of the thread index: keeps the compiler from
    // hoisting every LDS / global offset of the tile body out of the tile loop
    int tix = tid;
    asm volatile("" : "+v"(tix));
    const int lane = tix & 63, w = tix >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int r = lane & 31, h = lane >> 5;
    const int g = find_group(sm.pre, G, tile);
    const int local = tile - sm.pre[g];
    const int64_t m = group_extent(sm.off, g);
    const int64_t ng = p.tab.n[g];
    const int64_t mtiles = (m + BM - 1) / BM;
    const int64_t mt = local % mtiles, nt = local / mtiles;
    const int64_t row0 = sm.off[g] + mt * BM;
    const int64_t n0 = nt * BN;
    const int64_t brow0 = p.tab.brow[g] + n0;
    TileDesc t;
    t.lda = p.k / 2;
    t.ldas = p.k / 16;
    t.a = p.a + row0 * t.lda;
    t.as = p.as + row0 * t.ldas;
    t.b = p.b + brow0 * t.lda;
    t.bs = p.bs + brow0 * t.ldas;
    const int64_t rv = sm.off[g] + m - row0, cv = ng - n0;
    t.a_rows = (int)(rv < BM ? rv : BM);
    t.b_rows = (int)(cv < BN ? cv : BN);
    t.kl = p.k;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(t.a, (int64_t)t.a_rows * t.lda);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(t.b, (int64_t)t.b_rows * t.lda);
    const __amdgpu_buffer_rsrc_t rsa = make_rsrc(t.as, (int64_t)t.a_rows * t.ldas);
    const __amdgpu_buffer_rsrc_t rsb = make_rsrc(t.bs, (int64_t)t.b_rows * t.ldas);

    // outer scales of this tile's rows and columns, for the epilogue
    sm.aout[tix] = tix < t.a_rows ? p.aout[row0 + tix] : 0.0f;
    sm.bout[tix] = tix < t.b_rows ? p.bout[brow0 + tix] : 0.0f;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    const int64_t nk = t.kl / BK;
    Raw x;
    if (nk > 0) {
      load_raw(t, ra, rb, rsa, rsb, 0, tix, x);
      dequant_store(sm.a[0], tix, x.a, x.sa);
      dequant_store(sm.b[0], tix, x.b, x.sb);
    }
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      const int st = (int)(kt & 1);
      if (kt + 1 < nk) load_raw(t, ra, rb, rsa, rsb, kt + 1, tix, x);
      mfma_substep<0>(sm, st, wm, wn, r, h, acc);
      mfma_substep<1>(sm, st, wm, wn, r, h, acc);
      mfma_substep<2>(sm, st, wm, wn, r, h, acc);
      mfma_substep<3>(sm, st, wm, wn, r, h, acc);
      if (kt + 1 < nk) {
        dequant_store(sm.a[st ^ 1], tix, x.a, x.sa);
        dequant_store(sm.b[st ^ 1], tix, x.b, x.sb);
      }
      __syncthreads();
    }

    // epilogue: S -> (S * a_outer) * b_outer, or S itself into the scratch
    const bool fused = p.scratch == nullptr;
    const int esz = (fused && !p.out_f32) ? 2 : 4;
    char* obase = fused ? reinterpret_cast<char*>(p.out) : reinterpret_cast<char*>(p.scratch);
    obase += (row0 * p.ld_out + n0) * esz;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(obase, (int64_t)t.a_rows * p.ld_out * esz);
    int ldc = (int)p.ld_out;
    asm volatile("" : "+s"(ldc));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = wn * 128 + 32 * j + r;
        if (col >= t.b_rows) continue;
        const float bo = sm.bout[col];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * 128 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          const int idx = row * ldc + col;
          float y = acc[i][j][v];
          if (fused) {
            y = (y * sm.aout[row < BM ? row : 0]) * bo;
            if (p.out_f32)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(y), ro, idx * 4, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_rne(y), ro, idx * 2,
                                                    0, 0);
          } else {
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(y), ro, idx * 4, 0, 0);
          }
        }
      }
    __syncthreads();  // aout / bout are rewritten by the next tile
  }
}

// Unfused second step: Y[r, n] = (S[r, n] * a_outer[r]) * b_outer_g[n] for the
// live rows r of group g and n < N_g, one block per row.
__global__ __launch_bounds__(256) void nv_postscale_kernel(const float* __restrict__ scratch,
                                                           const float* __restrict__ aout,
                                                           const float* __restrict__ bout,
                                                           const int64_t* __restrict__ offsets,
                                                           int64_t rows_cap, int G, void* out,
                                                           int64_t ld_out, int out_f32,
                                                           NvGroupTable tab) {
  __shared__ int64_t s_off[kMaxGroups + 1];
  load_offsets_clamped(offsets, G, rows_cap, s_off, nullptr);
  const int64_t row = blockIdx.x;
  if (row >= s_off[G]) return;
  int lo = 0, hi = G - 1;  // group: largest g with s_off[g] <= row and a non-empty extent
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int ng = tab.n[g];
  const float ao = aout[row];
  const float* bo = bout + tab.brow[g];
  for (int n = threadIdx.x; n < ng; n += blockDim.x) {
    const float y = (scratch[row * ld_out + n] * ao) * bo[n];
    if (out_f32)
      reinterpret_cast<float*>(out)[row * ld_out + n] = y;
    else
      reinterpret_cast<uint16_t*>(out)[row * ld_out + n] = (uint16_t)f32_to_bf16_rne(y);
  }
}

}  // namespace

hipError_t launch_gemm_nvfp4(int G, const uint8_t* a, const uint8_t* a_scales,
                             const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                             int64_t k, const uint8_t* b, const uint8_t* b_scales,
                             const float* b_outer, const NvGroupTable& table, int max_n,
                             void* out, int64_t ld_out, int out_f32, float* scratch,
                             uint32_t* status, hipStream_t stream) {
  NvArgs p;
  p.a = a; p.as = a_scales; p.aout = a_outer; p.offsets = offsets; p.rows_cap = rows_cap; p.k = k;
  p.b = b; p.bs = b_scales; p.bout = b_outer; p.out = out; p.ld_out = ld_out; p.scratch = scratch;
  p.status = status; p.G = G; p.out_f32 = out_f32; p.tab = table;
  const int64_t bound = ((rows_cap + BM - 1) / BM + G) * ((max_n + BN - 1) / BN);
  int64_t grid = device_cu_count();
  if (bound < grid) grid = bound;
  if (grid > 0) {
    hipLaunchKernelGGL(nv_gemm_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (scratch != nullptr && rows_cap > 0) {
    hipLaunchKernelGGL(nv_postscale_kernel, dim3((unsigned)rows_cap), dim3(256), 0, stream,
                       scratch, a_outer, b_outer, offsets, rows_cap, G, out, ld_out, out_f32,
                       table);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace bsg
