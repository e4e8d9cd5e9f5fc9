// Grouped MXFP8 GEMM on gfx950 scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4,
// E4M3 x E4M3 with one E8M0 scale per 32 elements of each operand), FP32
// accumulation, one persistent launch over all groups.
//
// "gemm.py", grouped_gemm: fprop contracts the last dims of a ragged lhs
// [sum m_g, K] and an rhs [G, N, K] (output rows follow the lhs groups); wgrad
// contracts over the ragged token dim, giving a uniform [G, N, K] output.
// "[JAX] MXFP8 Grouped Quant+GEMM": a single graph-safe grouped GEMM whose
// per-group operand and scale pointers follow from the device offsets (scale
// offset = data offset / 32).
//
// Both modes reduce to one "both operands K-major" tile kernel:
//   FPROP_TN:  A = X rows of group g [m_g, K],   B = W[g] [N, K]
//   WGRAD_NT:  A = dY^T of group g [N, m~_g],    B = X^T of group g [K, m~_g]
// (the columnwise copies are already transposed and 128-padded with zeros).
//
// Tile 256 x 256 x 128, 4 wavefronts (one per SIMD) in a 2 x 2 grid, each
// owning 128 x 128 of the output as 4 x 4 MFMA blocks of 32 x 32 (256
// accumulator registers per lane).  Operands are staged through LDS
// in 128-byte rows whose 16-byte chunks are XOR-swizzled by (row / 2) % 8 so
// that the MFMA fragment reads (32 rows, same chunk) spread over all banks.
// Global loads of K-step k+1 are issued before the MFMAs of step k and written
// to the other LDS buffer afterwards (one barrier per K-step).
//
// Scaled-MFMA operand layout (measured on the device): lane l holds row l % 32;
// its 32 bytes are two 16-byte chunks covering K = 32c + 16 (l / 32) + [0, 16),
// c = 0, 1; the lane's scale byte (picked by op_sel) scales K-block l / 32 of
// its row.  With the quantizer's b0, b2, b1, b3 order, half h of a row's scale
// dword holds the bytes of blocks h and 2 + h: op_sel 0 and 1 of the two MFMAs
// of a 128-wide K-step.
#include "bsg_internal.h"

namespace bsg {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 128;
constexpr int kThreads = 256;

struct MxArgs {
  const uint8_t* a;
  const uint8_t* as;
  const uint8_t* b;
  const uint8_t* bs;
  const int64_t* offsets;
  int64_t rows_cap;
  int64_t n;
  int64_t k;
  void* out;
  uint32_t* status;
  int G;
  int out_f32;
};

struct TileDesc {
  const uint8_t* a;   // row 0 of the A tile, K offset 0
  const uint8_t* as;  // its scale row 0
  const uint8_t* b;
  const uint8_t* bs;
  int64_t lda, ldb;   // bytes per data row
  int64_t ldas, ldbs; // bytes per scale row
  int a_rows, b_rows; // valid rows (rows past them load as zeros)
  int64_t kl;         // contraction length, multiple of BK
  char* out;          // element (0, 0) of the output tile
  int64_t ldc;        // output row stride in elements
  int out_rows, out_cols;
};

struct Smem {
  uint8_t a[2][BM * BK];
  uint8_t b[2][BN * BK];
  uint32_t sa[2][BM];
  uint32_t sb[2][BN];
  int64_t off[kMaxGroups + 1];
  int32_t cnt[kMaxGroups];
  int32_t pre[kMaxGroups + 1];
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ ((row >> 1) & 7)) << 4);
}

struct Prefetch {
  v4i a[8];
  v4i b[8];
  int sa, sb;
};

// Raw buffer descriptor over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

struct TileRsrc {
  __amdgpu_buffer_rsrc_t a, b, as, bs;
};

__device__ __forceinline__ TileRsrc tile_rsrc(const TileDesc& t) {
  TileRsrc r;
  r.a = make_rsrc(t.a, (int64_t)t.a_rows * t.lda);
  r.b = make_rsrc(t.b, (int64_t)t.b_rows * t.ldb);
  r.as = make_rsrc(t.as, (int64_t)t.a_rows * t.ldas);
  r.bs = make_rsrc(t.bs, (int64_t)t.b_rows * t.ldbs);
  return r;
}

// Thread tid loads 16-byte chunk (tid % 8) of rows tid / 8 + 32 p, p = 0..7, of
// both operand tiles, and the scale dwords of row tid.  Rows past the valid
// ones read as zeros (buffer range check).
__device__ __forceinline__ void load_step(const TileDesc& t, const TileRsrc& rs, int64_t kt,
                                          int tid, Prefetch& pf) {
  const int row = tid >> 3, ch = tid & 7;
  const int koff = (int)(kt * BK) + ch * 16;
  const int oa = row * (int)t.lda + koff;
  const int ob = row * (int)t.ldb + koff;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    pf.a[p] = __builtin_amdgcn_raw_buffer_load_b128(rs.a, oa, 32 * p * (int)t.lda, 0);
    pf.b[p] = __builtin_amdgcn_raw_buffer_load_b128(rs.b, ob, 32 * p * (int)t.ldb, 0);
  }
  pf.sa = __builtin_amdgcn_raw_buffer_load_b32(rs.as, tid * (int)t.ldas + (int)kt * (BK / 32), 0, 0);
  pf.sb = __builtin_amdgcn_raw_buffer_load_b32(rs.bs, tid * (int)t.ldbs + (int)kt * (BK / 32), 0, 0);
}

__device__ __forceinline__ void store_step(Smem& sm, int st, int tid, const Prefetch& pf) {
  const int row = tid >> 3, ch = tid & 7;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    *reinterpret_cast<v4i*>(&sm.a[st][swz(row + 32 * p, ch)]) = pf.a[p];
    *reinterpret_cast<v4i*>(&sm.b[st][swz(row + 32 * p, ch)]) = pf.b[p];
  }
  sm.sa[st][tid] = (uint32_t)pf.sa;
  sm.sb[st][tid] = (uint32_t)pf.sb;
}

__device__ __forceinline__ v8i frag(const uint8_t* base, int row, int c0, int c1) {
  const v4i lo = *reinterpret_cast<const v4i*>(base + swz(row, c0));
  const v4i hi = *reinterpret_cast<const v4i*>(base + swz(row, c1));
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

template <int S>
__device__ __forceinline__ void mfma_substep(const Smem& sm, int st, int wm, int wn, int r, int h,
                                             const int (&sa)[4], const int (&sb)[4],
                                             v16f (&acc)[4][4]) {
  v8i af[4], bf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) af[i] = frag(sm.a[st], wm * 128 + 32 * i + r, 4 * S + h, 4 * S + 2 + h);
#pragma unroll
  for (int j = 0; j < 4; ++j) bf[j] = frag(sm.b[st], wn * 128 + 32 * j + r, 4 * S + h, 4 * S + 2 + h);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, S,
                                                                  sa[i], S, sb[j]);
}

// Stores one 32 x 32 accumulator block: lane (column r, half h), register v
// holds row 8 (v / 4) + 4 h + v % 4.  `ro` covers the tile's valid rows, so
// stores to rows past them are dropped by the buffer range check; columns are
// masked here.
__device__ __forceinline__ void store_block(const v16f& acc, __amdgpu_buffer_rsrc_t ro, int ldc,
                                            int row0, int col, int h, int out_cols, int out_f32) {
  if (col >= out_cols) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int row = row0 + 8 * (v >> 2) + 4 * h + (v & 3);
    const int idx = row * ldc + col;
    if (out_f32)
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(acc[v]), ro, idx * 4, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_rne(acc[v]), ro, idx * 2, 0, 0);
  }
}

__device__ void run_tile(Smem& sm, const TileDesc& t, int out_f32) {
  // opaque per-tile copy of the thread index: keeps the compiler from hoisting
  // every LDS / global offset of the tile body out of the persistent tile loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int r = lane & 31, h = lane >> 5;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  const int64_t nk = t.kl / BK;
  Prefetch pf;
  const TileRsrc rs = tile_rsrc(t);
  if (nk > 0) {
    load_step(t, rs, 0, tid, pf);
    store_step(sm, 0, tid, pf);
  }
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int st = (int)(kt & 1);
    if (kt + 1 < nk) load_step(t, rs, kt + 1, tid, pf);
    int sa[4], sb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = (int)((sm.sa[st][wm * 128 + 32 * i + r] >> (16 * h)) & 0xffffu);
#pragma unroll
    for (int j = 0; j < 4; ++j) sb[j] = (int)((sm.sb[st][wn * 128 + 32 * j + r] >> (16 * h)) & 0xffffu);
    mfma_substep<0>(sm, st, wm, wn, r, h, sa, sb, acc);
    mfma_substep<1>(sm, st, wm, wn, r, h, sa, sb, acc);
    if (kt + 1 < nk) store_step(sm, st ^ 1, tid, pf);
    __syncthreads();
  }

  const int esz = out_f32 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(t.out, (int64_t)t.out_rows * t.ldc * esz);
  // opaque copy of the row stride: keeps the compiler from hoisting all 256
  // store offsets out of the persistent tile loop into registers
  int ldc = (int)t.ldc;
  asm volatile("" : "+s"(ldc));
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      store_block(acc[i][j], ro, ldc, wm * 128 + 32 * i, wn * 128 + 32 * j + r, h,
                  t.out_cols, out_f32);
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void mx_gemm_kernel(MxArgs p) {
  __shared__ Smem sm;
  const int G = p.G;
  const int tid = threadIdx.x;
  uint32_t* status = blockIdx.x == 0 ? p.status : nullptr;
  load_offsets_clamped(p.offsets, G, p.rows_cap, sm.off, status);
  const int64_t ntn = (p.n + BN - 1) / BN;
  for (int g = tid; g < G; g += kThreads) {
    int64_t c;
    if (MODE == 0) {
      c = ((group_extent(sm.off, g) + BM - 1) / BM) * ntn;
    } else {
      const int64_t mp = group_extent(sm.off, g);
      if ((sm.off[g] % kColPad) != 0 || (mp % kColPad) != 0) dev_status_or(status, kDevBadPadding);
      c = ((p.n + BM - 1) / BM) * ((p.k + BN - 1) / BN);
    }
    sm.cnt[g] = (int32_t)c;
  }
  __syncthreads();
  wave0_exclusive_scan(sm.cnt, G, sm.pre);
  __syncthreads();
  const int total = sm.pre[G];
  const int out_elem = p.out_f32 ? 4 : 2;

  for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int g = find_group(sm.pre, G, tile);
    const int local = tile - sm.pre[g];
    TileDesc t;
    if (MODE == 0) {
      const int64_t m = group_extent(sm.off, g);
      const int64_t mtiles = (m + BM - 1) / BM;
      const int64_t mt = local % mtiles, nt = local / mtiles;
      const int64_t row0 = sm.off[g] + mt * BM;
      const int64_t n0 = nt * BN;
      const int64_t ks = ((p.k / 32 + 3) / 4) * 4;
      t.a = p.a + row0 * p.k;
      t.as = p.as + row0 * ks;
      t.b = p.b + ((int64_t)g * p.n + n0) * p.k;
      t.bs = p.bs + ((int64_t)g * p.n + n0) * ks;
      t.lda = t.ldb = p.k;
      t.ldas = t.ldbs = ks;
      const int64_t rv = sm.off[g] + m - row0;
      t.a_rows = (int)(rv < BM ? rv : BM);
      const int64_t cv = p.n - n0;
      t.b_rows = (int)(cv < BN ? cv : BN);
      t.kl = p.k;
      t.out = reinterpret_cast<char*>(p.out) + (row0 * p.n + n0) * out_elem;
      t.ldc = p.n;
      t.out_rows = t.a_rows;
      t.out_cols = t.b_rows;
    } else {
      const int64_t mp = group_extent(sm.off, g);
      const bool ok = (sm.off[g] % kColPad) == 0 && (mp % kColPad) == 0;
      const int64_t ntk = (p.k + BN - 1) / BN;
      const int64_t it = local / ntk, jt = local % ntk;
      const int64_t n0 = it * BM, c0 = jt * BN;
      const int64_t t0 = sm.off[g];
      t.a = p.a + t0 * p.n + n0 * mp;
      t.as = p.as + t0 * p.n / 32 + n0 * (mp / 32);
      t.b = p.b + t0 * p.k + c0 * mp;
      t.bs = p.bs + t0 * p.k / 32 + c0 * (mp / 32);
      t.lda = t.ldb = mp;
      t.ldas = t.ldbs = mp / 32;
      const int64_t rv = p.n - n0, cv = p.k - c0;
      t.a_rows = (int)(rv < BM ? rv : BM);
      t.b_rows = (int)(cv < BN ? cv : BN);
      t.kl = ok ? mp : 0;
      t.out = reinterpret_cast<char*>(p.out) + (((int64_t)g * p.n + n0) * p.k + c0) * out_elem;
      t.ldc = p.k;
      t.out_rows = t.a_rows;
      t.out_cols = t.b_rows;
    }
    run_tile(sm, t, p.out_f32);
  }
}

}  // namespace

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
      cu = 256;
    cached[dev] = cu;
  }
  return cached[dev];
}

hipError_t launch_gemm_mxfp8(int mode, int G, const uint8_t* a, const uint8_t* a_scales,
                             const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                             int64_t rows_cap, int64_t n, int64_t k, void* out, int out_f32,
                             uint32_t* status, hipStream_t stream) {
  MxArgs p{a, a_scales, b, b_scales, offsets, rows_cap, n, k, out, status, G, out_f32};
  // upper bound of the tile count from host-known shapes
  int64_t bound;
  if (mode == 0) bound = ((rows_cap + BM - 1) / BM + G) * ((n + BN - 1) / BN);
  else bound = (int64_t)G * ((n + BM - 1) / BM) * ((k + BN - 1) / BN);
  int64_t grid = device_cu_count();
  if (bound < grid) grid = bound;
  if (grid <= 0) return hipSuccess;
  if (mode == 0)
    hipLaunchKernelGGL(mx_gemm_kernel<0>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(mx_gemm_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace bsg
