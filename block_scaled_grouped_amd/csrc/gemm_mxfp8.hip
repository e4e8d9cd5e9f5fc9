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
// Tile 256 x 256, K-steps of 64 (one MFMA deep), 4 wavefronts (one per SIMD)
// in a 2 x 2 grid, each owning 128 x 128 of the output as 4 x 4 MFMA blocks of
// 32 x 32 (256 accumulator registers per lane).
//
// A and the scales go global -> LDS by the buffer unit directly (LDS-DMA: lane
// l of a load lands at LDS base + 16 l, so a swizzled layout is made by
// permuting each lane's source address); B goes through registers (ordinary
// buffer loads issued a pair ahead, each written to its swizzled LDS slot one
// K-step later), which splits a CU's copy work between the two paths.  An LDS
// buffer holds two K-steps: 128-byte rows, so every copy request is one whole
// 128-byte line, plus the one scale dword per row that covers those 128 K.  Two buffers: while pair p is consumed from one,
// pair p + 1 lands in the other, and the copies of pair p + 2 are issued as soon
// as pair p's last fragments are in registers.  16-byte chunk c of row r sits
// in slot c ^ ((r / 2) % 8), which spreads the MFMA fragment reads (32 rows,
// same chunk) over all banks.  One barrier per pair; the schedule of a K-step
// is written out MFMA by MFMA (copy issues and next-step fragment reads placed
// between them) and fenced so the compiler keeps it.
//
// Tiles are handed out XCD-aware: workgroup b runs on XCD b % 8, and the 32
// workgroups of one XCD take a 4 x 8 block of output tiles of one group at a
// time, so the A rows and B columns they stream are shared through that XCD's
// L2.
//
// Scaled-MFMA operand layout (measured on the device): lane l holds row l % 32;
// its 32 bytes are two 16-byte chunks covering K = 32c + 16 (l / 32) + [0, 16),
// c = 0, 1; the lane's scale byte (picked by op_sel) scales K-block l / 32 of
// its row.  With the quantizer's b0, b2, b1, b3 order, half h of a row's scale
// dword (one dword per 128 K) holds the bytes of blocks h and 2 + h: op_sel 0
// for the first 64-wide K-step of the dword and op_sel 1 for the second.
#include <utility>

#include "bsg_internal.h"
#include "lds_dma.h"
#include "store_tile.h"

namespace bsg {

namespace {

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(<N-1>), so every
// register-array index in the K-step schedule is a constant.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;                 // bytes (= E4M3 elements) per row per K-step
constexpr int kPairK = 2 * BK;         // bytes per row per LDS buffer: two K-steps,
                                       // one scale word (one full 128-byte line)
constexpr int kThreads = 256;
constexpr int kBufs = 2;
constexpr int kTileA = BM * kPairK;    // 32 KiB
constexpr int kTileB = BN * kPairK;
constexpr int kBufBytes = kTileA + kTileB + 4 * BM + 4 * BN;
constexpr int kDmaPerPair = 18;        // per wave and pair: 8 A, 8 B, 1 A-scale, 1 B-scale
constexpr int kLdsDmaPerPair = 10;     // of which copied global -> LDS directly: A, scales
constexpr int kRegPerPair = 8;         // and global -> registers -> LDS: B
constexpr int kBarrierAfter = 2;       // MFMA index of a pair's second step after which it
                                       // waits + barriers
constexpr int kSuperM = 4, kSuperN = 8;  // tile block one XCD works on

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
  const float* alpha;  // [G] or null (1): epilogue terms, used by the EX kernels
  const float* beta;   // [G] or null (0)
  const float* bias;   // [G, output columns] or null
  char* ws;            // split workspace (see below) or null: no split
};

// Split of the last round.  With T output tiles and a grid of P workgroups,
// the last round holds L = T mod P tiles and leaves P - L workgroups idle.
// Given a workspace, each of those L tiles is split along the contraction into
// S <= min(P / L, kSplitMax) parts of whole K-step pairs (at least two each);
// workgroup L * S' + s of the last round takes part s of tile L' and writes its
// FP32 accumulators to the workspace, and mx_split_reduce_kernel, launched after
// the GEMM on the same stream, sums each tile's parts in the order s = 0, 1, ..
// (so the result does not depend on which part finished first) and stores the
// tile.  Workspace layout: a header (L, S), one record per split tile (where
// its output goes), then the parts, kPartBytes each, the accumulators of each
// wave's 4 x 4 blocks lane by lane.
constexpr int kSplitMax = 8;
constexpr int64_t kWsHeader = 16384;
constexpr int64_t kPartBytes = (int64_t)BM * BN * 4;
constexpr int kMaxSplitTiles = (int)((kWsHeader - 64) / 32);

struct SplitRecord {
  int64_t out_off;  // byte offset of the tile's first output element
  int32_t out_rows, out_cols, ldc, pad;
};

struct TileDesc {
  const uint8_t* a;   // row 0 of the A tile, K offset 0
  const uint8_t* as;  // scale word (K-group 0, tile row 0)
  const uint8_t* b;
  const uint8_t* bs;
  int64_t lda, ldb;   // bytes per data row
  int64_t sqa, sqb;   // bytes between the scale words of consecutive 128-wide K-groups
  int64_t as_bytes, bs_bytes;  // scale bytes readable from `as` / `bs`
  int a_rows, b_rows; // valid rows (rows past them load as zeros)
  int64_t kl;         // contraction length, multiple of 32; data past it (the last
                      // pair's tail) is copied as zeros
  char* out;          // element (0, 0) of the output tile
  int64_t ldc;        // output row stride in elements
  int out_rows, out_cols;
  float alpha, beta;  // the group's epilogue terms (EX kernels)
  const float* bias;  // the group's bias at the tile's first column, or null
};

struct Sched {
  int64_t off[kMaxGroups + 1];
  int32_t cnt[kMaxGroups];
  int32_t pre[kMaxGroups + 1];
};

typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ v4i lds_read16(uint32_t addr) {
  return *reinterpret_cast<const lds_v4i*>((size_t)addr);
}
__device__ __forceinline__ uint32_t lds_read4(uint32_t addr) {
  return *reinterpret_cast<const lds_u32*>((size_t)addr);
}
template <typename T>
__device__ __forceinline__ uint32_t lds_offset(T* shared_ptr) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) T*)(shared_ptr);
}

// Buffer s: A tile, B tile, A scale dwords, B scale dwords.
__device__ __forceinline__ uint32_t st_a(uint32_t base, int s) { return base + s * kBufBytes; }
__device__ __forceinline__ uint32_t st_b(uint32_t base, int s) { return st_a(base, s) + kTileA; }
__device__ __forceinline__ uint32_t st_sa(uint32_t base, int s) { return st_b(base, s) + kTileB; }
__device__ __forceinline__ uint32_t st_sb(uint32_t base, int s) { return st_sa(base, s) + 4 * BM; }

// Raw buffer descriptor over [base, base + bytes): accesses past the end are
// dropped (loads return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Vector-memory operations complete in issue order, so "at most N
// outstanding" means everything but the N most recent has landed.  Also waits
// for this wave's LDS reads, then joins the barrier: afterwards the stage whose
// copies were older than the last N is complete for every wave, and no wave
// still reads the stage that the next copies overwrite.
template <int N>
__device__ __forceinline__ void wait_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// A wavefront's share of one pair's copies.  Wave w fills rows
// [64 w, 64 w + 64) of both operand tiles, eight 128-byte rows (1 KiB) per
// load: in load q lane l writes row 64 w + 8 q + l / 8, slot l % 8, which must
// hold logical chunk (l % 8) ^ ((row / 2) % 8) = (l % 8) ^ (4 (q % 2) + l / 16),
// so even and odd loads need their own lane offsets.  The scale words of its 64
// rows for the pair's 128-wide K-group are 256 contiguous bytes.
struct Dma {
  v4i ra, rb, rsa, rsb;  // descriptors (uniform)
  v4i rnone;             // zero-length descriptor: turns a copy into a no-op
  int a[2], b[2];        // lane source offsets of even / odd loads (q = 0, 1), pair 0
  int s;                 // lane scale-word offset (row 64 w + l, K-group 0)
  int lda16, ldb16;      // 16 rows of stride (uniform)
  int sqa, sqb;          // scale K-group strides (uniform)
  __amdgpu_buffer_rsrc_t rbv, rbv_none;  // B descriptors for the register path
  int bl;                // lane offset of a register-path B load (q = 0, pair 0)
  int bw[2];             // lane LDS offset of its store in the B tile, q = 0 rows, with
                         // the slot swizzle of an even / odd q
  int ldb8;              // 8 rows of B stride (uniform)
  int ka[2];             // K offset within a pair of this lane's chunk in even / odd loads
  int kb;                // the same for its register-path B loads
  int kl;                // contraction length (uniform)
};

// A lane's copy of a chunk that starts at or past the contraction end gets an
// offset past every descriptor's range, so the buffer unit returns zeros for it
// (the bytes past k in a row are the next row's, or stale bytes of rows no group
// owns, which may hold NaN codes).
__device__ __forceinline__ int k_mask(int voff, int kpos, int lim) {
  return kpos < lim ? voff : kDmaOutOfRange;
}

__device__ __forceinline__ Dma make_dma(const TileDesc& t, int w, int lane) {
  Dma d;
  d.ra = make_rsrc_words(t.a, (int64_t)t.a_rows * t.lda);
  d.rb = make_rsrc_words(t.b, (int64_t)t.b_rows * t.ldb);
  d.rsa = make_rsrc_words(t.as, t.as_bytes);
  d.rsb = make_rsrc_words(t.bs, t.bs_bytes);
  d.rnone = make_rsrc_words(t.a, 0);
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int row = 64 * w + 8 * e + (lane >> 3);
    const int c = (lane & 7) ^ (4 * e + (lane >> 4));
    d.a[e] = row * (int)t.lda + c * 16;
    d.b[e] = row * (int)t.ldb + c * 16;
    d.ka[e] = c * 16;
  }
  d.kb = (lane & 7) * 16;
  d.kl = __builtin_amdgcn_readfirstlane((int)t.kl);
  d.s = 4 * (64 * w + lane);
  d.rbv = make_rsrc(t.b, (int64_t)t.b_rows * t.ldb);
  d.rbv_none = make_rsrc(t.b, 0);
  d.bl = (64 * w + (lane >> 3)) * (int)t.ldb + (lane & 7) * 16;
#pragma unroll
  for (int e = 0; e < 2; ++e)
    d.bw[e] = (64 * w + (lane >> 3)) * kPairK + (((lane & 7) ^ (4 * e + (lane >> 4))) << 4);
  d.ldb8 = __builtin_amdgcn_readfirstlane(8 * (int)t.ldb);
  d.lda16 = __builtin_amdgcn_readfirstlane(16 * (int)t.lda);
  d.ldb16 = __builtin_amdgcn_readfirstlane(16 * (int)t.ldb);
  d.sqa = __builtin_amdgcn_readfirstlane((int)t.sqa);
  d.sqb = __builtin_amdgcn_readfirstlane((int)t.sqb);
  return d;
}

// Copy piece P (0..7 A rows, 8..15 B rows, 16 A scales, 17 B scales) of pair
// kp (K bytes [128 kp, 128 kp + 128)) into buffer s; `live` false makes it a
// no-op copy (past the last pair).
template <int P>
__device__ __forceinline__ void dma_piece(const Dma& d, uint32_t lds, int w, int s, int kp,
                                          bool live) {
  const int koff = kp * kPairK;
  const int lim = d.kl - koff;  // K bytes of this pair inside the contraction
  if constexpr (P < 8) {
    dma16(live ? d.ra : d.rnone, st_a(lds, s) + (64 * w + 8 * P) * kPairK,
          k_mask(d.a[P & 1] + (P >> 1) * d.lda16 + koff, d.ka[P & 1], lim));
  } else if constexpr (P < 16) {
    constexpr int q = P - 8;
    dma16(live ? d.rb : d.rnone, st_b(lds, s) + (64 * w + 8 * q) * kPairK,
          k_mask(d.b[q & 1] + (q >> 1) * d.ldb16 + koff, d.ka[q & 1], lim));
  } else if constexpr (P == 16) {
    dma4(live ? d.rsa : d.rnone, st_sa(lds, s) + 4 * 64 * w, d.s + kp * d.sqa);
  } else {
    dma4(live ? d.rsb : d.rnone, st_sb(lds, s) + 4 * 64 * w, d.s + kp * d.sqb);
  }
}

// Register path for the B tile (the LDS-DMA path alone cannot feed a CU at the
// rate the MFMAs consume: it sustains about one 1 KiB copy per 32 cycles).
// Load q of pair kp: lane l reads row 64 w + 8 q + l / 8, logical chunk l % 8,
// into registers; store_b writes it one K-step later to its swizzled slot.
template <int Q>
__device__ __forceinline__ void load_b(const Dma& d, int kp, bool live, v4i (&stage)[kRegPerPair]) {
  stage[Q] = __builtin_amdgcn_raw_buffer_load_b128(
      live ? d.rbv : d.rbv_none,
      k_mask(d.bl + Q * d.ldb8 + kp * kPairK, d.kb, d.kl - kp * kPairK), 0, 0);
}

template <int Q>
__device__ __forceinline__ void store_b(const Dma& d, uint32_t lds, int s,
                                        const v4i (&stage)[kRegPerPair]) {
  *reinterpret_cast<lds_v4i*>((size_t)(st_b(lds, s) + d.bw[Q & 1] + Q * 8 * kPairK)) = stage[Q];
}

// Per-lane LDS offsets of the fragment reads.  Lane (r, h) of wave (wm, wn)
// reads rows wm*128 + 32 i + r of A (wn*128 + 32 j + r of B); for K-step S of
// the pair, logical chunks 4 S + h and 4 S + 2 + h.  The swizzle term
// (row / 2) % 8 = (r / 2) % 8 is the same for all four rows of a lane, so each
// (S, part) needs one offset and the 32-row steps are immediates.  With 64-bank
// LDS, 16 lanes reading one chunk of 16 consecutive rows hit 16 distinct 16-byte
// bank groups.
struct FragOff {
  int a[2][2], b[2][2];
};

__device__ __forceinline__ FragOff make_frag_off(int wm, int wn, int r, int h) {
  FragOff f;
  const int x = (r >> 1) & 7;
#pragma unroll
  for (int S = 0; S < 2; ++S)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = ((4 * S + 2 * p + h) ^ x) << 4;
      f.a[S][p] = (wm * 128 + r) * kPairK + c;
      f.b[S][p] = (wn * 128 + r) * kPairK + c;
      asm volatile("" : "+v"(f.a[S][p]));
      asm volatile("" : "+v"(f.b[S][p]));
    }
  return f;
}

__device__ __forceinline__ v8i frag2(uint32_t base, int off0, int off1, int rowstep) {
  const v4i lo = lds_read16(base + off0 + rowstep);
  const v4i hi = lds_read16(base + off1 + rowstep);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Fragment K of the 8 K-step S of a pair needs, in the order the MFMAs
// (i-major over the 4 x 4 blocks) first use them: A0, B0, B1, B2, B3, A1, A2, A3.
template <int S, int K>
__device__ __forceinline__ void read_frag(uint32_t lds, int s, const FragOff& fo, v8i (&fa)[4],
                                          v8i (&fb)[4]) {
  if constexpr (K == 0 || K >= 5) {
    constexpr int ia = K == 0 ? 0 : K - 4;
    fa[ia] = frag2(st_a(lds, s), fo.a[S][0], fo.a[S][1], 32 * ia * kPairK);
  } else {
    constexpr int jb = K - 1;
    fb[jb] = frag2(st_b(lds, s), fo.b[S][0], fo.b[S][1], 32 * jb * kPairK);
  }
}

// This lane's two scale bytes of each of its rows (half h of the row's dword).
__device__ __forceinline__ void read_scales(uint32_t lds, int s, int wm, int wn, int r, int h,
                                            int (&sa)[4], int (&sb)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    sa[i] = (int)((lds_read4(st_sa(lds, s) + 4 * (wm * 128 + 32 * i + r)) >> (16 * h)) & 0xffffu);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    sb[j] = (int)((lds_read4(st_sb(lds, s) + 4 * (wn * 128 + 32 * j + r)) >> (16 * h)) & 0xffffu);
}

// B is the MFMA's first operand and A its second, so the accumulator of block
// (i, j) is its transpose: lane (r, h) holds output row 32 i + r, and register
// v column 32 j + 8 (v / 4) + 4 h + v % 4 -- four runs of four consecutive
// columns, which the epilogue stores as whole 8- or 16-byte pieces.
// AT: A's element format as the scaled MFMA encodes it (0 = E4M3, 1 = E5M2);
// B is always E4M3.  B is the instruction's first source, A its second.
template <int OPSEL, int M, int AT>
__device__ __forceinline__ void mfma(const v8i (&fa)[4], const v8i (&fb)[4], const int (&sa)[4],
                                     const int (&sb)[4], v16f (&acc)[4][4]) {
  constexpr int i = M >> 2, j = M & 3;
  acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fb[j], fa[i], acc[i][j], 0, AT, OPSEL,
                                                              sb[j], OPSEL, sa[i]);
  // the MFMA intrinsic has no side effects, so IR passes may sink it past the
  // schedule's fences; an opaque use of its result keeps it in place
  asm volatile("" : "+a"(acc[i][j]));
}

// The first K-step of pair kp (buffer s = kp % 2, scale byte 0 of the lane's
// half dword): its 16 MFMAs, and between them the fragments of the pair's
// second K-step (same buffer, which has landed); then, one register at a time,
// the staged B rows of pair kp + 1 into buffer s ^ 1 (free since the last
// barrier) and the loads of pair kp + 2's B rows into the freed register.
template <int AT>
__device__ __forceinline__ void step_even(uint32_t lds, const Dma& d, int s, int kp, int np,
                                          const FragOff& fo, const v8i (&fa)[4],
                                          const v8i (&fb)[4], const int (&sa)[4],
                                          const int (&sb)[4], v8i (&na)[4], v8i (&nb)[4],
                                          v4i (&stage)[kRegPerPair], v16f (&acc)[4][4]) {
  const bool live = kp + 2 < np;
  static_for<16>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    mfma<0, m, AT>(fa, fb, sa, sb, acc);
    fence();
    if constexpr (m < 8) read_frag<1, m>(lds, s, fo, na, nb);
    if constexpr (m >= 8) {
      store_b<m - 8>(d, lds, s ^ 1, stage);
      load_b<m - 8>(d, kp + 2, live, stage);
    }
    fence();
  });
}

// The second K-step of pair kp (scale byte 1).  After MFMA kBarrierAfter: wait
// until only the B loads of pair kp + 2 (the newest copies) are outstanding,
// so pair kp + 1's LDS copies have landed, and for this wave's LDS accesses
// (pair kp + 1's B rows stored); then a barrier: now buffer s ^ 1 holds pair
// kp + 1 for every wave, and buffer s (whose last fragments were read during
// the first K-step) is free.  Between the remaining MFMAs, one per slot: the
// LDS copies of pair kp + 2's A rows and scales into buffer s, and the scales
// and first-step fragments of pair kp + 1.
template <int AT>
__device__ __forceinline__ void step_odd(uint32_t lds, const Dma& d, int w, int s, int kp, int np,
                                         const FragOff& fo, int wm, int wn, int r, int h,
                                         const v8i (&fa)[4], const v8i (&fb)[4],
                                         const int (&sa)[4], const int (&sb)[4], v8i (&na)[4],
                                         v8i (&nb)[4], int (&nsa)[4], int (&nsb)[4],
                                         v16f (&acc)[4][4]) {
  static_assert(kBarrierAfter >= 0 && kBarrierAfter + kLdsDmaPerPair <= 16 &&
                    kBarrierAfter + 8 <= 16, "K-step schedule");
  const bool live = kp + 2 < np;
  static_for<16>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    mfma<1, m, AT>(fa, fb, sa, sb, acc);
    fence();
    if constexpr (m == kBarrierAfter) {
      wait_and_barrier<kRegPerPair>();
      read_scales(lds, s ^ 1, wm, wn, r, h, nsa, nsb);
    }
    if constexpr (m >= kBarrierAfter) {
      constexpr int q = m - kBarrierAfter;
      if constexpr (q < 8) dma_piece<q>(d, lds, w, s, kp + 2, live);
      else if constexpr (q < kLdsDmaPerPair) dma_piece<q + 8>(d, lds, w, s, kp + 2, live);
      if constexpr (q < 8) read_frag<0, q>(lds, s ^ 1, fo, na, nb);
    }
    fence();
  });
}

// The accumulators of one part of a split tile: unit u = 16 w + 4 i + j (wave
// w's block (i, j)) at part + 1024 u floats, lane l's 16 values at + 16 l.
__device__ __forceinline__ void store_part(float* __restrict__ part, const v16f (&acc)[4][4],
                                           int w, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float* dst = part + (int64_t)(16 * w + 4 * i + j) * 1024 + 16 * lane;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<v4f*>(dst + 4 * q) =
            v4f{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
}

// One tile: its K-loop, then the epilogue into the output, or (part != null)
// the accumulators into a part of the split workspace.
template <int AT, bool EX>
__device__ __forceinline__ void run_tile(uint32_t lds, const TileDesc& t, int out_f32,
                                         float* part) {
  // opaque per-tile copy of the thread index: keeps the compiler from hoisting
  // every LDS / global offset of the tile body out of the persistent tile loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  const int r = lane & 31, h = lane >> 5;

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

  const int np = (int)((t.kl + kPairK - 1) / kPairK);  // pairs of K-steps, the last maybe partial
  if (np > 0) {
    const Dma d = make_dma(t, w, lane);
    const FragOff fo = make_frag_off(wm, wn, r, h);
    // prologue: pair 0 into buffer 0; pair 1's A rows and scales into buffer 1
    // and its B rows into registers (stored during pair 0's first K-step);
    // wait for pair 0
    v4i stage[kRegPerPair];
    static_for<kDmaPerPair>([&](auto pc) { dma_piece<decltype(pc)::value>(d, lds, w, 0, 0, true); });
    const bool live1 = np > 1;
    static_for<8>([&](auto pc) { dma_piece<decltype(pc)::value>(d, lds, w, 1, 1, live1); });
    dma_piece<16>(d, lds, w, 1, 1, live1);
    dma_piece<17>(d, lds, w, 1, 1, live1);
    static_for<kRegPerPair>([&](auto qc) { load_b<decltype(qc)::value>(d, 1, live1, stage); });
    wait_and_barrier<kLdsDmaPerPair + kRegPerPair>();
    v8i f0a[4], f0b[4], f1a[4], f1b[4];
    int sca[4], scb[4], nsa[4], nsb[4];
    read_scales(lds, 0, wm, wn, r, h, sca, scb);
    static_for<8>([&](auto kc) { read_frag<0, decltype(kc)::value>(lds, 0, fo, f0a, f0b); });
    for (int kp = 0; kp < np; ++kp) {
      const int s = kp & 1;
      step_even<AT>(lds, d, s, kp, np, fo, f0a, f0b, sca, scb, f1a, f1b, stage, acc);
      step_odd<AT>(lds, d, w, s, kp, np, fo, wm, wn, r, h, f1a, f1b, sca, scb, f0a, f0b, nsa, nsb,
                   acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sca[i] = nsa[i];
        scb[i] = nsb[i];
      }
    }
  }
  // every copy has landed and no wave still reads a stage before the next
  // tile's prologue copies into them
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (part != nullptr) {
    store_part(part, acc, w, lane);
    return;
  }

  const int esz = out_f32 ? 4 : 2;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(t.out, (int64_t)t.out_rows * t.ldc * esz);
  // opaque copy of the row stride: keeps the compiler from hoisting all 256
  // store offsets out of the persistent tile loop into registers
  int ldc = (int)t.ldc;
  asm volatile("" : "+s"(ldc));
  const int row = wm * 128 + r, col = wn * 128 + 4 * h;
  if constexpr (EX) {
    EpiTerms ep;
    ep.alpha = t.alpha;
    ep.beta = t.beta;
    ep.has_bias = t.bias != nullptr;
    ep.bias = make_rsrc(t.bias, ep.has_bias ? (int64_t)t.out_cols * 4 : 0);
    const bool wide = (ldc & 3) == 0 && (t.out_cols & 3) == 0;
    if (out_f32) {
      if (wide) store_tile_ex<true, true>(acc, ro, ldc, row, col, t.out_cols, ep);
      else store_tile_ex<false, true>(acc, ro, ldc, row, col, t.out_cols, ep);
    } else {
      if (wide) store_tile_ex<true, false>(acc, ro, ldc, row, col, t.out_cols, ep);
      else store_tile_ex<false, false>(acc, ro, ldc, row, col, t.out_cols, ep);
    }
    return;
  }
  if (out_f32) {
    if ((ldc & 3) == 0 && (t.out_cols & 3) == 0)
      store_tile<true, true>(acc, ro, ldc, row, col, h, t.out_cols);
    else
      store_tile<false, true>(acc, ro, ldc, row, col, h, t.out_cols);
  } else {
    if ((ldc & 7) == 0 && (t.out_cols & 7) == 0)
      store_tile<true, false>(acc, ro, ldc, row, col, h, t.out_cols);
    else
      store_tile<false, false>(acc, ro, ldc, row, col, h, t.out_cols);
  }
}

// MODE: 0 FPROP_TN, 1 WGRAD_NT, 2 DGRAD_NN (E5M2 A), 3 WGRAD_NT with an E5M2 A.
template <int MODE, bool EX>
__global__ __launch_bounds__(kThreads) void mx_gemm_kernel(MxArgs p) {
  constexpr bool kWgrad = MODE == 1 || MODE == 3;
  __shared__ __attribute__((aligned(16))) uint8_t lds_ring[kBufs * kBufBytes];
  __shared__ Sched sm;
  const uint32_t lds = lds_offset(lds_ring);
  const int G = p.G;
  const int tid = threadIdx.x;
  uint32_t* status = blockIdx.x == 0 ? p.status : nullptr;
  load_offsets_clamped(p.offsets, G, p.rows_cap, sm.off, status);
  const int64_t ntn = (p.n + BN - 1) / BN;
  for (int g = tid; g < G; g += kThreads) {
    int64_t c;
    if (!kWgrad) {
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

  // the split of the last round (fprop / dgrad, whose tiles all contract k)
  const int grid = (int)gridDim.x;
  const int full = total / grid, left = total - full * grid;
  int nsplit = 1;
  if (!kWgrad && p.ws != nullptr && left > 0 && left <= kMaxSplitTiles) {
    const int np = (int)((p.k + kPairK - 1) / kPairK);
    nsplit = grid / left;
    if (nsplit > kSplitMax) nsplit = kSplitMax;
    if (nsplit > np / 2) nsplit = np / 2;
    if (nsplit < 2) nsplit = 1;
  }
  if (p.ws != nullptr && blockIdx.x == 0 && tid == 0) {
    int32_t* hdr = reinterpret_cast<int32_t*>(p.ws);
    hdr[0] = nsplit > 1 ? left : 0;
    hdr[1] = nsplit;
  }

  const int slot = xcd_slot();

  for (int round = 0;; ++round) {
    int tile = round * grid + slot;
    int part = -1;  // >= 0: part `part` of a split tile
    if (nsplit > 1 && round == full) {
      if (slot >= left * nsplit) break;
      tile = full * grid + slot / nsplit;
      part = slot % nsplit;
    }
    if (tile >= total) break;
    const int g = find_group(sm.pre, G, tile);
    const int local = tile - sm.pre[g];
    TileDesc t;
    int64_t col_first;  // the tile's first output column
    if (!kWgrad) {
      const int64_t m = group_extent(sm.off, g);
      const int mtiles = (int)((m + BM - 1) / BM);
      int mt, nt;
      super_tile<kSuperM, kSuperN>(local, mtiles, (int)ntn, mt, nt);
      const int64_t row0 = sm.off[g] + (int64_t)mt * BM;
      const int64_t n0 = (int64_t)nt * BN;
      col_first = n0;
      const int64_t nq = (p.k + 127) / 128;    // scale words per row
      const int64_t brow0 = (int64_t)g * p.n + n0;
      t.a = p.a + row0 * p.k;
      t.as = p.as + 4 * row0;                  // A scales: [nq][rows_cap] words
      t.sqa = 4 * p.rows_cap;
      t.as_bytes = nq * t.sqa - 4 * row0;
      if (MODE == 0) {
        t.b = p.b + brow0 * p.k;
        t.bs = p.bs + 4 * brow0;               // B scales: [nq][G * n] words
        t.sqb = 4 * (int64_t)G * p.n;
        t.bs_bytes = nq * t.sqb - 4 * brow0;
        t.ldb = p.k;
      } else {
        // DGRAD: B = the columnwise copy of W, whose experts are padded to
        // kp = 128 nq tokens: expert g's [n][kp] block at byte g * n * kp with
        // its own [nq][n] scale words at byte g * n * kp / 32
        const int64_t kpad = 128 * nq;
        t.b = p.b + (int64_t)g * p.n * kpad + n0 * kpad;
        t.bs = p.bs + (int64_t)g * p.n * kpad / 32 + 4 * n0;
        t.sqb = 4 * p.n;
        t.bs_bytes = nq * t.sqb - 4 * n0;
        t.ldb = kpad;
      }
      t.lda = p.k;
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
      const int ntm = (int)((p.n + BM - 1) / BM), ntk = (int)((p.k + BN - 1) / BN);
      int it, jt;
      super_tile<kSuperM, kSuperN>(local, ntm, ntk, it, jt);
      const int64_t n0 = (int64_t)it * BM, c0 = (int64_t)jt * BN;
      col_first = c0;
      const int64_t t0 = sm.off[g];
      // group g's blocks: data [n or k][mp], scales [mp / 128][n or k] words
      t.a = p.a + t0 * p.n + n0 * mp;
      t.b = p.b + t0 * p.k + c0 * mp;
      t.as = p.as + t0 * p.n / 32 + 4 * n0;
      t.sqa = 4 * p.n;
      t.as_bytes = (mp / 128) * t.sqa - 4 * n0;
      t.bs = p.bs + t0 * p.k / 32 + 4 * c0;
      t.sqb = 4 * p.k;
      t.bs_bytes = (mp / 128) * t.sqb - 4 * c0;
      t.lda = t.ldb = mp;
      const int64_t rv = p.n - n0, cv = p.k - c0;
      t.a_rows = (int)(rv < BM ? rv : BM);
      t.b_rows = (int)(cv < BN ? cv : BN);
      t.kl = ok ? mp : 0;
      t.out = reinterpret_cast<char*>(p.out) + (((int64_t)g * p.n + n0) * p.k + c0) * out_elem;
      t.ldc = p.k;
      t.out_rows = t.a_rows;
      t.out_cols = t.b_rows;
    }
    if constexpr (EX) {
      // the group's terms, made provably uniform (g comes from LDS)
      const int64_t outw = kWgrad ? p.k : p.n;  // output columns
      const int gu = __builtin_amdgcn_readfirstlane(g);
      const float al = p.alpha != nullptr ? p.alpha[gu] : 1.0f;
      const float be = p.beta != nullptr ? p.beta[gu] : 0.0f;
      t.alpha = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, al)));
      t.beta = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, be)));
      t.bias = p.bias != nullptr ? p.bias + (int64_t)gu * outw + col_first : nullptr;
    }
    float* part_dst = nullptr;
    if (part >= 0) {
      // pairs [np * part / S, np * (part + 1) / S) of the contraction
      const int np = (int)((t.kl + kPairK - 1) / kPairK);
      const int p0 = np * part / nsplit, p1 = np * (part + 1) / nsplit;
      const int64_t k0 = (int64_t)p0 * kPairK;
      const int64_t k1 = (int64_t)p1 * kPairK < t.kl ? (int64_t)p1 * kPairK : t.kl;
      t.a += k0;
      t.b += k0;
      t.as += p0 * t.sqa;
      t.as_bytes -= p0 * t.sqa;
      t.bs += p0 * t.sqb;
      t.bs_bytes -= p0 * t.sqb;
      t.kl = k1 - k0;
      part_dst = reinterpret_cast<float*>(p.ws + kWsHeader + (int64_t)slot * kPartBytes);
      if (part == 0 && tid == 0) {
        SplitRecord* rec = reinterpret_cast<SplitRecord*>(p.ws + 64) + slot / nsplit;
        rec->out_off = t.out - reinterpret_cast<char*>(p.out);
        rec->out_rows = t.out_rows;
        rec->out_cols = t.out_cols;
        rec->ldc = (int32_t)t.ldc;
        rec->pad = 0;
      }
    }
    run_tile<(MODE == 2 || MODE == 3) ? 1 : 0, EX>(lds, t, p.out_f32, part_dst);
  }
}

// The second step of a split: each split tile's parts summed in the order
// s = 0, 1, .. and stored as the plain epilogue stores a tile.  Work item
// (tile l, group ug of four units): wave w sums unit 4 ug + w of the parts.
__global__ __launch_bounds__(kThreads) void mx_split_reduce_kernel(const char* __restrict__ ws,
                                                                   void* out, int out_f32) {
  const int32_t* hdr = reinterpret_cast<const int32_t*>(ws);
  const int nl = hdr[0], nsplit = hdr[1];
  if (nl <= 0) return;
  const SplitRecord* recs = reinterpret_cast<const SplitRecord*>(ws + 64);
  const float* parts = reinterpret_cast<const float*>(ws + kWsHeader);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = lane & 31, h = lane >> 5;
  const int esz = out_f32 ? 4 : 2;
  for (int it = blockIdx.x; it < nl * 16; it += gridDim.x) {
    const int l = it / 16;
    const int u = 4 * (it % 16) + w;  // unit: source wave u / 16, block ((u / 4) % 4, u % 4)
    v16f y = v16f{};
    for (int sp = 0; sp < nsplit; ++sp) {
      const float* src = parts + (int64_t)(l * nsplit + sp) * (kPartBytes / 4) +
                         (int64_t)u * 1024 + 16 * lane;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4f v = *reinterpret_cast<const v4f*>(src + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) y[4 * q + e] += v[e];
      }
    }
    const SplitRecord rec = recs[l];
    const int wsrc = u / 16, i = (u / 4) % 4, j = u % 4;
    const int row = (wsrc >> 1) * 128 + 32 * i + r, col = (wsrc & 1) * 128 + 32 * j + 4 * h;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(reinterpret_cast<char*>(out) + rec.out_off, (int64_t)rec.out_rows * rec.ldc * esz);
    const int ldc = rec.ldc;
    if (out_f32) {
      if ((ldc & 3) == 0 && (rec.out_cols & 3) == 0)
        store_block<true, true>(y, ro, ldc, row, col, h, rec.out_cols);
      else
        store_block<false, true>(y, ro, ldc, row, col, h, rec.out_cols);
    } else {
      if ((ldc & 7) == 0 && (rec.out_cols & 7) == 0)
        store_block<true, false>(y, ro, ldc, row, col, h, rec.out_cols);
      else
        store_block<false, false>(y, ro, ldc, row, col, h, rec.out_cols);
    }
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

size_t gemm_mxfp8_workspace_bytes() {
  return (size_t)kWsHeader + (size_t)device_cu_count() * (size_t)kPartBytes;
}

hipError_t launch_gemm_mxfp8(int mode, int G, const uint8_t* a, const uint8_t* a_scales,
                             const uint8_t* b, const uint8_t* b_scales, const int64_t* offsets,
                             int64_t rows_cap, int64_t n, int64_t k, void* out, int out_f32,
                             uint32_t* status, hipStream_t stream, const float* alpha,
                             const float* beta, const float* bias, void* ws) {
  const bool ex = alpha != nullptr || beta != nullptr || bias != nullptr;
  if (ex) ws = nullptr;  // the epilogue terms are applied by the plain epilogue only
  MxArgs p{a,      a_scales, b,       b_scales, offsets, rows_cap, n,    k,
           out,    status,   G,       out_f32,  alpha,   beta,     bias, static_cast<char*>(ws)};
  // upper bound of the tile count from host-known shapes
  int64_t bound;
  if (mode != 1 && mode != 3) bound = ((rows_cap + BM - 1) / BM + G) * ((n + BN - 1) / BN);
  else bound = (int64_t)G * ((n + BM - 1) / BM) * ((k + BN - 1) / BN);
  int64_t grid = device_cu_count();
  if (bound < grid) grid = bound;
  if (grid <= 0) return hipSuccess;
  const dim3 gd((unsigned)grid), bd(kThreads);
  if (!ex) {
    if (mode == 0) hipLaunchKernelGGL((mx_gemm_kernel<0, false>), gd, bd, 0, stream, p);
    else if (mode == 1) hipLaunchKernelGGL((mx_gemm_kernel<1, false>), gd, bd, 0, stream, p);
    else if (mode == 3) hipLaunchKernelGGL((mx_gemm_kernel<3, false>), gd, bd, 0, stream, p);
    else hipLaunchKernelGGL((mx_gemm_kernel<2, false>), gd, bd, 0, stream, p);
  } else {
    if (mode == 0) hipLaunchKernelGGL((mx_gemm_kernel<0, true>), gd, bd, 0, stream, p);
    else if (mode == 1) hipLaunchKernelGGL((mx_gemm_kernel<1, true>), gd, bd, 0, stream, p);
    else if (mode == 3) hipLaunchKernelGGL((mx_gemm_kernel<3, true>), gd, bd, 0, stream, p);
    else hipLaunchKernelGGL((mx_gemm_kernel<2, true>), gd, bd, 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  // a split needs FPROP / DGRAD and at least two parts of two pairs each
  const bool may_split = mode != 1 && mode != 3 && (k + kPairK - 1) / kPairK >= 4;
  if (e != hipSuccess || ws == nullptr || !may_split) return e;
  // the split tiles' second step (returns at once when the GEMM split nothing)
  const int64_t rgrid = device_cu_count();
  hipLaunchKernelGGL(mx_split_reduce_kernel, dim3((unsigned)rgrid), dim3(kThreads), 0, stream,
                     static_cast<const char*>(ws), out, out_f32);
  return hipGetLastError();
}

}  // namespace bsg
