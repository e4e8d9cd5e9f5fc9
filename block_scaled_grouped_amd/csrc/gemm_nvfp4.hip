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
// The same kernel serves per-tensor NVFP4 ("gemm.py": alpha = the product of
// the two operands' tensor scales amax / (6 * 448)), one tensor per group:
// Y[r, n] = S[r, n] * alpha_g, alpha_g = (amax_A[g] / 2688) * (amax_B[g] / 2688).
//
// gfx950's scaled MFMA takes only power-of-two (E8M0) scales per 32 elements,
// and E2M1 x E4M3 needs up to 6 significant bits, so no FP8/FP6/FP4 MFMA input
// holds it exactly.  Each element is instead decoded in registers right before
// the MFMA that uses it: E2M1 -> fp16 pairs (hardware convert, unit scale),
// times its decoded E4M3 block scale with one packed fp16 multiply per pair --
// exact, since the product has at most 6 significant bits and lies in
// [2^-10, 2688], all normal fp16.  The product then runs on fp16 MFMA
// (v_mfma_f32_32x32x16_f16, the bf16 rate) with FP32 accumulation: exact
// products, FP32 sums.
//
// Tile 256 x 256, K-steps of 64, 4 wavefronts (2 x 2) of 128 x 128, each as
// 4 x 4 MFMA blocks of 32 x 32 (256 accumulator registers per lane).  What LDS
// holds is the packed operands, not decoded ones: a 3-deep ring of stages of
// two K-steps (64 bytes of E2M1 per row, XOR chunk swizzle) plus each row's
// E4M3 scale bytes of the stage, all copied global -> LDS by the buffer unit
// (LDS-DMA), a quarter of the LDS traffic of staging fp16.  Each wave reads,
// per K-step, 16 bytes and one scale dword for each of its 4 + 4 row blocks
// and decodes its own fragments: a lane's 16 bytes hold 32 consecutive
// elements, of which MFMA substep S takes dword S, and A and B lanes take the
// same elements in the same substep, so the contraction runs over the K-step's
// 64 elements in a permuted order.  The next K-step's bytes are read during
// the first substep and each next substep is decoded under the current one's
// MFMAs.  One barrier per stage; the copies of the stage three ahead are spread
// over the substeps that follow it.  Tiles are software-pipelined: the next
// tile's first stages and outer scales are copied before this tile's epilogue
// stores, and the epilogue reads one 32 x 32 accumulator block at a time.  B
// is the MFMA's first operand, so each lane holds an output row (see
// store_tile.h).  Tiles are handed out XCD-aware in 4 x 8 blocks of one group,
// as in the MXFP8 GEMM, so the operand rows that the 32 workgroups of an XCD
// stream meet in its L2.
#include <utility>

#include "lds_dma.h"
#include "store_tile.h"

namespace bsg {

namespace {

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
constexpr int BK = 64;                  // elements per K-step: four 16-deep MFMA substeps
constexpr int kStageK = 2 * BK;         // elements per LDS stage (two K-steps)
constexpr int kRowB = kStageK / 2;      // staged E2M1 bytes per row: 64
constexpr int kStages = 3;              // LDS ring depth
constexpr int kThreads = 256;
constexpr int kOpB = BM * kRowB;        // one operand's rows of a stage: 16 KiB
constexpr int kSclRowB = 16;            // staged scale bytes per row (room for the 2-byte form)
constexpr int kSclOpB = BM * kSclRowB;  // 4 KiB
constexpr int kStageB = 2 * kOpB + 2 * kSclOpB;  // A rows, B rows, A scales, B scales
constexpr int kBarrierSlot = 2;         // MFMA slot of an odd K-step's first substep after
                                        // which it waits for the next stage and barriers
constexpr int kSuperM = 4, kSuperN = 8; // tile block one XCD works on

// How a stage's E4M3 block scales are copied, from the contraction length k:
//   kSclDword  k % 64 == 0: a row's scale bytes of a stage are two aligned dwords,
//              one per K-step (4-byte copies; 8 staged bytes per row)
//   kSclShort  k % 64 == 32: the row stride k / 16 is only 2-aligned: four 2-byte
//              copies per row, (K-step ks, half h) into dword 2 ks + h
constexpr int kSclDword = 0, kSclShort = 1;
template <int SM>
constexpr int scl_row_bytes() { return SM == kSclDword ? 8 : 16; }
template <int SM>
constexpr int scl_copies() { return SM == kSclDword ? 2 : 4; }  // per operand, wave and stage
template <int SM>
constexpr int copies_per_stage() { return 8 + 2 * scl_copies<SM>(); }  // per wave

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) float lds_f32;

struct NvArgs {
  const uint8_t* a;
  const uint8_t* as;
  const float* aout;
  const int64_t* offsets;  // live row offsets; padded token offsets in wgrad
  int64_t rows_cap;        // capacity those offsets are clamped to
  int64_t k;               // contraction (fprop); dW columns (wgrad)
  int64_t n;               // dW rows (wgrad)
  const uint8_t* b;
  const uint8_t* bs;
  const float* bout;
  void* out;
  int64_t ld_out;
  float* s_buf;            // FP32 S of the two-step flow, or null (fused epilogue)
  char* ws;                // split workspace (fused fprop epilogue only), or null
  uint32_t* status;
  int G;
  int out_f32;
  int per_tensor;  // aout / bout hold one amax per group (per-tensor NVFP4)
  int accumulate;  // out = out_previous + Y instead of Y (row-scaled flows)
  NvGroupTable tab;
};

// The split of a partly filled last round of tiles along the contraction
// (fprop with the fused epilogue, as in the MXFP8 GEMM): the workspace holds a
// 16 KiB header -- the number of split tiles and of parts per tile, then one
// NvSplitRecord per split tile from byte 64 -- and one 256 KiB FP32 part per
// workgroup of that round; a second kernel sums each tile's parts in a fixed
// order and applies the outer scales (or alpha) and the store.
constexpr int kSplitMax = 8;
constexpr int64_t kWsHeader = 16384;
constexpr int64_t kPartBytes = (int64_t)BM * BN * 4;

struct NvSplitRecord {
  int64_t out_off;      // byte offset of the tile's first output element
  const float* aout_t;  // row-scaled: the outer scales of the tile's rows
  const float* bout_t;  // and of its columns
  float alpha;          // per-tensor: alpha_g of every row (columns 1)
  int32_t out_rows, out_cols, ldc, per_tensor;
};
static_assert(sizeof(NvSplitRecord) == 48, "split record layout");
constexpr int kMaxSplitTiles = (int)((kWsHeader - 64) / sizeof(NvSplitRecord));

struct Smem {
  uint8_t ring[kStages][kStageB];
  float aout[2][BM];  // outer scales of a tile's rows and columns, for its epilogue;
  float bout[2][BN];  // two sets, so the next tile's can land during this one's
  int64_t off[kMaxGroups + 1];
  int32_t cnt[kMaxGroups];
  int32_t pre[kMaxGroups + 1];
};

// Staged rows are 64 bytes, four 16-byte chunks; logical chunk c of row r sits
// in slot c ^ sw4(r).  sw4 takes bits 1..3 of r, so it is the same for rows 16
// apart (every copy covers 16 aligned rows, every fragment read 32), and both
// the 16 rows that one read cycle of a 64-bank LDS serves and the 8 of a
// 32-bank one land on distinct banks.
__device__ __forceinline__ int sw4(int r) {
  return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1);
}

__device__ __forceinline__ v4i lds_read16(uint32_t addr) {
  return *reinterpret_cast<const lds_v4i*>((size_t)addr);
}
__device__ __forceinline__ uint32_t lds_read4(uint32_t addr) {
  return *reinterpret_cast<const lds_u32*>((size_t)addr);
}

// One byte (two E2M1 nibbles, low nibble first) of dword w, times the block
// scale (in both halves of sd2), as a packed fp16 pair (low element first).
// The convert takes only the exponent of its scale operand, so the E4M3 scale
// is applied by the multiply (exact: at most 6 significant bits).
template <int SEL>
__device__ __forceinline__ uint32_t dq_pair(uint32_t w, v2h sd2) {
  const v2h f = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
  return __builtin_bit_cast(uint32_t, f * sd2);
}

// E4M3 codes in bytes 0 and 1 of c as fp16 (exact: every E4M3 value is a
// normal fp16; a unit scale leaves the value as it is).
__device__ __forceinline__ v2h e4m3_pair_h2(uint32_t c) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(c, 1.0f, false);
}

struct TileDesc {
  const uint8_t* a;
  const uint8_t* as;
  const uint8_t* b;
  const uint8_t* bs;
  int64_t lda, ldas;  // bytes per row: k/2 and k/16 (the same for both operands)
  int a_rows, b_rows;
  int64_t kl;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// A wavefront's share of one stage's copies: rows [64 w, 64 w + 64) of both
// operands, 16 rows (1 KiB) per data copy -- in copy q lane l fills row
// 64 w + 16 q + l / 4, slot l % 4, which must hold logical chunk
// (l % 4) ^ sw4(l / 4) -- and the same rows' scale bytes of the stage (32 rows
// of two dwords, or 16 rows of four 2-byte pieces, per copy).  A chunk or scale
// piece that starts at or past the contraction end is given an offset past
// every range, so it lands as zeros (the bytes there belong to the next row).
struct Dma {
  v4i ra, rb, rsa, rsb;  // descriptors (uniform)
  int src;               // lane data offset, copy q = 0, stage 0
  int kc;                // first element of its chunk within a stage
  int ld16;              // 16 rows of data stride (uniform)
  int ssrc;              // lane scale offset, copy q = 0, stage 0
  int skc;               // first element its scale piece covers within a stage
  int sstep;             // rows of one scale copy times the scale row stride (uniform)
  int kl;                // contraction length (uniform)
};

template <int SM>
__device__ __forceinline__ Dma make_dma(const TileDesc& t, int w, int lane) {
  Dma d;
  d.ra = make_rsrc_words(t.a, (int64_t)t.a_rows * t.lda);
  d.rb = make_rsrc_words(t.b, (int64_t)t.b_rows * t.lda);
  d.rsa = make_rsrc_words(t.as, (int64_t)t.a_rows * t.ldas);
  d.rsb = make_rsrc_words(t.bs, (int64_t)t.b_rows * t.ldas);
  const int c = (lane & 3) ^ sw4(lane >> 2);
  d.src = (64 * w + (lane >> 2)) * (int)t.lda + 16 * c;
  d.kc = 32 * c;
  d.ld16 = __builtin_amdgcn_readfirstlane(16 * (int)t.lda);
  if constexpr (SM == kSclDword) {
    d.ssrc = (64 * w + (lane >> 1)) * (int)t.ldas + 4 * (lane & 1);
    d.skc = BK * (lane & 1);
    d.sstep = __builtin_amdgcn_readfirstlane(32 * (int)t.ldas);
  } else {
    d.ssrc = (64 * w + (lane >> 2)) * (int)t.ldas + 2 * (lane & 3);
    d.skc = (BK / 2) * (lane & 3);
    d.sstep = __builtin_amdgcn_readfirstlane(16 * (int)t.ldas);
  }
  d.kl = __builtin_amdgcn_readfirstlane((int)t.kl);
  return d;
}

// Copy Q of this wave's share of stage sp into ring buffer `buf`: Q 0..3 A
// rows, 4..7 B rows, then the A and B scale copies.  A stage past the last
// (sp * 128 >= kl) has every piece past the contraction end, so it lands as
// zeros without reading.
template <int Q, int SM>
__device__ __forceinline__ void dma_piece(const Dma& d, uint32_t ring, int w, int buf, int sp) {
  const uint32_t st = ring + (uint32_t)(buf * kStageB);
  constexpr int SC = scl_copies<SM>();
  if constexpr (Q < 8) {
    constexpr int op = Q >> 2, q = Q & 3;
    const int off = d.kc + kStageK * sp < d.kl ? d.src + q * d.ld16 + kRowB * sp : kDmaOutOfRange;
    dma16(op ? d.rb : d.ra, st + op * kOpB + (64 * w + 16 * q) * kRowB, off);
  } else {
    constexpr int op = (Q - 8) / SC, q = (Q - 8) % SC;
    constexpr int rows = 64 / SC;  // rows per scale copy
    const uint32_t dst =
        st + 2 * kOpB + op * kSclOpB + (64 * w + rows * q) * scl_row_bytes<SM>();
    const int off = d.skc + kStageK * sp < d.kl ? d.ssrc + q * d.sstep + (kStageK / 16) * sp
                                                : kDmaOutOfRange;
    if constexpr (SM == kSclDword) dma4(op ? d.rsb : d.rsa, dst, off);
    else dma2(op ? d.rsb : d.rsa, dst, off);
  }
}

// Per-lane LDS offsets of the fragment reads within a stage, for its K-steps
// ks = 0, 1.  Lane (r, h) of wave (wm, wn) reads, of rows wm*128 + 32 i + r of A
// (wn*128 + 32 j + r of B), the 16 bytes of K-step ks that hold elements
// 32 h .. 32 h + 31 (logical chunk 2 ks + h), and the dword that holds the
// scales of their blocks 2 h and 2 h + 1 (bits ssh .. ssh + 15).
struct Frag {
  int da[2], db[2], sa[2], sb[2];
  int ssh;
};

template <int SM>
__device__ __forceinline__ Frag make_frag(int wm, int wn, int r, int h) {
  Frag f;
  constexpr int SR = scl_row_bytes<SM>();
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int c = ((2 * ks + h) ^ sw4(r)) << 4;
    const int sd = SM == kSclDword ? 4 * ks : 4 * (2 * ks + h);
    f.da[ks] = (wm * 128 + r) * kRowB + c;
    f.db[ks] = kOpB + (wn * 128 + r) * kRowB + c;
    f.sa[ks] = 2 * kOpB + (wm * 128 + r) * SR + sd;
    f.sb[ks] = 2 * kOpB + kSclOpB + (wn * 128 + r) * SR + sd;
    asm volatile("" : "+v"(f.da[ks]));
    asm volatile("" : "+v"(f.db[ks]));
    asm volatile("" : "+v"(f.sa[ks]));
    asm volatile("" : "+v"(f.sb[ks]));
  }
  f.ssh = SM == kSclDword ? 16 * h : 0;
  return f;
}

// One K-step's packed operands of this lane: 16 bytes and a scale dword for
// each of its four A and four B row blocks (0..3 A, 4..7 B).
struct Raw {
  v4i d[8];
  uint32_t s[8];
};

// Read item I (0..15) of a K-step from the stage at `st`: I < 8 the data of
// row block I, else the scale dword of row block I - 8.
template <int I, int KS, int SM>
__device__ __forceinline__ void read_item(uint32_t st, const Frag& f, Raw& x) {
  constexpr int SR = scl_row_bytes<SM>();
  if constexpr (I < 4) x.d[I] = lds_read16(st + f.da[KS] + 32 * I * kRowB);
  else if constexpr (I < 8) x.d[I] = lds_read16(st + f.db[KS] + 32 * (I - 4) * kRowB);
  else if constexpr (I < 12) x.s[I - 8] = lds_read4(st + f.sa[KS] + 32 * (I - 8) * SR);
  else x.s[I - 8] = lds_read4(st + f.sb[KS] + 32 * (I - 12) * SR);
}

// Half HALF (fp16 pairs 2 HALF, 2 HALF + 1) of the decoded fragment of substep
// S of a row block: dword S of its 16 bytes (elements 32 h + 8 S .. + 7, all in
// block 2 h + S / 2) times that block's scale.  A and B lanes hold the same
// elements in every substep, so the substeps together contract all 64 elements
// of the K-step in a permuted order.
template <int S, int HALF>
__device__ __forceinline__ void decode_half(const v4i& x, v2h s01, v4i& out) {
  const uint32_t w = (uint32_t)x[S];
  const _Float16 s = s01[S >> 1];
  const v2h s2 = v2h{s, s};
  out[2 * HALF] = (int)dq_pair<2 * HALF>(w, s2);
  out[2 * HALF + 1] = (int)dq_pair<2 * HALF + 1>(w, s2);
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// B is the MFMA's first operand and A its second, so each lane holds output
// rows (see store_tile.h).
template <int M>
__device__ __forceinline__ void mfma(const v4i (&df)[8], v16f (&acc)[4][4]) {
  constexpr int i = M >> 2, j = M & 3;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, df[4 + j]),
                                                      __builtin_bit_cast(v8h, df[i]), acc[i][j],
                                                      0, 0, 0);
  asm volatile("" : "+a"(acc[i][j]));  // keeps the pure intrinsic in schedule order
}

// K-step 2 sp + ODD of stage sp (ring buffer sp % 3), whose substep-0
// fragments are decoded in d0 and whose operands and block scales are in xc and
// sc.  Between its 64 MFMAs: the next K-step's operands are read into xn during
// the first substep (an odd step first waits until the next stage has landed
// for every wave and barriers; by then every wave has read the last of stage
// sp), each next substep's fragments are decoded, and during the fourth
// substep the next K-step's scales (into sn) and substep-0 fragments (into d0)
// follow.  An odd step also issues, spread over its last three substeps, the
// copies of stage sp + 3 into the buffer that stage sp leaves; at its barrier
// the copies issued after stage sp + 1's are exactly those of stage sp + 2.
template <bool ODD, int SM>
__device__ __forceinline__ void k_step(uint32_t ring, const Dma& d, const Frag& f, int w, int sp,
                                       int np, const Raw& xc, const v2h (&sc)[8], Raw& xn,
                                       v2h (&sn)[8], v4i (&d0)[8], v4i (&d1)[8],
                                       v16f (&acc)[4][4]) {
  constexpr int KS = ODD ? 0 : 1;  // the next K-step's half of its stage
  constexpr int kCopies = copies_per_stage<SM>();
  constexpr int kReadSlot = ODD ? kBarrierSlot + 1 : 0;
  constexpr int kCopyGap = 48 / kCopies;  // the copies spread over substeps 1 .. 3
  static_assert(kReadSlot + 8 <= 16 && kCopyGap >= 1, "K-step schedule");
  const bool more = !ODD || sp + 1 < np;
  const uint32_t rd = ring + (uint32_t)(((ODD ? sp + 1 : sp) % kStages) * kStageB);
  static_for<4>([&](auto sc_) {
    constexpr int S = decltype(sc_)::value;
    v4i(&cur)[8] = (S & 1) ? d1 : d0;
    v4i(&nxt)[8] = (S & 1) ? d0 : d1;
    static_for<16>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int b = m >> 1;  // the row block this slot decodes
      mfma<m>(cur, acc);
      fence();
      if constexpr (S == 0) {
        if constexpr (ODD && m == kBarrierSlot)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kCopies) : "memory");
        if constexpr (m >= kReadSlot && m < kReadSlot + 8) {
          if (more) {
            read_item<m - kReadSlot, KS, SM>(rd, f, xn);
            read_item<m - kReadSlot + 8, KS, SM>(rd, f, xn);
          }
        }
      }
      // one copy every kCopyGap MFMA slots from the second substep on, so
      // that the copies do not queue up behind each other in the memory pipe
      constexpr int slot = 16 * S + m - 16;
      if constexpr (ODD && slot >= 0 && slot % kCopyGap == 0 && slot / kCopyGap < kCopies)
        dma_piece<slot / kCopyGap, SM>(d, ring, w, (sp + 3) % kStages, sp + 3);
      if constexpr (S < 3) {
        decode_half<S + 1, m & 1>(xc.d[b], sc[b], nxt[b]);
      } else {
        if constexpr ((m & 1) == 0) sn[b] = e4m3_pair_h2(xn.s[b] >> f.ssh);
        decode_half<0, m & 1>(xn.d[b], sn[b], nxt[b]);
      }
      fence();
    });
  });
}

// The epilogue of a tile, one 32 x 32 block at a time: the block's
// accumulators are read into a temporary (pinned to that block, so that the
// whole tile is never copied out of the accumulators at once), scaled by
// a_outer[r] * b_outer[n] when fused, and stored (or, ACC, added to the
// output's previous contents and stored).
template <bool F32, bool WIDE, bool ACC>
__device__ __forceinline__ void epilogue_tile(const v16f (&acc)[4][4], bool fused,
                                              uint32_t ao_base, uint32_t bo_base,
                                              __amdgpu_buffer_rsrc_t ro, int ldc, int row, int col,
                                              int h, int out_cols) {
  static_for<16>([&](auto bc) {
    constexpr int i = decltype(bc)::value >> 2, j = decltype(bc)::value & 3;
    fence();
    v16f y = acc[i][j];
    asm volatile("" : "+v"(y));
    if (fused) {
      const float ao = *reinterpret_cast<const lds_f32*>((size_t)(ao_base + 4 * (row + 32 * i)));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const v4i bo = lds_read16(bo_base + 4 * (col + 32 * j + 8 * q));
#pragma unroll
        for (int e = 0; e < 4; ++e) y[4 * q + e] = (y[4 * q + e] * ao) * __int_as_float(bo[e]);
      }
    }
    const int rr = row + 32 * i, cc = col + 32 * j;
    if constexpr (ACC) {
      // copy-or-accumulate: Y + the output's previous value, rounded once
      EpiTerms ep;
      ep.alpha = 1.0f;
      ep.beta = 1.0f;
      ep.has_bias = false;
      ep.bias = ro;
      store_block_ex<WIDE, F32>(y, ro, ldc, rr, cc, out_cols, ep);
    } else {
      store_block<WIDE, F32>(y, ro, ldc, rr, cc, h, out_cols);
    }
    fence();
  });
}

// The accumulators of one part of a split tile: unit u = 16 w + 4 i + j (wave
// w's block (i, j)) at part + 1024 u floats, lane l's 16 values at + 16 l; one
// block at a time, like the epilogue.
__device__ __forceinline__ void store_part(float* __restrict__ part, const v16f (&acc)[4][4],
                                           int w, int lane) {
  static_for<16>([&](auto bc) {
    constexpr int i = decltype(bc)::value >> 2, j = decltype(bc)::value & 3;
    fence();
    v16f y = acc[i][j];
    asm volatile("" : "+v"(y));
    float* dst = part + (int64_t)(16 * w + 4 * i + j) * 1024 + 16 * lane;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<v4f*>(dst + 4 * q) = v4f{y[4 * q], y[4 * q + 1], y[4 * q + 2], y[4 * q + 3]};
    fence();
  });
}

// What a tile's epilogue needs besides its TileDesc.
struct TileJob {
  TileDesc t;
  int64_t out_off, ld_out;  // element offset of the tile's first output, row stride
};

// Tile `tile`'s descriptor, output position and outer-scale sources.
// part >= 0 (fprop): the tile's part `part` of `nsplit`, stages
// [np * part / nsplit, np * (part + 1) / nsplit) of the contraction.
template <bool WGRAD>
__device__ __forceinline__ TileJob make_job(const NvArgs& p, const Smem& sm, int G, int tile,
                                            int& g, const float*& aout_t, const float*& bout_t,
                                            int part = -1, int nsplit = 1) {
  g = __builtin_amdgcn_readfirstlane(find_group(sm.pre, G, tile));
  const int local = tile - sm.pre[g];
  TileJob job;
  TileDesc& t = job.t;
  if constexpr (WGRAD) {
    const int64_t mp = group_extent(sm.off, g);
    const bool usable = sm.off[g] % kColPad == 0 && mp % kColPad == 0;
    int mt, nt;
    super_tile<kSuperM, kSuperN>(local, (int)((p.n + BM - 1) / BM), (int)((p.k + BN - 1) / BN),
                                 mt, nt);
    const int64_t i0 = (int64_t)mt * BM, j0 = (int64_t)nt * BN;
    t.lda = mp / 2;
    t.ldas = mp / 16;
    t.a = p.a + sm.off[g] * p.n / 2 + i0 * t.lda;
    t.as = p.as + sm.off[g] * p.n / 16 + i0 * t.ldas;
    t.b = p.b + sm.off[g] * p.k / 2 + j0 * t.lda;
    t.bs = p.bs + sm.off[g] * p.k / 16 + j0 * t.ldas;
    t.a_rows = (int)(p.n - i0 < BM ? p.n - i0 : BM);
    t.b_rows = (int)(p.k - j0 < BN ? p.k - j0 : BN);
    t.kl = usable ? mp : 0;
    aout_t = p.aout + (int64_t)g * p.n + i0;
    bout_t = p.bout + (int64_t)g * p.k + j0;
    job.out_off = ((int64_t)g * p.n + i0) * p.k + j0;
    job.ld_out = p.k;
  } else {
    const int64_t m = group_extent(sm.off, g);
    const int64_t ng = p.tab.n[g];
    int mt, nt;
    super_tile<kSuperM, kSuperN>(local, (int)((m + BM - 1) / BM), (int)((ng + BN - 1) / BN), mt,
                                 nt);
    const int64_t row0 = sm.off[g] + (int64_t)mt * BM;
    const int64_t n0 = (int64_t)nt * BN;
    const int64_t brow0 = p.tab.brow[g] + n0;
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
    aout_t = p.aout + row0;
    bout_t = p.bout + brow0;
    job.out_off = row0 * p.ld_out + n0;
    job.ld_out = p.ld_out;
    if (part >= 0) {
      const int np = (int)((p.k + kStageK - 1) / kStageK);
      const int p0 = np * part / nsplit, p1 = np * (part + 1) / nsplit;
      const int64_t k0 = (int64_t)p0 * kStageK;
      const int64_t k1 = (int64_t)p1 * kStageK < p.k ? (int64_t)p1 * kStageK : p.k;
      t.a += k0 / 2;
      t.as += k0 / 16;
      t.b += k0 / 2;
      t.bs += k0 / 16;
      t.kl = k1 - k0;
    }
  }
  return job;
}

// The start of tile `tile`: the copies of its first three stages into ring
// buffers 0, 1, 2, and its outer scales into outer-scale set `set` (copied by
// the buffer unit too; zeros for rows and columns past the tile's and for a
// tile with nothing to contract, whose output is then exactly 0).  The caller
// waits for all of it (vmcnt(0) and a barrier) before use; the ring and the
// set must be free.
template <int SM, bool WGRAD>
__device__ __forceinline__ void start_tile(const NvArgs& p, Smem& sm, uint32_t ring, int G,
                                           int tile, int part, int nsplit, int set, int tid) {
  // opaque copy of the thread index: keeps the per-lane copy offsets from being
  // hoisted out of the tile loop (and spilled)
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int g;
  const float* aout_t;
  const float* bout_t;
  const TileJob job = make_job<WGRAD>(p, sm, G, tile, g, aout_t, bout_t, part, nsplit);
  const TileDesc& t = job.t;
  const bool contract = t.kl > 0;
  // per-tensor NVFP4: alpha_g = tsi(amax_A[g]) * tsi(amax_B[g]) on every row,
  // 1 on every column, so the epilogue computes S * alpha_g (read before the
  // copies are issued, so that waiting for it does not wait for them)
  const bool pt = !WGRAD && p.per_tensor;
  const float alpha = pt ? (p.aout[g] / 2688.0f) * (p.bout[g] / 2688.0f) : 0.0f;
  if (contract) {
    const Dma d = make_dma<SM>(t, w, lane);
    for (int sp = 0; sp < 3; ++sp)
      static_for<copies_per_stage<SM>()>([&](auto qc) {
        dma_piece<decltype(qc)::value, SM>(d, ring, w, sp, sp);
      });
  }
  const uint32_t ao = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)sm.aout[set];
  const uint32_t bo = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)sm.bout[set];
  if (pt) {
    sm.aout[set][tid] = contract && tid < t.a_rows ? alpha : 0.0f;
    sm.bout[set][tid] = contract && tid < t.b_rows ? 1.0f : 0.0f;
  } else {
    // wave w copies rows / columns 64 w .. 64 w + 63
    dma4(make_rsrc_words(aout_t, contract ? (int64_t)t.a_rows * 4 : 0), ao + 256 * w,
         4 * (64 * w + lane));
    dma4(make_rsrc_words(bout_t, contract ? (int64_t)t.b_rows * 4 : 0), bo + 256 * w,
         4 * (64 * w + lane));
  }
}

// WGRAD: expert g contracts its padded tokens, A = dY^T_g [n, m~_g], B =
// X^T_g [k, m~_g] (the columnwise copies), dW[g] = (S * a_outer[g, i]) *
// b_outer[g, j] into out [G, n, k]; every expert has its n x k tiles, an empty
// one (or one whose padded offsets are not multiples of 128, flagged) zeros.
template <int SM, bool WGRAD>
__global__ __launch_bounds__(kThreads) void nv_gemm_kernel(NvArgs p) {
  __shared__ Smem sm;
  const int G = p.G;
  const int tid0 = threadIdx.x;
  uint32_t* status = blockIdx.x == 0 ? p.status : nullptr;
  load_offsets_clamped(p.offsets, G, p.rows_cap, sm.off, status);
  for (int g = tid0; g < G; g += kThreads) {
    if constexpr (WGRAD) {
      const int64_t mp = group_extent(sm.off, g);
      if (sm.off[g] % kColPad != 0 || mp % kColPad != 0) dev_status_or(status, kDevBadPadding);
      sm.cnt[g] = (int32_t)(((p.n + BM - 1) / BM) * ((p.k + BN - 1) / BN));
    } else {
      const int64_t m = group_extent(sm.off, g);
      const int64_t ng = p.tab.n[g];
      sm.cnt[g] = (int32_t)(((m + BM - 1) / BM) * ((ng + BN - 1) / BN));
    }
  }
  __syncthreads();
  wave0_exclusive_scan(sm.cnt, G, sm.pre);
  __syncthreads();
  const int total = sm.pre[G];
  const uint32_t ring = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)sm.ring[0];

  // the split of a partly filled last round (fprop, fused epilogue)
  const int grid = (int)gridDim.x;
  const int full = total / grid, left = total - full * grid;
  int nsplit = 1;
  if (!WGRAD && p.ws != nullptr && p.s_buf == nullptr && left > 0 && left <= kMaxSplitTiles) {
    const int np = (int)((p.k + kStageK - 1) / kStageK);
    nsplit = grid / left;
    if (nsplit > kSplitMax) nsplit = kSplitMax;
    if (nsplit > np / 2) nsplit = np / 2;
    if (nsplit < 2) nsplit = 1;
  }
  if (p.ws != nullptr && blockIdx.x == 0 && tid0 == 0) {
    int32_t* hdr = reinterpret_cast<int32_t*>(p.ws);
    hdr[0] = nsplit > 1 ? left : 0;
    hdr[1] = nsplit;
  }

  const int slot = xcd_slot();
  // This workgroup's unit of round r: a whole tile (part -1), or in a split
  // last round part slot % nsplit of tile full * grid + slot / nsplit.
  auto unit = [&](int r, int& tl, int& pt) -> bool {
    if (nsplit > 1 && r >= full) {
      if (r > full || slot >= left * nsplit) return false;
      tl = full * grid + slot / nsplit;
      pt = slot % nsplit;
      return true;
    }
    tl = r * grid + slot;
    pt = -1;
    return tl < total;
  };
  // Tiles are software-pipelined: the next tile's set-up, its first three
  // stages' copies and its outer scales are issued before this tile's
  // epilogue, so they land while its stores drain.
  int round = 0, tile = 0, part = -1, set = 0;
  bool have = unit(0, tile, part);
  if (have) start_tile<SM, WGRAD>(p, sm, ring, G, tile, part, nsplit, set, tid0);
  while (have) {
    // opaque copies of the thread and tile indices: keep the compiler from
    // hoisting every LDS / global offset of the tile body out of the tile loop,
    // or carrying the tile's descriptor through the previous epilogue
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    asm volatile("" : "+s"(tile));
    asm volatile("" : "+s"(part));
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int r = lane & 31, h = lane >> 5;
    int g_t;
    const float* aout_t;
    const float* bout_t;
    const TileJob job = make_job<WGRAD>(p, sm, G, tile, g_t, aout_t, bout_t, part, nsplit);
    const TileDesc& t = job.t;
    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    // every copy of the tile's start (and the previous tile's stores) has
    // landed; the outer scales written by other waves are visible
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int np = (int)((t.kl + kStageK - 1) / kStageK);  // stages; >= 1 unless nothing to
                                                             // contract (a tail reads as zeros)
    if (np > 0) {
      const Dma d = make_dma<SM>(t, w, lane);
      const Frag f = make_frag<SM>(wm, wn, r, h);
      // K-step 0's operands and scales (stage 0), and its substep-0 fragments
      Raw x0, x1;
      v2h s0[8], s1[8];
      v4i d0[8], d1[8];
      static_for<16>([&](auto ic) { read_item<decltype(ic)::value, 0, SM>(ring, f, x0); });
      static_for<8>([&](auto bc) {
        constexpr int b = decltype(bc)::value;
        s0[b] = e4m3_pair_h2(x0.s[b] >> f.ssh);
        decode_half<0, 0>(x0.d[b], s0[b], d0[b]);
        decode_half<0, 1>(x0.d[b], s0[b], d0[b]);
      });
      for (int sp = 0; sp < np; ++sp) {
        k_step<false, SM>(ring, d, f, w, sp, np, x0, s0, x1, s1, d0, d1, acc);
        k_step<true, SM>(ring, d, f, w, sp, np, x1, s1, x0, s0, d0, d1, acc);
      }
      // every copy (those of the stages past the last included) has landed and
      // no wave still reads the ring before the next tile's copies
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }

    // the next tile's start, into the other outer-scale set (whose last reader,
    // the previous epilogue, every wave has left at the barriers above)
    const int64_t out_off = job.out_off, ld_out = job.ld_out;
    const int a_rows = t.a_rows, b_rows = t.b_rows;
    int next = 0, npart = -1;
    const bool nhave = unit(round + 1, next, npart);
    if (nhave) start_tile<SM, WGRAD>(p, sm, ring, G, next, npart, nsplit, set ^ 1, tid0);

    if (part >= 0) {
      // a part of a split tile: its raw sums into this workgroup's part slot;
      // part 0 records where the tile's output and outer scales are
      store_part(reinterpret_cast<float*>(p.ws + kWsHeader + (int64_t)slot * kPartBytes), acc, w,
                 lane);
      if (part == 0 && tid0 == 0) {
        NvSplitRecord* rec = reinterpret_cast<NvSplitRecord*>(p.ws + 64) + slot / nsplit;
        rec->out_off = out_off * (p.out_f32 ? 4 : 2);
        rec->aout_t = aout_t;
        rec->bout_t = bout_t;
        rec->alpha = p.per_tensor ? (p.aout[g_t] / 2688.0f) * (p.bout[g_t] / 2688.0f) : 0.0f;
        rec->out_rows = a_rows;
        rec->out_cols = b_rows;
        rec->ldc = (int32_t)ld_out;
        rec->per_tensor = p.per_tensor;
      }
      tile = next;
      part = npart;
      have = nhave;
      ++round;
      set ^= 1;
      continue;
    }

    // epilogue: S -> (S * a_outer) * b_outer, or S itself into the scratch
    const bool fused = p.s_buf == nullptr;
    const bool f32out = !fused || p.out_f32;
    const int esz = f32out ? 4 : 2;
    char* obase = fused ? reinterpret_cast<char*>(p.out) : reinterpret_cast<char*>(p.s_buf);
    obase += out_off * esz;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(obase, (int64_t)a_rows * ld_out * esz);
    int ldc = (int)ld_out;
    asm volatile("" : "+s"(ldc));
    const int row = wm * 128 + r, col = wn * 128 + 4 * h;
    const uint32_t ao_base = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)sm.aout[set];
    const uint32_t bo_base = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)sm.bout[set];
    const bool wide = f32out ? ((ldc & 3) == 0 && (b_rows & 3) == 0)
                             : ((ldc & 7) == 0 && (b_rows & 7) == 0);
    if (fused && p.accumulate) {
      const bool wide4 = (ldc & 3) == 0 && (b_rows & 3) == 0;
      if (p.out_f32) {
        if (wide4) epilogue_tile<true, true, true>(acc, true, ao_base, bo_base, ro, ldc, row, col, h, b_rows);
        else epilogue_tile<true, false, true>(acc, true, ao_base, bo_base, ro, ldc, row, col, h, b_rows);
      } else {
        if (wide4) epilogue_tile<false, true, true>(acc, true, ao_base, bo_base, ro, ldc, row, col, h, b_rows);
        else epilogue_tile<false, false, true>(acc, true, ao_base, bo_base, ro, ldc, row, col, h, b_rows);
      }
    } else if (f32out) {
      if (wide) epilogue_tile<true, true, false>(acc, fused, ao_base, bo_base, ro, ldc, row, col, h, b_rows);
      else epilogue_tile<true, false, false>(acc, fused, ao_base, bo_base, ro, ldc, row, col, h, b_rows);
    } else {
      if (wide) epilogue_tile<false, true, false>(acc, fused, ao_base, bo_base, ro, ldc, row, col, h, b_rows);
      else epilogue_tile<false, false, false>(acc, fused, ao_base, bo_base, ro, ldc, row, col, h, b_rows);
    }
    tile = next;
    part = npart;
    have = nhave;
    ++round;
    set ^= 1;
  }
  // the last tile's stores, and copies of a start that had no tile, complete
  // before the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Unfused second step: Y[r, n] = (S[r, n] * a_outer[r]) * b_outer_g[n] for the
// live rows r of group g and n < N_g, one block per row (with the accumulate
// flag, Y is added to the output's previous value, then rounded once).  VEC
// (row stride a multiple of 4, 16-byte aligned buffers): each thread takes four
// consecutive columns per step -- one 16-byte read of S (streamed: read once)
// and of b_outer, one 16- or 8-byte store; the last N_g mod 4 columns one by one.
template <bool VEC>
__global__ __launch_bounds__(256) void nv_postscale_kernel(const float* __restrict__ s_buf,
                                                           const float* __restrict__ aout,
                                                           const float* __restrict__ bout,
                                                           const int64_t* __restrict__ offsets,
                                                           int64_t rows_cap, int G, void* out,
                                                           int64_t ld_out, int out_f32,
                                                           int accumulate, NvGroupTable tab) {
  __shared__ int64_t s_off[kMaxGroups + 1];
  load_offsets_clamped(offsets, G, rows_cap, s_off, nullptr);
  const int64_t row = blockIdx.x;
  if (row < s_off[0] || row >= s_off[G]) return;  // rows no group owns stay untouched
  int lo = 0, hi = G - 1;  // group: largest g with s_off[g] <= row and a non-empty extent
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (s_off[mid] <= row) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const int ng = tab.n[g];
  const float ao = aout[row];
  const float* bo = bout + tab.brow[g];
  const float* srow = s_buf + row * ld_out;
  int n0 = 0;
  if constexpr (VEC) {
    const int n4 = ng & ~3;
    for (int n = 4 * (int)threadIdx.x; n < n4; n += 4 * (int)blockDim.x) {
      const v4f sv = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(srow + n));
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = (sv[e] * ao) * bo[n + e];
      if (out_f32) {
        v4f* o = reinterpret_cast<v4f*>(reinterpret_cast<float*>(out) + row * ld_out + n);
        if (accumulate) {
          const v4f old = *o;
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = old[e] + y[e];
        }
        *o = v4f{y[0], y[1], y[2], y[3]};
      } else {
        v2i* o = reinterpret_cast<v2i*>(reinterpret_cast<uint16_t*>(out) + row * ld_out + n);
        if (accumulate) {
          const v2i old = *o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wd = (uint32_t)old[e >> 1];
            y[e] = bf16_to_f32((e & 1) ? (wd >> 16) : (wd & 0xffffu)) + y[e];
          }
        }
        *o = v2i{(int)(f32_to_bf16_rne(y[0]) | (f32_to_bf16_rne(y[1]) << 16)),
                 (int)(f32_to_bf16_rne(y[2]) | (f32_to_bf16_rne(y[3]) << 16))};
      }
    }
    n0 = n4;
  }
  for (int n = n0 + (int)threadIdx.x; n < ng; n += blockDim.x) {
    float y = (srow[n] * ao) * bo[n];
    if (out_f32) {
      float* o = reinterpret_cast<float*>(out) + row * ld_out + n;
      if (accumulate) y = *o + y;
      *o = y;
    } else {
      uint16_t* o = reinterpret_cast<uint16_t*>(out) + row * ld_out + n;
      if (accumulate) y = bf16_to_f32(*o) + y;
      *o = (uint16_t)f32_to_bf16_rne(y);
    }
  }
}

// The second step of a split: each split tile's parts summed in the order
// s = 0, 1, .., then Y = (S * a_outer[r]) * b_outer[n] (per-tensor: S * alpha_g)
// and the fused epilogue's store (or, with accumulate, its read-add-store).
// Work item (tile l, group ug of four units): wave w takes unit 4 ug + w.
__global__ __launch_bounds__(kThreads) void nv_split_reduce_kernel(const char* __restrict__ ws,
                                                                   void* out, int out_f32,
                                                                   int accumulate) {
  const int32_t* hdr = reinterpret_cast<const int32_t*>(ws);
  const int nl = hdr[0], nsplit = hdr[1];
  if (nl <= 0) return;
  const NvSplitRecord* recs = reinterpret_cast<const NvSplitRecord*>(ws + 64);
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
    const NvSplitRecord rec = recs[l];
    const int wsrc = u / 16, i = (u / 4) % 4, j = u % 4;
    const int row = (wsrc >> 1) * 128 + 32 * i + r, col = (wsrc & 1) * 128 + 32 * j + 4 * h;
    // outer scales as the fused epilogue takes them: rows and columns past
    // the tile's read 0 (their stores are dropped anyway)
    float ao;
    if (rec.per_tensor) {
      ao = rec.alpha;
    } else {
      const __amdgpu_buffer_rsrc_t ra = make_rsrc(rec.aout_t, (int64_t)rec.out_rows * 4);
      ao = __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(ra, 4 * row, 0, 0));
    }
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(rec.bout_t, rec.per_tensor ? 0 : (int64_t)rec.out_cols * 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float bo = rec.per_tensor ? 1.0f
                                        : __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                                              rb, 4 * (col + 8 * q + e), 0, 0));
        y[4 * q + e] = (y[4 * q + e] * ao) * bo;
      }
    }
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(reinterpret_cast<char*>(out) + rec.out_off, (int64_t)rec.out_rows * rec.ldc * esz);
    const int ldc = rec.ldc;
    if (accumulate) {
      EpiTerms ep;
      ep.alpha = 1.0f;
      ep.beta = 1.0f;
      ep.has_bias = false;
      ep.bias = ro;
      const bool wide4 = (ldc & 3) == 0 && (rec.out_cols & 3) == 0;
      if (out_f32) {
        if (wide4) store_block_ex<true, true>(y, ro, ldc, row, col, rec.out_cols, ep);
        else store_block_ex<false, true>(y, ro, ldc, row, col, rec.out_cols, ep);
      } else {
        if (wide4) store_block_ex<true, false>(y, ro, ldc, row, col, rec.out_cols, ep);
        else store_block_ex<false, false>(y, ro, ldc, row, col, rec.out_cols, ep);
      }
    } else if (out_f32) {
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

size_t gemm_nvfp4_workspace_bytes() {
  return (size_t)kWsHeader + (size_t)device_cu_count() * (size_t)kPartBytes;
}

hipError_t launch_gemm_nvfp4(int G, const uint8_t* a, const uint8_t* a_scales,
                             const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                             int64_t k, const uint8_t* b, const uint8_t* b_scales,
                             const float* b_outer, const NvGroupTable& table, int max_n,
                             void* out, int64_t ld_out, int out_f32, float* s_buf,
                             uint32_t* status, hipStream_t stream, bool per_tensor,
                             bool accumulate, void* ws) {
  NvArgs p;
  p.a = a; p.as = a_scales; p.aout = a_outer; p.offsets = offsets; p.rows_cap = rows_cap; p.k = k;
  p.n = 0;
  p.b = b; p.bs = b_scales; p.bout = b_outer; p.out = out; p.ld_out = ld_out; p.s_buf = s_buf;
  if (s_buf != nullptr) ws = nullptr;  // the split serves the fused epilogue only
  p.ws = static_cast<char*>(ws);
  p.status = status; p.G = G; p.out_f32 = out_f32; p.per_tensor = per_tensor ? 1 : 0;
  p.accumulate = accumulate ? 1 : 0;
  p.tab = table;
  if (per_tensor && s_buf != nullptr) return hipErrorInvalidValue;
  const int64_t bound = ((rows_cap + BM - 1) / BM + G) * ((max_n + BN - 1) / BN);
  int64_t grid = device_cu_count();
  if (bound < grid) grid = bound;
  if (grid > 0) {
    // k % 64 == 0 keeps each row's scale dword of a K-step 4-aligned
    if (k % BK == 0)
      hipLaunchKernelGGL((nv_gemm_kernel<kSclDword, false>), dim3((unsigned)grid),
                         dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((nv_gemm_kernel<kSclShort, false>), dim3((unsigned)grid),
                         dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the split tiles' second step (returns at once when the GEMM split
    // nothing); a split needs at least two parts of two stages each.  Eight
    // workgroups per CU: each work item is a short chain of loads, so many
    // in flight keep it from being latency-bound (empty, it costs the same)
    if (ws != nullptr && (k + kStageK - 1) / kStageK >= 4) {
      hipLaunchKernelGGL(nv_split_reduce_kernel, dim3((unsigned)(8 * device_cu_count())), dim3(kThreads),
                         0, stream, static_cast<const char*>(ws), out, out_f32, accumulate ? 1 : 0);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  if (s_buf != nullptr && rows_cap > 0) {
    const bool vec = ld_out % 4 == 0 && reinterpret_cast<uintptr_t>(s_buf) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(out) % 16 == 0;
    if (vec)
      hipLaunchKernelGGL(nv_postscale_kernel<true>, dim3((unsigned)rows_cap), dim3(256), 0, stream,
                         s_buf, a_outer, b_outer, offsets, rows_cap, G, out, ld_out, out_f32,
                         accumulate ? 1 : 0, table);
    else
      hipLaunchKernelGGL(nv_postscale_kernel<false>, dim3((unsigned)rows_cap), dim3(256), 0,
                         stream, s_buf, a_outer, b_outer, offsets, rows_cap, G, out, ld_out,
                         out_f32, accumulate ? 1 : 0, table);
    return hipGetLastError();
  }
  return hipSuccess;
}

// ---------------------------------------------------------------- no-allocation form
//
// The two-step flow above with its FP32 S in a library-owned device array, for
// callers that cannot allocate (code under HIP-graph capture, serving loops,
// harnesses that forbid allocation).  Each GPU holds its own copy of the array
// until the process ends; every call on a GPU shares it, so calls that overlap
// on one GPU race.  The GEMM writes S for every (live row, column < N_g) before
// the post-scale kernel reads exactly those entries, so nothing needs clearing.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
float* g_scratch_ptr[kMaxDevices] = {};  // the array's device address on each GPU
}  // namespace

// The array's address on the current device, looked up once per device (with
// that device current); the host-side name `scratch` is not a device address.
hipError_t noalloc_scratch_ptr(float** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* p = __atomic_load_n(&g_scratch_ptr[dev], __ATOMIC_ACQUIRE);
  if (p == nullptr) {
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (addr == nullptr) return hipErrorInvalidSymbol;
    p = static_cast<float*>(addr);
    __atomic_store_n(&g_scratch_ptr[dev], p, __ATOMIC_RELEASE);
  }
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_gemm_nvfp4_noalloc(int G, const uint8_t* a, const uint8_t* a_scales,
                                     const float* a_outer, const int64_t* offsets,
                                     int64_t rows_cap, int64_t k, const uint8_t* b,
                                     const uint8_t* b_scales, const float* b_outer,
                                     const NvGroupTable& table, int max_n, void* out,
                                     int64_t ld_out, int out_f32, uint32_t* status,
                                     hipStream_t stream) {
  if (rows_cap * ld_out > (int64_t)(kNoAllocScratchBytes / sizeof(float)))
    return hipErrorInvalidValue;  // the C-ABI layer rejects this size first
  float* ptr = nullptr;
  const hipError_t e = noalloc_scratch_ptr(&ptr);
  if (e != hipSuccess) return e;
  return launch_gemm_nvfp4(G, a, a_scales, a_outer, offsets, rows_cap, k, b, b_scales, b_outer,
                           table, max_n, out, ld_out, out_f32, ptr, status, stream, false, false);
}

hipError_t launch_gemm_nvfp4_wgrad(int G, const uint8_t* a, const uint8_t* a_scales,
                                   const float* a_outer, const uint8_t* b, const uint8_t* b_scales,
                                   const float* b_outer, const int64_t* padded_offsets,
                                   int64_t col_rows_cap, int64_t n, int64_t k, void* out,
                                   int out_f32, uint32_t* status, hipStream_t stream,
                                   bool accumulate) {
  NvArgs p;
  p.a = a; p.as = a_scales; p.aout = a_outer; p.offsets = padded_offsets;
  p.rows_cap = col_rows_cap; p.k = k; p.n = n;
  p.b = b; p.bs = b_scales; p.bout = b_outer; p.out = out; p.ld_out = k; p.s_buf = nullptr;
  p.ws = nullptr;
  p.status = status; p.G = G; p.out_f32 = out_f32; p.per_tensor = 0; p.tab = NvGroupTable{};
  p.accumulate = accumulate ? 1 : 0;
  const int64_t bound = (int64_t)G * ((n + BM - 1) / BM) * ((k + BN - 1) / BN);
  int64_t grid = device_cu_count();
  if (bound < grid) grid = bound;
  if (grid <= 0) return hipSuccess;
  // padded token counts are multiples of 128: 4-aligned scale dwords
  hipLaunchKernelGGL((nv_gemm_kernel<kSclDword, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace bsg
