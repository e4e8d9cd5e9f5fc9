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
// holds it exactly.  Each element is instead decoded while it is staged into
// LDS: E2M1 -> fp16 pairs (hardware convert, unit scale), times its decoded E4M3
// block scale with one packed fp16 multiply per pair -- exact, since the product
// has at most 6 significant bits and lies in [2^-10, 2688], all normal fp16.
// The product then runs on fp16 MFMA (v_mfma_f32_32x32x16_f16, the bf16 rate)
// with FP32 accumulation: exact products, FP32 sums.
//
// Tile 256 x 256, K-steps of 64, 4 wavefronts (2 x 2) of 128 x 128, each as
// 4 x 4 MFMA blocks of 32 x 32 (256 accumulator registers per lane).  LDS holds
// two stages of fp16 rows (128 bytes per row per K-step) with an XOR chunk
// swizzle that keeps both the row-wise stores and the fragment reads free of
// bank conflicts.  Waves 0-1 decode A and waves 2-3 B, thread t rows t % 128
// and t % 128 + 128 of its operand: the raw E2M1 bytes and E4M3 scales of
// K-step k + 1 are decoded into the other stage, one fp16 pair at a time,
// between the MFMAs of step k, and the raw bytes of step k + 2 are already
// being loaded.  One barrier per K-step, placed before the
// last MFMAs so that the next step's first fragments are read under them.  B is
// the MFMA's first operand, so each lane holds an output row (see store_tile.h).
// Tiles are handed out XCD-aware in 4 x 8 blocks of one group, as in the MXFP8
// GEMM, so the operand rows that the 32 workgroups of an XCD stream meet in its
// L2.
#include <utility>

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
constexpr int BK = 64;          // elements per K-step (32 bytes of E2M1 per row)
constexpr int kThreads = 256;
constexpr int kDecodeSlots = 48; // the next step's decode is spread over MFMA slots 0 .. 47
constexpr int kBarrierSlot = 4;  // MFMA slot of the last substep after which the step barriers
constexpr int kSuperM = 4, kSuperN = 8;  // tile block one XCD works on

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i lds_v4i;
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
  uint32_t* status;
  int G;
  int out_f32;
  int per_tensor;  // aout / bout hold one amax per group (per-tensor NVFP4)
  int accumulate;  // out = out_previous + Y instead of Y (row-scaled flows)
  NvGroupTable tab;
};

static_assert(BM == BN, "A and B stage halves share one layout");
// the next step's decode units (slots 0 .. kDecodeSlots - 1 of the 64) must all
// be written before the step's barrier, which follows the decode of slot
// 48 + kBarrierSlot: a later unit would write the stage other waves then read
static_assert(kDecodeSlots <= 3 * 16 + kBarrierSlot + 1 && kDecodeSlots <= 64 &&
                  kBarrierSlot >= 0 && kBarrierSlot < 16,
              "decode must finish before the step's barrier");
constexpr int kHalfStage = BM * 128;  // one operand's rows of one K-step, fp16
constexpr int kOperandB = 2 * kHalfStage;

struct Smem {
  // A stage 0, A stage 1, B stage 0, B stage 1: every offset between the
  // stages, and between rows r and r + 128, fits an LDS instruction's
  // immediate offset field
  uint8_t stage[4][kHalfStage];
  float aout[BM];
  float bout[BN];
  int64_t off[kMaxGroups + 1];
  int32_t cnt[kMaxGroups];
  int32_t pre[kMaxGroups + 1];
};

// LDS byte offset of 16-byte chunk c (fp16 elements 8 c .. 8 c + 7) of row r:
// the chunk is XORed with a 3-bit term of r % 16.  Over 8 aligned rows the term
// takes 8 values (as over the even and the odd rows of 16 aligned ones), and its
// low two bits 4 values over 4 aligned rows (as over the even and the odd rows
// of 8 aligned ones), so both 16-byte access patterns used here -- one chunk of
// 64 consecutive rows (fragment reads), and chunks q and q + 4 of 32 rows by
// lane pairs (decode stores) -- are conflict-free whether the LDS serves 8
// lanes per 128-byte bank window or 16 lanes per 256-byte window.
__device__ __forceinline__ int swz(int row, int chunk) {
  const int term = (row & 3) ^ (((row >> 2) & 1) * 5) ^ ((row >> 3) & 1);
  return row * 128 + ((chunk ^ term) << 4);
}

__device__ __forceinline__ v4i lds_read16(uint32_t addr) {
  return *reinterpret_cast<const lds_v4i*>((size_t)addr);
}
__device__ __forceinline__ void lds_write16(uint32_t addr, v4i v) {
  *reinterpret_cast<lds_v4i*>((size_t)addr) = v;
}

// One byte (two E2M1 nibbles, low nibble first) of dword w, times the block
// scale (in both halves of sd2), as a packed fp16 pair (low element first).
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

// Per-lane LDS offsets, computed once per tile and kept opaque so that the
// compiler does not materialize one address per access.
struct Offs {
  int dec[4];       // chunk 4 hf + q of this thread's first decoded row (see Raw)
  int fa[4], fb[4]; // fragment part S: row wm*128 + r (A) / wn*128 + r (B), chunk 2 S + h
  int ssh;          // 16 hf: this thread's scale bytes within a row's scale word
};

__device__ __forceinline__ Offs make_offs(int tid, int wm, int wn, int r, int h) {
  Offs o;
  const int hf = tid & 1, r0 = (tid & 127) >> 1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    o.dec[q] = (tid >= 128 ? kOperandB : 0) + swz(r0, 4 * hf + q);
    asm volatile("" : "+v"(o.dec[q]));
  }
  o.ssh = 16 * hf;
#pragma unroll
  for (int S = 0; S < 4; ++S) {
    o.fa[S] = swz(wm * 128 + r, 2 * S + h);
    o.fb[S] = kOperandB + swz(wn * 128 + r, 2 * S + h);
    asm volatile("" : "+v"(o.fa[S]));
    asm volatile("" : "+v"(o.fb[S]));
  }
  return o;
}

// 16 raw bytes (32 elements, two 16-element blocks with scales s0, s1) -> 32
// fp16, written as this thread's four 16-byte chunks of a row at `base`
// relative to its first row.
__device__ __forceinline__ void decode_store(uint32_t base, const Offs& o, const v4i& d, v2h s0,
                                             v2h s1) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t w = (uint32_t)d[q];
    const v2h sd = q < 2 ? s0 : s1;
    v4i v;
    v[0] = (int)dq_pair<0>(w, sd);
    v[1] = (int)dq_pair<1>(w, sd);
    v[2] = (int)dq_pair<2>(w, sd);
    v[3] = (int)dq_pair<3>(w, sd);
    lds_write16(base + o.dec[q], v);
  }
}

// Raw E2M1 bytes of one K-step for this thread: waves 0 and 1 decode A,
// waves 2 and 3 B; with u = tid % 128, half hf = u % 2 (16 of the row's 32
// bytes) of rows u / 2 + 64 j, j = 0 .. 3.  The two threads of a row sit in
// adjacent lanes, so each load instruction reaches 32 rows, not 64.
struct Raw {
  v4i d[4];
};

// E4M3 block-scale words of two K-steps (kt, kt + 1; kt even) for the same
// four rows: word x of step kt, y of kt + 1, four scales each.
struct Scl {
  v2i s[4];
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

struct Rsrc {
  __amdgpu_buffer_rsrc_t d, s, none;  // this thread's operand and its scales
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// How a row's E4M3 scale words are loaded, from the contraction length k:
//   kScalePaired  k % 128 == 0: the two words of a step pair, one aligned 8-byte load
//   kScaleWord    k % 64 == 0: one aligned 4-byte load per step
//   kScaleHalf    k % 64 == 32: the row stride k / 16 is only 2-aligned and the last
//                 step is half past k: each thread loads its own two scale bytes
//                 (2-byte loads), and its raw bytes and scales past k read as zeros
constexpr int kScalePaired = 0, kScaleWord = 1, kScaleHalf = 2;

// An offset past every descriptor's range: the buffer unit returns zeros.
constexpr int kOutOfRange = 0x7ffffff0;

// This thread's raw bytes of K-step kt.  Rows past the valid ones, and steps
// past the last (`live` false), read as zeros; with kScaleHalf so does a
// half step past the contraction end (the bytes there are the next row's).
template <int SM>
__device__ __forceinline__ void load_raw(const TileDesc& t, const Rsrc& rs, int kt, bool live,
                                         int tid, Raw& x) {
  int od = ((tid & 127) >> 1) * (int)t.lda + (tid & 1) * 16 + kt * (BK / 2);
  if constexpr (SM == kScaleHalf)
    if (kt * BK + (tid & 1) * (BK / 2) >= (int)t.kl) od = kOutOfRange;
  const int rstep = 64 * (int)t.lda;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x.d[j] = __builtin_amdgcn_raw_buffer_load_b128(live ? rs.d : rs.none,
                                                   od == kOutOfRange ? od : od + j * rstep, 0, 0);
}

// The scale words of K-steps kt and kt + 1 (kt even) for this thread's rows;
// with kScalePaired / kScaleWord both threads of a row load the same bytes, one
// request, and a step past the last reads as zero.  With kScaleHalf thread half
// hf loads only the two bytes it decodes, into bits 16 hf .. 16 hf + 15 of the
// word (where the decode takes them from).
template <int SM>
__device__ __forceinline__ void load_scales(const TileDesc& t, const Rsrc& rs, int kt, int nk,
                                            int tid, Scl& x) {
  const int os = ((tid & 127) >> 1) * (int)t.ldas + kt * (BK / 16);
  const int rstep = 64 * (int)t.ldas;
  const bool l0 = kt < nk, l1 = kt + 1 < nk;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (SM == kScalePaired) {
      x.s[j] = __builtin_amdgcn_raw_buffer_load_b64(l0 ? rs.s : rs.none, os + j * rstep, 0, 0);
    } else if constexpr (SM == kScaleWord) {
      x.s[j][0] = __builtin_amdgcn_raw_buffer_load_b32(l0 ? rs.s : rs.none, os + j * rstep, 0, 0);
      x.s[j][1] =
          __builtin_amdgcn_raw_buffer_load_b32(l1 ? rs.s : rs.none, os + j * rstep + 4, 0, 0);
    } else {
      const int hf = tid & 1;
      const int kl = (int)t.kl;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int k0 = (kt + e) * BK + hf * (BK / 2);  // first element of this half step
        const int off = k0 < kl ? os + 4 * e + 2 * hf + j * rstep : kOutOfRange;
        const uint32_t v = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(
            (e ? l1 : l0) ? rs.s : rs.none, off, 0, 0);
        x.s[j][e] = (int)(v << (16 * hf));
      }
    }
  }
}

// This thread's two block scales of row j in scale word w, as fp16.
__device__ __forceinline__ v2h row_scales(uint32_t w, const Offs& o) {
  return e4m3_pair_h2(w >> o.ssh);
}

// Row J of this thread's decode of one K-step (scale words in `sw`) into the
// stage at `st`.
template <int J>
__device__ __forceinline__ void decode_row(uint32_t st, const Offs& o, const Raw& x,
                                           const uint32_t (&sw)[4]) {
  const v2h s01 = row_scales(sw[J], o);
  decode_store(st + J * 64 * 128, o, x.d[J], v2h{s01[0], s01[0]}, v2h{s01[1], s01[1]});
}

// Decode unit U (0..63) of a K-step: row U / 16 (as decode_row), word
// (U / 4) % 4 of its 16 raw bytes, nibble pair U % 4 -> one fp16 pair into
// `buf`; the fourth pair of a word writes the 16-byte chunk to LDS.  Spread one
// or two per MFMA slot, the decode's VALU work runs under the MFMAs.
template <int U>
__device__ __forceinline__ void decode_unit(uint32_t st, const Offs& o, const Raw& x,
                                            const uint32_t (&sw)[4], v2h (&sd)[2], v4i& buf) {
  constexpr int J = U / 16, q = (U / 4) % 4, pr = U % 4;
  if constexpr (U % 16 == 0) {
    const v2h s01 = row_scales(sw[J], o);
    sd[0] = v2h{s01[0], s01[0]};
    sd[1] = v2h{s01[1], s01[1]};
  }
  const uint32_t w = (uint32_t)x.d[J][q];
  buf[pr] = (int)dq_pair<pr>(w, q < 2 ? sd[0] : sd[1]);
  if constexpr (pr == 3) lds_write16(st + J * 64 * 128 + o.dec[q], buf);
}

__device__ __forceinline__ void fence() { __builtin_amdgcn_sched_barrier(0); }

// The fragments of substep S (16 elements of the K-step) for this lane: rows
// wm*128 + 32 i + r of A, wn*128 + 32 j + r of B, elements 16 S + 8 h .. + 7.
template <int S>
__device__ __forceinline__ void read_frags(uint32_t st, const Offs& o, v8h (&fa)[4],
                                           v8h (&fb)[4]) {
  // rows 32 apart share the lane's swizzle term: the row step is an immediate
#pragma unroll
  for (int i = 0; i < 4; ++i)
    fa[i] = __builtin_bit_cast(v8h, lds_read16(st + o.fa[S] + 32 * i * 128));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    fb[j] = __builtin_bit_cast(v8h, lds_read16(st + o.fb[S] + 32 * j * 128));
}

template <int M>
__device__ __forceinline__ void mfma(const v8h (&fa)[4], const v8h (&fb)[4], v16f (&acc)[4][4]) {
  constexpr int i = M >> 2, j = M & 3;
  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  asm volatile("" : "+a"(acc[i][j]));  // keeps the pure intrinsic in schedule order
}

// One K-step from stage `cur` (its substep-0 fragments already in f0): while
// its 64 MFMAs run, decode the raw bytes of the next step (xn, scale words sw)
// into stage `nxt`, load the raw bytes of the step after it (into xl) and, for
// an even step (SCALES), the scale words of that step and the next (into sl),
// read each next substep's fragments, and after the barrier the next step's
// first fragments.
template <bool SCALES, int SM>
__device__ __forceinline__ void k_step(uint32_t cur, uint32_t nxt, const TileDesc& t,
                                       const Rsrc& rs, int kt, int nk, int tid, const Offs& o,
                                       const Raw& xn, const uint32_t (&sw)[4], Raw& xl, Scl& sl,
                                       v8h (&f0a)[4], v8h (&f0b)[4], v8h (&f1a)[4],
                                       v8h (&f1b)[4], v16f (&acc)[4][4]) {
  load_raw<SM>(t, rs, kt + 2, kt + 2 < nk, tid, xl);
  if constexpr (SCALES) load_scales<SM>(t, rs, kt + 2, nk, tid, sl);
  v2h sd[2];
  v4i buf;
  static_for<4>([&](auto sc) {
    constexpr int S = decltype(sc)::value;
    v8h(&ca)[4] = (S & 1) ? f1a : f0a;
    v8h(&cb)[4] = (S & 1) ? f1b : f0b;
    v8h(&na)[4] = (S & 1) ? f0a : f1a;
    v8h(&nb)[4] = (S & 1) ? f0b : f1b;
    static_for<16>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      mfma<m>(ca, cb, acc);
      fence();
      if constexpr (m == 0 && S < 3) read_frags<S + 1>(cur, o, na, nb);
      // decode units assigned to this slot: U with floor(U * kDecodeSlots / 64) == slot
      constexpr int slot = 16 * S + m;
      constexpr int u0 = (slot * 64 + kDecodeSlots - 1) / kDecodeSlots;
      constexpr int u1 = ((slot + 1) * 64 + kDecodeSlots - 1) / kDecodeSlots;
      if constexpr (slot < kDecodeSlots) {
        static_for<(u1 < 64 ? u1 : 64) - u0>([&](auto uc) {
          decode_unit<u0 + decltype(uc)::value>(nxt, o, xn, sw, sd, buf);
        });
      }
      if constexpr (S == 3 && m == kBarrierSlot) {
        // the decode of the next step is in LDS and nobody still reads `cur`
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        read_frags<0>(nxt, o, na, nb);
      }
      fence();
    });
  });
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
  const uint32_t st0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)sm.stage[0];
  const uint32_t st1 = st0 + kHalfStage;

  const int slot = xcd_slot();
  for (int tile = slot; tile < total; tile += gridDim.x) {
    // opaque per-tile copy of the thread index: keeps the compiler from
    // hoisting every LDS / global offset of the tile body out of the tile loop
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;
    const int r = lane & 31, h = lane >> 5;
    const int g = find_group(sm.pre, G, tile);
    const int local = tile - sm.pre[g];
    TileDesc t;
    const float* aout_t;      // outer scales of the tile's rows / columns
    const float* bout_t;
    int64_t out_off, ld_out;  // element offset of the tile's first output, row stride
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
      out_off = ((int64_t)g * p.n + i0) * p.k + j0;
      ld_out = p.k;
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
      out_off = row0 * p.ld_out + n0;
      ld_out = p.ld_out;
    }
    // waves 0 and 1 decode A, waves 2 and 3 B
    const bool opb = w >= 2;
    Rsrc rs;
    rs.d = opb ? make_rsrc(t.b, (int64_t)t.b_rows * t.lda) : make_rsrc(t.a, (int64_t)t.a_rows * t.lda);
    rs.s = opb ? make_rsrc(t.bs, (int64_t)t.b_rows * t.ldas)
               : make_rsrc(t.as, (int64_t)t.a_rows * t.ldas);
    rs.none = make_rsrc(t.a, 0);

    // outer scales of this tile's rows and columns, for the epilogue (zeros for
    // a tile with nothing to contract, whose output is then exactly 0)
    const bool contract = t.kl > 0;
    if (!WGRAD && p.per_tensor) {
      // per-tensor NVFP4: alpha_g = tsi(amax_A[g]) * tsi(amax_B[g]) on every
      // row, 1 on every column, so the epilogue computes S * alpha_g
      const float alpha = (p.aout[g] / 2688.0f) * (p.bout[g] / 2688.0f);
      sm.aout[tid] = contract && tid < t.a_rows ? alpha : 0.0f;
      sm.bout[tid] = contract && tid < t.b_rows ? 1.0f : 0.0f;
    } else {
      sm.aout[tid] = contract && tid < t.a_rows ? aout_t[tid] : 0.0f;
      sm.bout[tid] = contract && tid < t.b_rows ? bout_t[tid] : 0.0f;
    }
    // the epilogue reads entries other waves wrote; a tile with nothing to
    // contract reaches it without the K-loop's barriers
    __syncthreads();

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    const int nk = (int)((t.kl + BK - 1) / BK);  // >= 1 unless nothing to contract
    const int nk2 = (nk + 1) & ~1;     // an odd last step runs on zeros
    if (nk > 0) {
      const Offs o = make_offs(tid, wm, wn, r, h);
      Raw x0, x1;
      Scl sc0, sc1;  // scale words of steps (kt, kt + 1) and (kt + 2, kt + 3)
      v8h f0a[4], f0b[4], f1a[4], f1b[4];
      load_scales<SM>(t, rs, 0, nk, tid, sc0);
      load_raw<SM>(t, rs, 0, true, tid, x0);
      load_raw<SM>(t, rs, 1, 1 < nk, tid, x1);
      {
        const uint32_t sw[4] = {(uint32_t)sc0.s[0][0], (uint32_t)sc0.s[1][0],
                                (uint32_t)sc0.s[2][0], (uint32_t)sc0.s[3][0]};
        static_for<4>([&](auto jc) { decode_row<decltype(jc)::value>(st0, o, x0, sw); });
      }
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      read_frags<0>(st0, o, f0a, f0b);
      for (int kt = 0; kt < nk2; kt += 2) {
        const uint32_t swa[4] = {(uint32_t)sc0.s[0][1], (uint32_t)sc0.s[1][1],
                                 (uint32_t)sc0.s[2][1], (uint32_t)sc0.s[3][1]};
        k_step<true, SM>(st0, st1, t, rs, kt, nk, tid, o, x1, swa, x0, sc1, f0a, f0b, f1a,
                         f1b, acc);
        const uint32_t swb[4] = {(uint32_t)sc1.s[0][0], (uint32_t)sc1.s[1][0],
                                 (uint32_t)sc1.s[2][0], (uint32_t)sc1.s[3][0]};
        k_step<false, SM>(st1, st0, t, rs, kt + 1, nk, tid, o, x0, swb, x1, sc1, f0a, f0b,
                          f1a, f1b, acc);
        sc0 = sc1;
      }
    }

    // epilogue: S -> (S * a_outer) * b_outer, or S itself into the scratch
    const bool fused = p.s_buf == nullptr;
    const bool f32out = !fused || p.out_f32;
    const int esz = f32out ? 4 : 2;
    char* obase = fused ? reinterpret_cast<char*>(p.out) : reinterpret_cast<char*>(p.s_buf);
    obase += out_off * esz;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(obase, (int64_t)t.a_rows * ld_out * esz);
    int ldc = (int)ld_out;
    asm volatile("" : "+s"(ldc));
    const int row = wm * 128 + r, col = wn * 128 + 4 * h;
    const uint32_t ao_base = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)sm.aout;
    const uint32_t bo_base = (uint32_t)(size_t)(__attribute__((address_space(3))) float*)sm.bout;
    const bool wide = f32out ? ((ldc & 3) == 0 && (t.b_rows & 3) == 0)
                             : ((ldc & 7) == 0 && (t.b_rows & 7) == 0);
    // one 32 x 32 block at a time: scaled into a temporary (fused) and stored
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ao = fused ? *reinterpret_cast<const lds_f32*>((size_t)(ao_base + 4 * (row + 32 * i)))
                             : 1.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v16f y = acc[i][j];
        if (fused) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const v4i bo = lds_read16(bo_base + 4 * (col + 32 * j + 8 * q));
#pragma unroll
            for (int e = 0; e < 4; ++e) y[4 * q + e] = (y[4 * q + e] * ao) * __int_as_float(bo[e]);
          }
        }
        const int rr = row + 32 * i, cc = col + 32 * j;
        if (fused && p.accumulate) {
          // copy-or-accumulate: Y + the output's previous value, rounded once
          EpiTerms ep;
          ep.alpha = 1.0f;
          ep.beta = 1.0f;
          ep.has_bias = false;
          ep.bias = ro;
          const bool wide4 = (ldc & 3) == 0 && (t.b_rows & 3) == 0;
          if (p.out_f32) {
            if (wide4) store_block_ex<true, true>(y, ro, ldc, rr, cc, t.b_rows, ep);
            else store_block_ex<false, true>(y, ro, ldc, rr, cc, t.b_rows, ep);
          } else {
            if (wide4) store_block_ex<true, false>(y, ro, ldc, rr, cc, t.b_rows, ep);
            else store_block_ex<false, false>(y, ro, ldc, rr, cc, t.b_rows, ep);
          }
        } else if (f32out) {
          if (wide) store_block<true, true>(y, ro, ldc, rr, cc, h, t.b_rows);
          else store_block<false, true>(y, ro, ldc, rr, cc, h, t.b_rows);
        } else {
          if (wide) store_block<true, false>(y, ro, ldc, rr, cc, h, t.b_rows);
          else store_block<false, false>(y, ro, ldc, rr, cc, h, t.b_rows);
        }
      }
    }
    __syncthreads();  // aout / bout and the stages are rewritten by the next tile
  }
}

// Unfused second step: Y[r, n] = (S[r, n] * a_outer[r]) * b_outer_g[n] for the
// live rows r of group g and n < N_g, one block per row.
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
  for (int n = threadIdx.x; n < ng; n += blockDim.x) {
    float y = (s_buf[row * ld_out + n] * ao) * bo[n];
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

}  // namespace

hipError_t launch_gemm_nvfp4(int G, const uint8_t* a, const uint8_t* a_scales,
                             const float* a_outer, const int64_t* offsets, int64_t rows_cap,
                             int64_t k, const uint8_t* b, const uint8_t* b_scales,
                             const float* b_outer, const NvGroupTable& table, int max_n,
                             void* out, int64_t ld_out, int out_f32, float* s_buf,
                             uint32_t* status, hipStream_t stream, bool per_tensor,
                             bool accumulate) {
  NvArgs p;
  p.a = a; p.as = a_scales; p.aout = a_outer; p.offsets = offsets; p.rows_cap = rows_cap; p.k = k;
  p.n = 0;
  p.b = b; p.bs = b_scales; p.bout = b_outer; p.out = out; p.ld_out = ld_out; p.s_buf = s_buf;
  p.status = status; p.G = G; p.out_f32 = out_f32; p.per_tensor = per_tensor ? 1 : 0;
  p.accumulate = accumulate ? 1 : 0;
  p.tab = table;
  if (per_tensor && s_buf != nullptr) return hipErrorInvalidValue;
  const int64_t bound = ((rows_cap + BM - 1) / BM + G) * ((max_n + BN - 1) / BN);
  int64_t grid = device_cu_count();
  if (bound < grid) grid = bound;
  if (grid > 0) {
    // an even step count keeps each row's scale words of a step pair 8-aligned
    if (k % (2 * BK) == 0)
      hipLaunchKernelGGL((nv_gemm_kernel<kScalePaired, false>), dim3((unsigned)grid),
                         dim3(kThreads), 0, stream, p);
    else if (k % BK == 0)
      hipLaunchKernelGGL((nv_gemm_kernel<kScaleWord, false>), dim3((unsigned)grid),
                         dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((nv_gemm_kernel<kScaleHalf, false>), dim3((unsigned)grid),
                         dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (s_buf != nullptr && rows_cap > 0) {
    hipLaunchKernelGGL(nv_postscale_kernel, dim3((unsigned)rows_cap), dim3(256), 0, stream,
                       s_buf, a_outer, b_outer, offsets, rows_cap, G, out, ld_out, out_f32,
                       accumulate ? 1 : 0, table);
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
  p.status = status; p.G = G; p.out_f32 = out_f32; p.per_tensor = 0; p.tab = NvGroupTable{};
  p.accumulate = accumulate ? 1 : 0;
  const int64_t bound = (int64_t)G * ((n + BM - 1) / BM) * ((k + BN - 1) / BN);
  int64_t grid = device_cu_count();
  if (bound < grid) grid = bound;
  if (grid <= 0) return hipSuccess;
  // padded token counts are multiples of 128: an even number of 64-deep steps
  hipLaunchKernelGGL((nv_gemm_kernel<kScalePaired, true>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace bsg
