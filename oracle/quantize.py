"""Grouped MXFP8, row-scaled NVFP4 and per-tensor NVFP4 quantize, and the
matching dequantize (oracle; test infrastructure only).

Operands are bf16 bit patterns (uint16) of a row-major [rows, cols] tensor whose
first ``offsets[G]`` rows are live and split into G consecutive groups
(``offsets`` as produced by ``oracle.offsets.group_offsets``).  Rows at or past
``offsets[G]`` are capacity rows: never read, never written.
"""

import numpy as np

from .formats import (bf16_bits_to_f64, e4m3_encode, e4m3_decode, e5m2_encode, e5m2_decode,
                      e2m1_encode, e2m1_decode, e8m0_from_amax, e8m0_decode, f32, E2M1_MAX,
                      E4M3_MAX, E4M3_EMAX, E5M2_EMAX)
from .layout import (mx_scales_to_gemm_order, mx_scales_from_gemm_order, mx_scale_row_bytes,
                     fp4_pack, fp4_unpack)

MX_BLOCK = 32
NVFP4_BLOCK = 16
COLWISE_PAD = 128
FLT_MAX = np.float32(np.finfo(np.float32).max)


# element formats of MXFP8: (encode, decode, emax)
MX_ELEMENTS = {"e4m3": (e4m3_encode, e4m3_decode, E4M3_EMAX),
               "e5m2": (e5m2_encode, e5m2_decode, E5M2_EMAX)}


def _mx_encode_blocks(vals, elem="e4m3"):
    """[..., 32] exact values -> (element codes [..., 32], E8M0 bytes [...]).

    One MX block: shared scale from the block's largest magnitude, each element
    divided by that power of two (exact) and rounded to the element format
    (E4M3, or E5M2 for gradients; ties to even, saturating)."""
    encode, _, emax = MX_ELEMENTS[elem]
    amax = np.abs(vals).max(axis=-1)
    sbyte = e8m0_from_amax(amax, emax)
    scaled = vals / e8m0_decode(sbyte)[..., None]
    return encode(scaled), sbyte


def mxfp8_rowwise(x_bits, offsets, elem="e4m3"):
    """Rowwise MXFP8 quantize: 32-element blocks along each row (the contraction
    dim of an fprop activation or of a weight, "gemm.py",
    ``_quantize_gemm_operands``); elements E4M3, or E5M2 for a gradient
    (``_compatible_fp8_gemm_dtypes`` pairs E5M2 with E4M3).

    Returns (data [live, C] uint8 codes, scales [NQ, live, 4] uint8 E8M0 words
    in the GEMM-ready order, NQ = ceil(C / 128))."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    live = int(offsets[-1])
    if live > rows:
        raise ValueError("sum of group sizes exceeds the row capacity")
    x = bf16_bits_to_f64(x_bits[:live]).reshape(live, cols // MX_BLOCK, MX_BLOCK)
    codes, sbyte = _mx_encode_blocks(x, elem)
    return codes.reshape(live, cols), mx_scales_to_gemm_order(sbyte)


def mxfp8_colwise(x_bits, offsets, padded_offsets, elem="e4m3"):
    """Columnwise MXFP8 quantize for a contraction over ragged token rows
    (wgrad): per group g and column c, 32-token blocks starting at the group's
    first row, written transposed; elements E4M3, or E5M2 for a gradient
    ("gemm.py", ``_compatible_fp8_gemm_dtypes`` pairs E5M2 with E4M3).

    Reading: a group's token count is padded to a multiple of 128 with zero
    values (so padding encodes to 0x00 and all-padding blocks get scale 0x00),
    following "padding is included in the group sizes" ("gemm.py",
    ``grouped_gemm``) and the 128-alignment of the V2 kernels ("[JAX] MXFP8
    Grouped Quant+GEMM", review threads).

    Group g's data is a row-major [C, m~_g] block at element offset
    ``padded_offsets[g] * C`` and its scales an [m~_g / 128, C, 4] block of words
    (GEMM-ready order) at ``padded_offsets[g] * C / 32``.  Returns (data, scales) as flat
    uint8 arrays of padded_offsets[G] * C and padded_offsets[G] * C / 32 bytes."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    off = np.asarray(offsets, dtype=np.int64)
    poff = np.asarray(padded_offsets, dtype=np.int64)
    if int(off[-1]) > rows:
        raise ValueError("sum of group sizes exceeds the row capacity")
    data = np.zeros(int(poff[-1]) * cols, dtype=np.uint8)
    scales = np.zeros(int(poff[-1]) * cols // MX_BLOCK, dtype=np.uint8)
    for g in range(len(off) - 1):
        m = int(off[g + 1] - off[g])
        mp = int(poff[g + 1] - poff[g])
        if mp < m or mp % COLWISE_PAD:
            raise ValueError("padded offsets inconsistent with the group sizes")
        if mp == 0:
            continue
        xt = np.zeros((cols, mp), dtype=np.float64)
        xt[:, :m] = bf16_bits_to_f64(x_bits[off[g]:off[g + 1]]).T
        codes, sbyte = _mx_encode_blocks(xt.reshape(cols, mp // MX_BLOCK, MX_BLOCK), elem)
        data[poff[g] * cols:poff[g + 1] * cols] = codes.reshape(-1)
        scales[poff[g] * cols // MX_BLOCK:poff[g + 1] * cols // MX_BLOCK] = \
            mx_scales_to_gemm_order(sbyte).reshape(-1)
    return data, scales


def mxfp8_dequant_rows(data, stored_scales, cols, elem="e4m3"):
    """Q->DQ of MXFP8 rows: undo the GEMM-ready scale order, then
    element * 2**(scale - 127).  data [R, cols], stored_scales [NQ, R, 4]."""
    data = np.asarray(data, dtype=np.uint8).reshape(-1, cols)
    nq = mx_scale_row_bytes(cols // MX_BLOCK) // 4
    sbyte = mx_scales_from_gemm_order(np.asarray(stored_scales).reshape(nq, data.shape[0], 4),
                                      cols // MX_BLOCK)
    vals = MX_ELEMENTS[elem][1](data).reshape(data.shape[0], cols // MX_BLOCK, MX_BLOCK)
    return (vals * e8m0_decode(sbyte)[..., None]).reshape(data.shape[0], cols)


def nvfp4_rowscaled(x_bits, offsets):
    """Row-scaled NVFP4 quantize of the live rows.

    Per row r: an FP32 outer scale from the row's largest magnitude, the
    per-row analogue of the tensor scale ``amax / (6 * 448)`` ("gemm.py",
    ``_get_nvfp4_tensor_scale_inv``; per-row / per-column outer scales: "[Common]
    [PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM").  Per
    16-element block: an E4M3 scale; elements in E2M1.

    Reading of the float32 steps (the pages fix only the outer scale), in this
    order, every operation rounded to float32:
      S    = 2688 / amax_r (1 if amax_r == 0; capped at FLT_MAX)
      s_f  = (bmax / 6) * S          -> s8 = E4M3(s_f), sd = decode(s8)
      enc  = S / sd (0 if sd == 0; capped at FLT_MAX)
      q    = E2M1(x * enc)
    so that x ~= e2m1(q) * sd * tsi_r with tsi_r = amax_r / 2688.

    Returns (packed [live, C/2] uint8, block scales [live, C/16] uint8 E4M3,
    outer scale tsi [live] float32)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    live = int(offsets[-1])
    if live > rows:
        raise ValueError("sum of group sizes exceeds the row capacity")
    x = f32(bf16_bits_to_f64(x_bits[:live]))                    # exact in float32
    two688 = np.float32(E2M1_MAX * E4M3_MAX)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        amax = np.abs(x).max(axis=1) if cols else np.zeros(live, np.float32)
        tsi = f32(amax / two688)
        big_s = np.where(amax > 0, f32(two688 / amax), np.float32(1.0))
        big_s = np.minimum(big_s, FLT_MAX).astype(np.float32)
        blocks = x.reshape(live, cols // NVFP4_BLOCK, NVFP4_BLOCK)
        bmax = np.abs(blocks).max(axis=2)
        s_f = f32(f32(bmax / np.float32(E2M1_MAX)) * big_s[:, None])
        s8 = e4m3_encode(s_f.astype(np.float64))
        sd = f32(e4m3_decode(s8))
        enc = np.where(sd == 0, np.float32(0.0), np.minimum(f32(big_s[:, None] / sd), FLT_MAX))
        enc = enc.astype(np.float32)
        v = f32(blocks * enc[..., None])
    q = e2m1_encode(v.astype(np.float64)).reshape(live, cols)
    return fp4_pack(q), s8, tsi.astype(np.float32)


def nvfp4_rowscaled_colwise(x_bits, offsets, padded_offsets):
    """Columnwise (transposed) row-scaled NVFP4 quantize for a contraction over
    ragged token rows (wgrad).  "[Common][PyTorch] Add row-scaled NVFP4 support
    to grouped-tensor GEMM" lifts the ban on columnwise use of row-scaled
    grouped tensors so that wgrad can consume the transpose, with the
    columnwise amax sized per column and split per expert.

    Reading: per group g, the transposed block X_g^T [C, m~_g] -- tokens padded
    with zeros to m~_g, a multiple of 128, as for the MXFP8 columnwise copies --
    is quantized row by row exactly as ``nvfp4_rowscaled`` quantizes rows, so
    column c of group g gets its own outer scale tsi[g, c] = (largest |x| over
    the group's tokens) / 2688 and 16-token blocks with E4M3 scales.

    Layout: group g's packed E2M1 data is a row-major [C, m~_g / 2] block at
    byte offset padded_offsets[g] * C / 2 (token 2j in the low nibble of byte
    j), its E4M3 block scales a row-major [C, m~_g / 16] block at
    padded_offsets[g] * C / 16, and the outer scales an f32 [G, C] array (0 for
    an empty group).  Returns (data, block_scales, outer)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    off = np.asarray(offsets, dtype=np.int64)
    poff = np.asarray(padded_offsets, dtype=np.int64)
    G = len(off) - 1
    if int(off[-1]) > rows:
        raise ValueError("sum of group sizes exceeds the row capacity")
    data = np.zeros(int(poff[-1]) * cols // 2, dtype=np.uint8)
    bscales = np.zeros(int(poff[-1]) * cols // NVFP4_BLOCK, dtype=np.uint8)
    outer = np.zeros((G, cols), dtype=np.float32)
    for g in range(G):
        m = int(off[g + 1] - off[g])
        mp = int(poff[g + 1] - poff[g])
        if mp < m or mp % COLWISE_PAD:
            raise ValueError("padded offsets inconsistent with the group sizes")
        if mp == 0:
            continue
        xt = np.zeros((cols, mp), dtype=np.uint16)              # +0.0 padding
        xt[:, :m] = x_bits[off[g]:off[g + 1]].T
        packed, s8, tsi = nvfp4_rowscaled(xt, np.array([0, cols]))
        data[poff[g] * cols // 2:poff[g + 1] * cols // 2] = packed.reshape(-1)
        bscales[poff[g] * cols // NVFP4_BLOCK:poff[g + 1] * cols // NVFP4_BLOCK] = s8.reshape(-1)
        outer[g] = tsi
    return data, bscales, outer


def nvfp4_tensor_scale_inv(amax):
    """Tensor-level NVFP4 outer scale, amax / (E2M1 max * E4M3 max) = amax /
    2688, in float32 ("gemm.py", ``_get_nvfp4_tensor_scale_inv``)."""
    return f32(np.asarray(amax, dtype=np.float32) / np.float32(E2M1_MAX * E4M3_MAX))


def nvfp4_pertensor(x_bits, offsets):
    """Per-tensor NVFP4 quantize of grouped live rows, each group (expert) one
    tensor: "gemm.py" derives an NVFP4 operand's outer scale from the tensor's
    amax (``_get_nvfp4_tensor_scale_inv``, alpha = the product of the two
    operands' outer scales); split per expert, each group carries its own amax
    ("[Common][PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM":
    one amax entry per split for tensor-scaled quantizers).

    Reading: the float32 steps of ``nvfp4_rowscaled`` with the row's amax
    replaced by the group's,
      S_g  = 2688 / amax_g (1 if amax_g == 0; capped at FLT_MAX)
      s_f  = (bmax / 6) * S_g        -> s8 = E4M3(s_f), sd = decode(s8)
      enc  = S_g / sd (0 if sd == 0; capped at FLT_MAX)
      q    = E2M1(x * enc)
    so that x ~= e2m1(q) * sd * tsi_g, tsi_g = amax_g / 2688.  An empty group
    has amax 0.  The groups start at row 0 (offsets[0] == 0).

    Returns (packed [live, C/2] uint8, block scales [live, C/16] uint8 E4M3,
    amax [G] float32)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    live = int(np.asarray(offsets)[-1])
    if live > rows:
        raise ValueError("sum of group sizes exceeds the row capacity")
    return nvfp4_pertensor_values(f32(bf16_bits_to_f64(x_bits[:live])), offsets)


def nvfp4_pertensor_values(x, offsets):
    """``nvfp4_pertensor`` of float32 values x [live, C] (the bf16 inputs, or
    their randomized Hadamard transform)."""
    x = np.asarray(x, dtype=np.float32)
    live, cols = x.shape
    off = np.asarray(offsets, dtype=np.int64)
    G = len(off) - 1
    if int(off[0]) != 0 or int(off[-1]) != live:
        raise ValueError("offsets must run from 0 to the live rows")
    if np.any(np.diff(off) < 0):
        raise ValueError("negative group size")
    two688 = np.float32(E2M1_MAX * E4M3_MAX)
    amax = np.zeros(G, np.float32)
    for g in range(G):
        if off[g + 1] > off[g] and cols:
            amax[g] = np.abs(x[off[g]:off[g + 1]]).max()
    # each live row takes its group's S
    row_group = np.repeat(np.arange(G), np.diff(off))
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        big_s_g = np.where(amax > 0, f32(two688 / amax), np.float32(1.0))
        big_s_g = np.minimum(big_s_g, FLT_MAX).astype(np.float32)
        big_s = big_s_g[row_group]
        blocks = x.reshape(live, cols // NVFP4_BLOCK, NVFP4_BLOCK)
        bmax = np.abs(blocks).max(axis=2)
        s_f = f32(f32(bmax / np.float32(E2M1_MAX)) * big_s[:, None])
        s8 = e4m3_encode(s_f.astype(np.float64))
        sd = f32(e4m3_decode(s8))
        enc = np.where(sd == 0, np.float32(0.0), np.minimum(f32(big_s[:, None] / sd), FLT_MAX))
        enc = enc.astype(np.float32)
        v = f32(blocks * enc[..., None])
    q = e2m1_encode(v.astype(np.float64)).reshape(live, cols)
    return fp4_pack(q), s8, amax


def nvfp4_pertensor_rht(x_bits, offsets, sign_mask):
    """Per-tensor NVFP4 of the randomized Hadamard transform of the rows
    ("gemm.py", ``_quantize_gemm_operands``: with NVFP4 1-D scaling both GEMM
    operands carry the RHT so that it cancels; transform in ``oracle.rht``):
    the rows' 16-element blocks along the contraction are transformed in
    float32, then quantized exactly as ``nvfp4_pertensor`` quantizes values, the
    group amax taken over the transformed values.  Returns what
    ``nvfp4_pertensor`` returns."""
    from .rht import rht16
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    live = int(np.asarray(offsets)[-1])
    if live > rows:
        raise ValueError("sum of group sizes exceeds the row capacity")
    return nvfp4_pertensor_values(rht16(f32(bf16_bits_to_f64(x_bits[:live])), sign_mask), offsets)


def nvfp4_pertensor_2d(x_bits, offsets):
    """Per-tensor NVFP4 with 2-D block scales ("gemm.py", ``_jax_scaled_matmul``
    accepts an ``NVFP4_2D_SCALING`` mode next to the 1-D one; the pages give no
    block shape).  Reading: one E4M3 scale per 16 x 16 block -- 16 rows by 16
    columns, the NVFP4 block size in both directions, so that a tensor and its
    transpose quantize to transposed codes -- with the float32 steps of
    ``nvfp4_pertensor`` and the block maximum taken over the whole 16 x 16
    block.  Block rows start at each group's first row; a group's last block
    row holds its remaining (fewer than 16) rows.  The group's amax and outer
    scale are the per-tensor ones.  The scales are written in the GEMM's
    per-row layout: each row of a block row carries its block's scale byte, so
    ``grouped_gemm_nvfp4_pertensor`` consumes the result unchanged.  Returns
    what ``nvfp4_pertensor`` returns."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    rows, cols = x_bits.shape
    if cols % MX_BLOCK:
        raise ValueError("cols must be a multiple of 32")
    off = np.asarray(offsets, dtype=np.int64)
    live = int(off[-1])
    if live > rows or int(off[0]) != 0 or np.any(np.diff(off) < 0):
        raise ValueError("offsets must run from 0 to at most the row capacity")
    x = f32(bf16_bits_to_f64(x_bits[:live]))
    G = len(off) - 1
    two688 = np.float32(E2M1_MAX * E4M3_MAX)
    nb = cols // NVFP4_BLOCK
    codes = np.zeros((live, cols), np.uint8)
    s8 = np.zeros((live, nb), np.uint8)
    amax = np.zeros(G, np.float32)
    with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
        for g in range(G):
            r0, r1 = int(off[g]), int(off[g + 1])
            if r1 == r0:
                continue
            amax[g] = np.abs(x[r0:r1]).max() if cols else np.float32(0)
            big_s = f32(two688 / amax[g]) if amax[g] > 0 else np.float32(1.0)
            big_s = np.float32(min(big_s, FLT_MAX))
            for b0 in range(r0, r1, NVFP4_BLOCK):
                b1 = min(b0 + NVFP4_BLOCK, r1)
                blk = x[b0:b1].reshape(b1 - b0, nb, NVFP4_BLOCK)
                bmax = np.abs(blk).max(axis=(0, 2))                    # [nb]
                s_f = f32(f32(bmax / np.float32(E2M1_MAX)) * big_s)
                sc = e4m3_encode(s_f.astype(np.float64))
                sd = f32(e4m3_decode(sc))
                enc = np.where(sd == 0, np.float32(0.0), np.minimum(f32(big_s / sd), FLT_MAX))
                enc = enc.astype(np.float32)
                v = f32(blk * enc[None, :, None])
                codes[b0:b1] = e2m1_encode(v.astype(np.float64)).reshape(b1 - b0, cols)
                s8[b0:b1] = sc[None, :]
    return fp4_pack(codes), s8, amax


def nvfp4_block_dequant(packed, block_scales, cols):
    """E2M1 element times its decoded E4M3 block scale (no outer scale)."""
    q = fp4_unpack(np.asarray(packed).reshape(-1, cols // 2))
    vals = e2m1_decode(q).reshape(q.shape[0], cols // NVFP4_BLOCK, NVFP4_BLOCK)
    sd = e4m3_decode(np.asarray(block_scales).reshape(q.shape[0], cols // NVFP4_BLOCK))
    return (vals * sd[..., None]).reshape(q.shape[0], cols)


def nvfp4_dequant(packed, block_scales, tsi, cols):
    """Full Q->DQ: e2m1 * block scale * outer scale."""
    return nvfp4_block_dequant(packed, block_scales, cols) * \
        np.asarray(tsi, dtype=np.float64)[:, None]


def mx_scale_words(cols):
    """Number of 4-byte scale words (128-element groups) per MXFP8 row."""
    return mx_scale_row_bytes(cols // MX_BLOCK) // 4
