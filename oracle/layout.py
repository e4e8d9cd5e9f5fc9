"""Byte layouts the quantizers write and the GEMMs read (oracle; test infrastructure only).

"[JAX] MXFP8 Grouped Quant+GEMM" (description; Greptile summary) moves the scale
swizzle out of the GEMM and into the quantize: the quantize writes its scales
directly in the order the GEMM consumes, and the Q->DQ test dequantizer first
undoes that order.  The order itself is the GEMM's business (the pages' one is
the cuBLAS 128x4 tile swizzle of "gemm.py", ``swizzled_scale``).  The
order used here:

* MXFP8 scales of a rowwise tensor with R rows and K columns: NQ = ceil(K/128)
  groups of 128 columns; the scales are an [NQ][R] array of 4-byte words, word
  (q, r) holding row r's logical scale bytes b_4q, b_4q+1, b_4q+2, b_4q+3 in the
  stored order b_4q, b_4q+2, b_4q+1, b_4q+3 (bytes past K/32 are 0x00).  The
  GEMM reads, per 128-wide K-slice, the words of 64 consecutive rows as one
  contiguous 256-byte copy, and the byte order puts the two bytes each half of
  a wavefront needs into one 16-bit half.  Any row's scales are found from its
  row index alone, so a group may start at any row.
* MXFP8 scales of a columnwise copy: group g's block of C columns and m~_g
  padded tokens (a multiple of 128) is an [m~_g/128][C] array of words laid out
  the same way along the token dimension, at byte offset
  padded_offsets[g] * C / 32 -- the group's data offset / 32, the relation the
  V2 setup kernel uses (review thread on ``gemm.py`` in the same PR).
* NVFP4 block-scale rows are stored in logical order (identity).
* NVFP4 data: element 2j in the low nibble of byte j, element 2j+1 in the high.

The functions here implement the orders and their inverses; the tests check
that one undoes the other.
"""

import numpy as np

MX_GROUP = 4                       # logical scale bytes per word (128 elements)
MX_PERM = (0, 2, 1, 3)             # stored byte i of a word holds logical byte MX_PERM[i]


def mx_scale_row_bytes(n_blk):
    """Stored scale bytes per row with n_blk logical scale bytes (4 * NQ)."""
    return ((n_blk + MX_GROUP - 1) // MX_GROUP) * MX_GROUP


def mx_scales_to_gemm_order(logical):
    """[R, n_blk] logical E8M0 bytes -> [NQ, R, 4] stored bytes (word (q, r))."""
    logical = np.asarray(logical, dtype=np.uint8)
    rows, n_blk = logical.shape
    width = mx_scale_row_bytes(n_blk)
    padded = np.zeros((rows, width), dtype=np.uint8)
    padded[:, :n_blk] = logical
    nq = width // MX_GROUP
    stored = np.zeros((nq, rows, MX_GROUP), dtype=np.uint8)
    for q in range(nq):
        for pos in range(MX_GROUP):
            stored[q, :, pos] = padded[:, q * MX_GROUP + MX_PERM[pos]]
    return stored


def mx_scales_from_gemm_order(stored, n_blk):
    """Inverse of ``mx_scales_to_gemm_order``: [NQ, R, 4] -> [R, n_blk]."""
    stored = np.asarray(stored, dtype=np.uint8)
    nq, rows, four = stored.shape
    if four != MX_GROUP or nq * MX_GROUP != mx_scale_row_bytes(n_blk):
        raise ValueError("stored scale array does not match n_blk")
    logical = np.zeros((rows, nq * MX_GROUP), dtype=np.uint8)
    for q in range(nq):
        for pos in range(MX_GROUP):
            logical[:, q * MX_GROUP + MX_PERM[pos]] = stored[q, :, pos]
    return logical[:, :n_blk]


def fp4_pack(codes):
    """[R, C] 4-bit codes (C even) -> [R, C/2] bytes, element 2j in the low nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def fp4_unpack(packed):
    """[R, C/2] bytes -> [R, C] 4-bit codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.zeros((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out
