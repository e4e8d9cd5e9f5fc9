"""Byte layouts the quantizers write and the GEMMs read (oracle; test infrastructure only).

"[JAX] MXFP8 Grouped Quant+GEMM" (description; Greptile summary) moves the scale
swizzle out of the GEMM and into the quantize: the quantize writes its scales
directly in the order the GEMM consumes, and the Q->DQ test dequantizer first
undoes that order.  The order itself is the GEMM's business (the pages' one is
the cuBLAS 128x4 tile swizzle of "gemm.py", ``swizzled_scale``).  This build's
order is row-local, so any group start row needs no padding, and the scale
offset of a group is its data offset / 32 (the relation the V2 setup kernel
uses, review thread on ``gemm.py`` in the same PR):

* MXFP8 scale rows.  A row with ``n_blk = K / 32`` logical scale bytes
  ``b_0 .. b_{n_blk-1}`` is stored in ``roundup(n_blk, 4)`` bytes.  Within each
  group of four logical bytes (one 128-element stretch of the row) the stored
  order is ``b_0, b_2, b_1, b_3``; bytes a short last group lacks are 0x00.
* NVFP4 block-scale rows are stored in logical order (identity).
* NVFP4 data: element 2j in the low nibble of byte j, element 2j+1 in the high.

The functions here implement the order and its inverse; the tests check that
one undoes the other.
"""

import numpy as np

MX_GROUP = 4                       # logical scale bytes per permutation group
MX_PERM = (0, 2, 1, 3)             # stored position i holds logical byte MX_PERM[i]


def mx_scale_row_bytes(n_blk):
    """Stored bytes per MXFP8 scale row with n_blk logical scale bytes."""
    return ((n_blk + MX_GROUP - 1) // MX_GROUP) * MX_GROUP


def mx_scales_to_gemm_order(logical):
    """[R, n_blk] logical E8M0 bytes -> [R, roundup(n_blk, 4)] stored bytes."""
    logical = np.asarray(logical, dtype=np.uint8)
    rows, n_blk = logical.shape
    width = mx_scale_row_bytes(n_blk)
    padded = np.zeros((rows, width), dtype=np.uint8)
    padded[:, :n_blk] = logical
    stored = np.zeros_like(padded)
    for grp in range(width // MX_GROUP):
        base = grp * MX_GROUP
        for pos in range(MX_GROUP):
            stored[:, base + pos] = padded[:, base + MX_PERM[pos]]
    return stored


def mx_scales_from_gemm_order(stored, n_blk):
    """Inverse of ``mx_scales_to_gemm_order``: [R, roundup(n_blk, 4)] -> [R, n_blk]."""
    stored = np.asarray(stored, dtype=np.uint8)
    rows, width = stored.shape
    if width != mx_scale_row_bytes(n_blk):
        raise ValueError("stored scale row width does not match n_blk")
    logical = np.zeros((rows, width), dtype=np.uint8)
    for grp in range(width // MX_GROUP):
        base = grp * MX_GROUP
        for pos in range(MX_GROUP):
            logical[:, base + MX_PERM[pos]] = stored[:, base + pos]
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
