"""Randomized Hadamard transform applied to NVFP4 operands along the contraction
dimension (oracle; test infrastructure only).

"gemm.py", ``_quantize_gemm_operands``: with NVFP4 1-D scaling, an operand
quantized with RHT must meet another quantized with RHT, so that the transform
is applied to both and cancels in the GEMM.  The pages name neither the
transform's size nor its sign vector.  Reading taken here: the transform acts
on each 16-element block along the contraction (the NVFP4 block), as

    y = (1/4) * H16 * diag(s) * x,

H16 the 16 x 16 Sylvester Hadamard matrix (H16[i, j] = (-1)^popcount(i & j)),
s a vector of 16 signs given by the caller as a 16-bit mask (bit i set: s_i =
-1).  (1/4) H16 diag(s) is orthogonal, so for two operands transformed alike
A' B'^T = A Q^T Q B^T = A B^T.  Because the transformed values are then
quantized, the float32 arithmetic is part of the definition: the sign is
applied first (exact), then the butterfly of four stages d = 1, 2, 4, 8, each
replacing (y[i], y[i + d]) by (y[i] + y[i + d], y[i] - y[i + d]) for the i with
bit d clear, every operation rounded to float32, then the product by 1/4
(exact).  Parity unpinned by the pages: this order is a reading.
"""

import numpy as np

RHT_BLOCK = 16


def sign_vector(mask):
    """16 float32 signs from a 16-bit mask (bit i set -> -1)."""
    bits = (int(mask) >> np.arange(RHT_BLOCK)) & 1
    return np.where(bits == 1, np.float32(-1.0), np.float32(1.0)).astype(np.float32)


def rht16(x, mask):
    """The transform of every 16-element block along the last axis of float32
    array ``x`` (last dim a multiple of 16), in the float32 steps above."""
    x = np.asarray(x, dtype=np.float32)
    if x.shape[-1] % RHT_BLOCK:
        raise ValueError("last dim must be a multiple of 16")
    y = x.reshape(x.shape[:-1] + (x.shape[-1] // RHT_BLOCK, RHT_BLOCK)) * sign_vector(mask)
    y = y.astype(np.float32)
    for d in (1, 2, 4, 8):
        lo = np.array([i for i in range(RHT_BLOCK) if not i & d])
        u = y[..., lo].copy()
        v = y[..., lo + d].copy()
        y[..., lo] = (u + v).astype(np.float32)
        y[..., lo + d] = (u - v).astype(np.float32)
    y = (y * np.float32(0.25)).astype(np.float32)
    return y.reshape(x.shape)
