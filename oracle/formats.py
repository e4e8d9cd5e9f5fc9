"""Element and scale codecs of the block-scaled formats (oracle; test infrastructure only).

MXFP8 (the ``MXFP8_1D_SCALING`` mode of "gemm.py", ``_jax_scaled_matmul``; the
32-element blocks are described in the review of "[JAX] MXFP8 Grouped
Quant+GEMM"): E4M3 elements sharing one E8M0 power-of-two scale per 32 elements
along the contraction dimension.

NVFP4 ("gemm.py", ``_get_nvfp4_tensor_scale_inv``; "[Common][PyTorch] Add
row-scaled NVFP4 support to grouped-tensor GEMM"): E2M1 elements, one E4M3 scale
per 16 elements, and an FP32 outer scale.

Everything here works on exact values: inputs are bf16 or fp32 numbers held in
float64 (which represents them exactly), and rounding to a format's grid is
written out as "divide by the grid quantum, round half to even, multiply back".
Codes are returned as uint8.
"""

import numpy as np

# E4M3 ("fn" variant: no infinities, only 0x7F/0xFF are NaN): bias 7, 3 mantissa bits.
E4M3_BIAS = 7
E4M3_MAN_BITS = 3
E4M3_MAX = 448.0          # 1.75 * 2**8, code 0x7E
E4M3_EMAX = 8             # exponent of E4M3_MAX
E4M3_EMIN = -6            # exponent of the smallest normal value (2**-6); subnormal step 2**-9

# E5M2 (exponent field 31 holds infinities and NaNs): bias 15, 2 mantissa bits.
E5M2_BIAS = 15
E5M2_MAN_BITS = 2
E5M2_MAX = 57344.0        # 1.75 * 2**15, code 0x7B
E5M2_EMAX = 15            # exponent of E5M2_MAX
E5M2_EMIN = -14           # exponent of the smallest normal value; subnormal step 2**-16

# E2M1: bias 1, 1 mantissa bit; grid {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
E2M1_MAX = 6.0
E2M1_EMIN = 0
E2M1_MAN_BITS = 1

E8M0_BIAS = 127


def bf16_bits_to_f64(bits):
    """bf16 bit patterns (uint16) -> exact float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    # signalling-NaN patterns become quiet NaNs when widened; numpy flags that
    # as an invalid operation, which is expected here
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def f32_to_bf16_bits_rne(x):
    """float32 values -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def _round_to_grid(a, emin, man_bits):
    """Round non-negative exact values ``a`` to the nearest point of a binary
    floating-point grid with ``man_bits`` mantissa bits and minimum normal
    exponent ``emin`` (subnormals below it), ties to even.  No saturation."""
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(a)                    # a = m * 2**ex, m in [0.5, 1)
    e = np.maximum(ex - 1, emin)           # exponent of the binade (or of the subnormal range)
    quantum = np.ldexp(1.0, e - man_bits)  # spacing of the grid in that binade
    return np.round(a / quantum) * quantum  # np.round rounds half to even


def e4m3_encode(v):
    """Exact values -> E4M3 codes, round half to even, saturating to +-448.

    Sign is kept (negative values that round to zero give 0x80).  Values whose
    magnitude reaches or exceeds 448 give 0x7E / 0xFE, never NaN."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E4M3 encode: non-finite input is outside the contract")
    neg = np.signbit(v)
    r = np.minimum(_round_to_grid(np.abs(v), E4M3_EMIN, E4M3_MAN_BITS), E4M3_MAX)
    code = np.zeros(r.shape, dtype=np.int64)
    sub = r < 2.0 ** E4M3_EMIN
    code[sub] = np.rint(r[sub] * 2.0 ** 9).astype(np.int64)            # exponent field 0
    m, ex = np.frexp(r[~sub])
    exp_field = (ex - 1) + E4M3_BIAS
    man_field = np.rint((m * 2.0 - 1.0) * 2 ** E4M3_MAN_BITS).astype(np.int64)
    code[~sub] = (exp_field << 3) | man_field
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(code):
    """E4M3 codes -> float64 values (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(code, dtype=np.int64)
    exp_field = (c >> 3) & 0xF
    man_field = c & 0x7
    mag = np.where(exp_field == 0,
                   man_field * 2.0 ** -9,
                   (1.0 + man_field / 8.0) * np.ldexp(1.0, exp_field - E4M3_BIAS))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def e5m2_encode(v):
    """Exact values -> E5M2 codes, round half to even, saturating to +-57344.

    Reading: the pages pair E5M2 gradients with E4M3 operands ("gemm.py",
    ``_compatible_fp8_gemm_dtypes``) but fix no overflow rule; the MX scale
    leaves a block's maximum below 2**16, and values that round past the
    largest finite E5M2 value saturate to it, as the E4M3 elements saturate to
    448, so a finite input never becomes an infinity."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E5M2 encode: non-finite input is outside the contract")
    neg = np.signbit(v)
    r = np.minimum(_round_to_grid(np.abs(v), E5M2_EMIN, E5M2_MAN_BITS), E5M2_MAX)
    code = np.zeros(r.shape, dtype=np.int64)
    sub = r < 2.0 ** E5M2_EMIN
    code[sub] = np.rint(r[sub] * 2.0 ** 16).astype(np.int64)           # exponent field 0
    m, ex = np.frexp(r[~sub])
    exp_field = (ex - 1) + E5M2_BIAS
    man_field = np.rint((m * 2.0 - 1.0) * 2 ** E5M2_MAN_BITS).astype(np.int64)
    code[~sub] = (exp_field << 2) | man_field
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def e5m2_decode(code):
    """E5M2 codes -> float64 values (exponent field 31: infinity or NaN)."""
    c = np.asarray(code, dtype=np.int64)
    exp_field = (c >> 2) & 0x1F
    man_field = c & 0x3
    mag = np.where(exp_field == 0,
                   man_field * 2.0 ** -16,
                   (1.0 + man_field / 4.0) * np.ldexp(1.0, exp_field - E5M2_BIAS))
    mag = np.where(exp_field == 31, np.where(man_field == 0, np.inf, np.nan), mag)
    return np.where(c & 0x80, -mag, mag)


def e2m1_encode(v):
    """Exact values -> E2M1 codes (4-bit, sign in bit 3), round half to even,
    saturating to +-6."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("E2M1 encode: non-finite input is outside the contract")
    neg = np.signbit(v)
    r = np.minimum(_round_to_grid(np.abs(v), E2M1_EMIN, E2M1_MAN_BITS), E2M1_MAX)
    code = np.zeros(r.shape, dtype=np.int64)
    sub = r < 1.0
    code[sub] = np.rint(r[sub] * 2.0).astype(np.int64)                 # 0 or 0.5
    m, ex = np.frexp(r[~sub])
    code[~sub] = ((ex - 1 + 1) << 1) | np.rint((m * 2.0 - 1.0) * 2).astype(np.int64)
    return (code | (neg.astype(np.int64) << 3)).astype(np.uint8)


def e2m1_decode(code):
    """E2M1 codes (low 4 bits) -> float64 values."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    exp_field = (c >> 1) & 0x3
    man_field = c & 0x1
    mag = np.where(exp_field == 0, man_field * 0.5,
                   (1.0 + man_field / 2.0) * np.ldexp(1.0, exp_field - 1))
    return np.where(c & 0x8, -mag, mag)


def e8m0_decode(byte):
    """E8M0 scale bytes -> 2**(byte - 127) (0xFF is NaN)."""
    b = np.asarray(byte, dtype=np.int64)
    return np.where(b == 0xFF, np.nan, np.ldexp(1.0, b - E8M0_BIAS))


def e8m0_from_amax(amax, emax=E4M3_EMAX):
    """Shared MX scale of a block from its largest magnitude.

    Reading (the pages give only the 32-element block): the OCP Microscaling
    v1.0 rule, scale exponent = floor(log2(amax)) - emax of the element format
    (8 for E4M3, 15 for E5M2), biased by 127 and clamped to [0, 254].  A block
    of zeros gets byte 0.  For E4M3 the block maximum then lands in [256, 512)
    before saturation, so values in (448, 512) saturate to 448; for E5M2 in
    [2**15, 2**16), values above 57344 saturating."""
    a = np.asarray(amax, dtype=np.float64)
    _, ex = np.frexp(a)                         # floor(log2(a)) == ex - 1 for a > 0
    byte = np.clip((ex - 1) - emax + E8M0_BIAS, 0, 254)
    return np.where(a > 0, byte, 0).astype(np.uint8)


def f32(x):
    """Round to float32 (the precision the NVFP4 recipe's scale arithmetic is defined in)."""
    return np.asarray(x, dtype=np.float32)
