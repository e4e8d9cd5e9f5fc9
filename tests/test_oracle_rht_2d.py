"""Pins of the oracle's randomized Hadamard transform and of the per-tensor
NVFP4 variants built on it (RHT) and on 2-D block scales, against mathematics
that does not come from the oracle: the Sylvester construction of H16 by
Kronecker products, orthogonality, exact integer arithmetic, transposition,
hand-worked blocks and the 1-D per-tensor oracle (pinned elsewhere)."""

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as GM
from oracle import quantize as Q
from oracle import rht as R


def _h16():
    h2 = np.array([[1, 1], [1, -1]], dtype=np.float64)
    h = h2
    for _ in range(3):
        h = np.kron(h, h2)
    return h


def test_transform_matrix_is_sylvester_hadamard_over_four():
    eye = np.eye(16, dtype=np.float32)
    m = R.rht16(eye, 0).astype(np.float64).T      # column i = transform of e_i
    assert np.array_equal(m, _h16() / 4)
    assert np.array_equal(m @ m.T, np.eye(16))


@pytest.mark.parametrize("mask", [0x0001, 0x8000, 0xA5C3, 0xFFFF])
def test_signs_multiply_the_columns(mask):
    eye = np.eye(16, dtype=np.float32)
    m = R.rht16(eye, mask).astype(np.float64).T
    s = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
    assert np.array_equal(m, (_h16() / 4) * s[None, :])


def test_hand_worked_blocks():
    e0 = np.zeros(16, np.float32)
    e0[0] = 1
    assert np.array_equal(R.rht16(e0, 0), np.full(16, 0.25, np.float32))
    ones = np.ones(16, np.float32)
    want = np.zeros(16, np.float32)
    want[0] = 4
    assert np.array_equal(R.rht16(ones, 0), want)
    assert np.array_equal(R.rht16(ones, 0xFFFF), -want)
    alt = np.array([1, -1] * 8, np.float32)        # the second Hadamard row: all mass at index 1
    want = np.zeros(16, np.float32)
    want[1] = 4
    assert np.array_equal(R.rht16(alt, 0), want)


def test_exact_on_small_integers_and_blockwise():
    rng = np.random.default_rng(3)
    x = rng.integers(-50, 51, (5, 64)).astype(np.float32)
    mask = 0x3C5A
    y = R.rht16(x, mask).astype(np.float64)
    s = R.sign_vector(mask).astype(np.float64)
    q = (_h16() / 4) * s[None, :]
    want = (x.astype(np.float64).reshape(5, 4, 16) @ q.T).reshape(5, 64)
    assert np.array_equal(y, want)


def test_transform_cancels_in_the_product():
    """(A Q^T)(B Q^T)^T = A B^T for the same transform on both operands: the
    property that lets both GEMM operands carry the RHT (float32 rounding of
    the transform only)."""
    rng = np.random.default_rng(4)
    a = rng.standard_normal((24, 96)).astype(np.float32)
    b = rng.standard_normal((40, 96)).astype(np.float32)
    mask = 0x9E37
    ya = R.rht16(a, mask).astype(np.float64)
    yb = R.rht16(b, mask).astype(np.float64)
    want = a.astype(np.float64) @ b.astype(np.float64).T
    assert np.max(np.abs(ya @ yb.T - want)) <= 1e-5 * np.max(np.abs(want))
    # with different transforms the product is not preserved
    yb2 = R.rht16(b, mask ^ 1).astype(np.float64)
    assert np.max(np.abs(ya @ yb2.T - want)) > 0.05 * np.max(np.abs(want))


def _bits(rng, shape, std=1.0):
    return F.f32_to_bf16_bits_rne((rng.standard_normal(shape) * std).astype(np.float32))


def test_pertensor_rht_quantizes_the_transformed_rows():
    rng = np.random.default_rng(5)
    xb = _bits(rng, (70, 64))
    off = np.array([0, 30, 30, 70])
    mask = 0x1234
    p, s8, am = Q.nvfp4_pertensor_rht(xb, off, mask)
    y = R.rht16(F.bf16_bits_to_f64(xb).astype(np.float32), mask)
    p2, s82, am2 = Q.nvfp4_pertensor_values(y, off)
    assert np.array_equal(p, p2) and np.array_equal(s8, s82) and np.array_equal(am, am2)
    for g in range(3):
        if off[g + 1] > off[g]:
            assert am[g] == np.abs(y[off[g]:off[g + 1]]).max()
    assert am[1] == 0
    # identity transform (no signs, H16 / 4 is not the identity) changes the codes
    p0, _, _ = Q.nvfp4_pertensor(xb, off)
    assert not np.array_equal(p0, p)


def test_rht_gemm_approximates_the_untransformed_product():
    """Both operands transformed with the same signs: the NVFP4 GEMM of the
    transformed, quantized operands approximates A W^T (the transform cancels;
    what remains is the NVFP4 quantization error); with different signs it
    does not."""
    rng = np.random.default_rng(6)
    K, M, N = 256, 48, 64
    xb, wb = _bits(rng, (M, K)), _bits(rng, (N, K), 0.02)
    want = F.bf16_bits_to_f64(xb) @ F.bf16_bits_to_f64(wb).T
    off, boff = np.array([0, M]), np.array([0, N])
    mask = 0xBEEF

    def product(ma, mb):
        a = Q.nvfp4_pertensor_rht(xb, off, ma)
        b = Q.nvfp4_pertensor_rht(wb, boff, mb)
        (_, y), = GM.nvfp4_pertensor_fprop(a[0], a[1], a[2], off, b[0], b[1], b[2], [N], K)
        return y

    err = np.linalg.norm(product(mask, mask) - want) / np.linalg.norm(want)
    # the same quantization without the transform: errors of one size
    a = Q.nvfp4_pertensor(xb, off)
    b = Q.nvfp4_pertensor(wb, boff)
    (_, y0), = GM.nvfp4_pertensor_fprop(a[0], a[1], a[2], off, b[0], b[1], b[2], [N], K)
    err0 = np.linalg.norm(y0 - want) / np.linalg.norm(want)
    assert err < 1.5 * err0 and err0 < 0.2, (err, err0)
    bad = np.linalg.norm(product(mask, mask ^ 0x0101) - want) / np.linalg.norm(want)
    assert bad > 0.5, bad


def test_2d_blocks_are_transposable():
    """A 16 x 16 block quantizes to the same codes whichever way the tensor is
    laid out: the 2-D quantize of X^T is the transpose of that of X."""
    rng = np.random.default_rng(7)
    xb = _bits(rng, (64, 96))
    p, s8, am = Q.nvfp4_pertensor_2d(xb, np.array([0, 64]))
    pt, s8t, amt = Q.nvfp4_pertensor_2d(np.ascontiguousarray(xb.T), np.array([0, 96]))
    codes = np.zeros((64, 96), np.uint8)
    codes[:, 0::2], codes[:, 1::2] = p & 0xF, p >> 4
    codes_t = np.zeros((96, 64), np.uint8)
    codes_t[:, 0::2], codes_t[:, 1::2] = pt & 0xF, pt >> 4
    assert np.array_equal(codes, codes_t.T)
    assert np.array_equal(s8[::16, :], s8t[::16, :].T)      # one byte per 16 x 16 block
    assert np.all(s8.reshape(4, 16, 6) == s8[::16][:, None, :])
    assert am[0] == amt[0]


def test_2d_reduces_to_1d_when_every_row_holds_its_block_max():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((48, 64)).astype(np.float32)
    # put each 16 x 16 block's largest magnitude into column 0 of every row of it
    for b0 in range(0, 48, 16):
        for c0 in range(0, 64, 16):
            blk = x[b0:b0 + 16, c0:c0 + 16]
            m = np.abs(blk).max() * 1.0625
            blk[:, 0] = np.where(np.arange(16) % 2 == 0, m, -m)
    xb = F.f32_to_bf16_bits_rne(x)
    off = np.array([0, 16, 48])
    assert np.array_equal(np.array(Q.nvfp4_pertensor_2d(xb, off), dtype=object)[0],
                          Q.nvfp4_pertensor(xb, off)[0])
    a2, a1 = Q.nvfp4_pertensor_2d(xb, off), Q.nvfp4_pertensor(xb, off)
    for u, v in zip(a2, a1):
        assert np.array_equal(u, v)


def test_2d_hand_worked_block():
    """Two 16 x 16 blocks, every element 0.5 but a single 6.0 in the first;
    group amax 6, so S = 448.  First block: scale E4M3(6 / 6 * 448) = 0x7E,
    enc = 1, 6.0 -> code 7 and 0.5 -> code 1 in all 16 rows.  Second block:
    scale E4M3(0.5 / 6 * 448 = 37.33) = 36 = 0x61, enc = 448 / 36, 0.5 -> 6.22
    -> code 7.  (The 1-D scales would give the first block's rows without the 6
    the second block's treatment: scale 0x61, code 7.)"""
    x = np.full((16, 32), 0.5, np.float32)
    x[3, 5] = 6.0
    xb = F.f32_to_bf16_bits_rne(x)
    p, s8, am = Q.nvfp4_pertensor_2d(xb, np.array([0, 16]))
    assert am[0] == 6.0
    assert np.all(s8[:, 0] == 0x7E) and np.all(s8[:, 1] == 0x61)
    want = np.full((16, 16), 0x11, np.uint8)
    want[:, 8:] = 0x77
    want[3, 2] = 0x71                 # element 5 is the high nibble of byte 2
    assert np.array_equal(p, want)
    p1, s1, _ = Q.nvfp4_pertensor(xb, np.array([0, 16]))
    assert s1[0, 0] == 0x61 and p1[0, 0] == 0x77 and p1[3, 2] == 0x71


def test_2d_block_rows_restart_at_each_group():
    """Groups of 20 and 30 rows: block rows [0, 16), [16, 20), [20, 36) and
    [36, 50), not windows of 16 absolute rows; a large value in row 17 scales
    only the block row [16, 20)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((50, 32)).astype(np.float32)
    x[17, 3] = 40.0
    xb = F.f32_to_bf16_bits_rne(x)
    p, s8, am = Q.nvfp4_pertensor_2d(xb, np.array([0, 20, 50]))
    xv = F.bf16_bits_to_f64(xb)
    assert am[0] == 40.0 and am[1] == np.abs(xv[20:50]).max()
    assert np.all(s8[16:20, 0] == 0x7E) and np.all(s8[0:16] == s8[0]) and s8[0, 0] != 0x7E
    for b0, b1 in ((20, 36), (36, 50)):
        assert np.all(s8[b0:b1] == s8[b0])
    # each group quantizes exactly as it would alone: blocks do not cross groups
    for r0, r1 in ((0, 20), (20, 50)):
        pg, sg, ag = Q.nvfp4_pertensor_2d(xb[r0:r1], np.array([0, r1 - r0]))
        assert np.array_equal(p[r0:r1], pg) and np.array_equal(s8[r0:r1], sg)
