"""GPU parity of the per-tensor NVFP4 variants: the randomized Hadamard
transform of the rows along the contraction (both GEMM operands transformed
alike, so the transform cancels) and 2-D (16 x 16) block scales.  Quantized
bytes and amax bit-exact against the oracle; GEMMs of the GPU-quantized
operands within the GEMM tolerance of the oracle's."""

import numpy as np
import pytest
import torch

import block_scaled_grouped_amd as bsg
from oracle import formats as F
from oracle import gemm as GM
from oracle import offsets as O
from oracle import quantize as Q
import workloads
from gpu_util import (SENTINEL, bf16_dev, device, filled_u8, gemm_tolerance_check, host, host_u8,
                      to_dev)

pytestmark = pytest.mark.gpu


def _bits(rng, rows, cols, spread=8, outliers=0.01):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-spread, spread + 1, (rows, 1))).astype(np.float32)
    x[rng.random((rows, cols)) < outliers] *= 20
    return F.f32_to_bf16_bits_rne(x)


CASES = [
    (400, 4096, [100, 0, 157, 43]),
    (64, 160, [17, 0, 30]),
    (300, 96, [0, 5, 0, 250, 1]),           # leading empty group, a one-row group
    (16, 32, [0]),                          # empty routing: only the amax is written (0)
    (3000, 64, [i % 23 for i in range(256)]),   # 256 groups (the maximum)
    (12, 16416, [3, 0, 5]),                 # longer rows than a thread's registers hold
]


def _run(fn, bits, off, rows_cap, cols, G, *extra):
    d = filled_u8((rows_cap, cols // 2))
    s = filled_u8((rows_cap, cols // 16))
    a = torch.full((G,), float("nan"), dtype=torch.float32, device=device())
    fn(bf16_dev(bits), to_dev(off), *extra, data=d, block_scales=s, amax=a)
    return host_u8(d), host_u8(s), host(a)


@pytest.mark.parametrize("rows_cap,cols,sizes", CASES)
@pytest.mark.parametrize("mask", [0x0000, 0xA5C3])
def test_pertensor_rht_bit_exact(rows_cap, cols, sizes, mask):
    rng = np.random.default_rng(rows_cap + 7 * cols + mask)
    bits = _bits(rng, rows_cap, cols)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS
    if live:
        bits[0] = 0
    _, off = O.group_offsets(sizes)
    wd, ws, wa = Q.nvfp4_pertensor_rht(bits, off, mask)
    d, s, a = _run(bsg.grouped_quantize_nvfp4_pertensor_rht, bits, off, rows_cap, cols,
                   len(sizes), mask)
    assert np.array_equal(a.view(np.uint32), wa.view(np.uint32))
    assert np.array_equal(d[:live], wd)
    assert np.array_equal(s[:live], ws)
    assert np.all(d[live:] == SENTINEL) and np.all(s[live:] == SENTINEL)


@pytest.mark.parametrize("rows_cap,cols,sizes", CASES + [(100, 256, [20, 13, 0, 47])])
def test_pertensor_2d_bit_exact(rows_cap, cols, sizes):
    rng = np.random.default_rng(rows_cap + 11 * cols)
    bits = _bits(rng, rows_cap, cols)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS
    if live:
        bits[0] = 0
    _, off = O.group_offsets(sizes)
    wd, ws, wa = Q.nvfp4_pertensor_2d(bits, off)
    d, s, a = _run(bsg.grouped_quantize_nvfp4_pertensor_2d, bits, off, rows_cap, cols, len(sizes))
    assert np.array_equal(a.view(np.uint32), wa.view(np.uint32))
    assert np.array_equal(d[:live], wd)
    assert np.array_equal(s[:live], ws)
    assert np.all(d[live:] == SENTINEL) and np.all(s[live:] == SENTINEL)


def test_2d_transposed_tensor_gives_transposed_codes():
    rng = np.random.default_rng(12)
    bits = _bits(rng, 64, 96)
    d, s, a = _run(bsg.grouped_quantize_nvfp4_pertensor_2d, bits, np.array([0, 64]), 64, 96, 1)
    dt, st, at = _run(bsg.grouped_quantize_nvfp4_pertensor_2d, np.ascontiguousarray(bits.T),
                      np.array([0, 96]), 96, 64, 1)

    def codes(p, rows, cols):
        c = np.zeros((rows, cols), np.uint8)
        c[:, 0::2], c[:, 1::2] = p & 0xF, p >> 4
        return c

    assert np.array_equal(codes(d, 64, 96), codes(dt, 96, 64).T)
    assert np.array_equal(s[::16], st[::16].T) and a[0] == at[0]


@pytest.mark.parametrize("K", [256, 96])
def test_rht_gemm_end_to_end(K):
    """X and W transformed with the same signs, quantized per tensor on the GPU,
    multiplied by the per-tensor GEMM: within the tolerance of the oracle's
    GEMM over the oracle's operands, and close to the untransformed product."""
    rng = np.random.default_rng(21 + K)
    sizes = np.array([150, 0, 106], np.int32)
    npg = [128, 256, 96]
    live = int(sizes.sum())
    rows_cap = live + 9
    mask = 0x6B2D
    xb = _bits(rng, rows_cap, K, spread=0, outliers=0)
    wb = F.f32_to_bf16_bits_rne((rng.standard_normal((sum(npg), K)) * 0.02).astype(np.float32))
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    doff = to_dev(off)
    a = bsg.grouped_quantize_nvfp4_pertensor_rht(bf16_dev(xb), doff, mask)
    b = bsg.grouped_quantize_nvfp4_pertensor_rht(bf16_dev(wb), to_dev(boff), mask)
    out = torch.full((rows_cap, max(npg)), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_gemm_nvfp4_pertensor(a[0], a[1], a[2], doff, K, b[0], b[1], b[2], npg, out=out,
                                     out_dtype=bsg.BSG_OUT_F32)
    y = host(out).astype(np.float64)
    ap, asc, aam = Q.nvfp4_pertensor_rht(xb, off, mask)
    bp, bsc, bam = Q.nvfp4_pertensor_rht(wb, boff, mask)
    xf, wf = F.bf16_bits_to_f64(xb), F.bf16_bits_to_f64(wb)
    for g, (rows, r) in enumerate(GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, True, "group %d" % g)
            exact = xf[rows] @ wf[boff[g]:boff[g + 1]].T
            assert np.linalg.norm(y[rows][:, :npg[g]] - exact) < 0.25 * np.linalg.norm(exact)
    assert np.all(np.isnan(y[live:]))


def test_2d_weights_gemm_end_to_end():
    """Activations per-tensor 1-D, expert weights with 2-D block scales, through
    the per-tensor GEMM: within the tolerance of the oracle's GEMM."""
    rng = np.random.default_rng(31)
    sizes = np.array([150, 0, 106], np.int32)
    npg = [128, 256, 96]
    K = 256
    live = int(sizes.sum())
    xb = _bits(rng, live, K)
    wb = F.f32_to_bf16_bits_rne((rng.standard_normal((sum(npg), K)) * 0.02).astype(np.float32))
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    a = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(xb), to_dev(off))
    b = bsg.grouped_quantize_nvfp4_pertensor_2d(bf16_dev(wb), to_dev(boff))
    out = torch.full((live, max(npg)), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_gemm_nvfp4_pertensor(a[0], a[1], a[2], to_dev(off), K, b[0], b[1], b[2], npg,
                                     out=out, out_dtype=bsg.BSG_OUT_F32)
    y = host(out).astype(np.float64)
    ap, asc, aam = Q.nvfp4_pertensor(xb, off)
    bp, bsc, bam = Q.nvfp4_pertensor_2d(wb, boff)
    assert np.array_equal(host_u8(b[0]), bp) and np.array_equal(host_u8(b[1]), bsc)
    for g, (rows, r) in enumerate(GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, True, "group %d" % g)


def test_rht_mask_rejected_past_16_bits():
    x = torch.zeros((16, 32), dtype=torch.bfloat16, device=device())
    off = torch.tensor([0, 16], dtype=torch.int64, device=device())
    with pytest.raises(bsg.BsgError):
        bsg.grouped_quantize_nvfp4_pertensor_rht(x, off, 0x10000)
