"""GPU parity over seeded random ragged shapes, end to end: the GPU quantizers'
bytes equal the oracle's, and every GEMM mode's output equals the oracle's
product of those bytes within the GEMM tolerance.  Each case draws the group
count, the group sizes (with empty groups), the output width, a contraction
that is any multiple of 32, the capacity, the output type and (where the
entry point has them) the last-round workspace, the FP32 scratch and the
per-expert output widths; rows and columns past the live ones must stay
untouched."""

import numpy as np
import pytest
import torch

import block_scaled_grouped_amd as bsg
from oracle import formats as F
from oracle import gemm as GM
from oracle import offsets as O
from oracle import quantize as Q
from gpu_util import (bf16_dev, bf16_out_to_f64, device, gemm_tolerance_check, host, host_u8,
                      to_dev)

pytestmark = pytest.mark.gpu

SEEDS = range(10)


def _bits(rng, shape, std=1.0):
    return F.f32_to_bf16_bits_rne((rng.standard_normal(shape) * std).astype(np.float32))


def _sizes(rng, gmax, mmax):
    G = int(rng.integers(1, gmax + 1))
    sizes = rng.integers(0, mmax + 1, G)
    sizes[rng.random(G) < 0.2] = 0
    return sizes.astype(np.int32)


def _workspace(rng):
    return bsg.gemm_workspace(device()) if rng.random() < 0.5 else None


@pytest.mark.parametrize("seed", SEEDS)
def test_random_mxfp8_fprop(seed):
    rng = np.random.default_rng(1000 + seed)
    sizes = _sizes(rng, 12, 400)
    G, live = len(sizes), int(sizes.sum())
    N, K = 32 * int(rng.integers(1, 21)), 32 * int(rng.integers(1, 25))
    rows_cap = live + int(rng.integers(0, 50))
    out_f32 = bool(rng.integers(0, 2))
    x = _bits(rng, (max(rows_cap, 1), K))
    w = _bits(rng, (G * N, K), 0.02)
    _, off = O.group_offsets(sizes)
    woff = np.array([0, G * N])
    qa = bsg.grouped_quantize_mxfp8(bf16_dev(x), to_dev(off))
    qb = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(woff))
    ad, asc = Q.mxfp8_rowwise(x, off)
    bd, bsc = Q.mxfp8_rowwise(w, woff)
    assert np.array_equal(host_u8(qa["row_data"])[:live], ad[:live])
    assert np.array_equal(host_u8(qb["row_data"]), bd)
    assert np.array_equal(host_u8(qb["row_scales"]), bsc)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((max(rows_cap, 1), N), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, qa["row_data"], qa["row_scales"], qb["row_data"],
                           qb["row_scales"], to_dev(off), rows_cap, N, K, out=out,
                           out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                           workspace=_workspace(rng))
    ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g]:
            gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32,
                                 "seed %d group %d" % (seed, g))
    assert np.all(np.isnan(y[live:]))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_mxfp8_wgrad(seed):
    rng = np.random.default_rng(2000 + seed)
    sizes = _sizes(rng, 8, 400)
    G, M = len(sizes), int(sizes.sum())
    N, K = 32 * int(rng.integers(1, 13)), 32 * int(rng.integers(1, 13))
    out_f32 = bool(rng.integers(0, 2))
    dy = _bits(rng, (max(M, 1), N))
    x = _bits(rng, (max(M, 1), K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    cap = max(M, 1) + 128 * G
    qd = bsg.grouped_quantize_mxfp8(bf16_dev(dy), to_dev(off), rowwise=False,
                                    padded_offsets=to_dev(poff), col_rows_cap=cap)
    qx = bsg.grouped_quantize_mxfp8(bf16_dev(x), to_dev(off), rowwise=False,
                                    padded_offsets=to_dev(poff), col_rows_cap=cap)
    dyc, dys = Q.mxfp8_colwise(dy, off, poff)
    xc, xs = Q.mxfp8_colwise(x, off, poff)
    n = int(poff[-1])
    assert np.array_equal(host_u8(qd["col_data"])[:n * N], dyc)
    assert np.array_equal(host_u8(qx["col_scales"])[:n * K // 32], xs)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((G, N, K), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_WGRAD_NT, qd["col_data"], qd["col_scales"], qx["col_data"],
                           qx["col_scales"], to_dev(poff), cap, N, K, out=out,
                           out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                           workspace=_workspace(rng))
    ref = GM.mxfp8_wgrad(dyc, dys, xc, xs, poff, N, K)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g] == 0:
            assert np.all(y[g] == 0.0) and not np.any(np.signbit(y[g]))
        else:
            gemm_tolerance_check(y[g], ref[g], out_f32, "seed %d group %d" % (seed, g))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_mxfp8_dgrad(seed):
    rng = np.random.default_rng(3000 + seed)
    sizes = _sizes(rng, 8, 400)
    G, M = len(sizes), int(sizes.sum())
    K, N = 32 * int(rng.integers(1, 25)), 32 * int(rng.integers(1, 13))  # K: contraction
    rows_cap = M + int(rng.integers(0, 20))
    dy = _bits(rng, (max(rows_cap, 1), K))
    w = _bits(rng, (G * K, N), std=0.05)
    _, off = O.group_offsets(sizes)
    # W's columnwise copy: each expert's K rows padded to a multiple of 128
    kpad = -(-K // 128) * 128
    woff = np.arange(G + 1, dtype=np.int64) * K
    wpoff = np.arange(G + 1, dtype=np.int64) * kpad
    dyd, dys = bsg.grouped_quantize_mxfp8_rowwise_e5m2(bf16_dev(dy), to_dev(off))
    wq = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(woff), rowwise=False,
                                    padded_offsets=to_dev(wpoff), col_rows_cap=G * kpad)
    rd, rs = Q.mxfp8_rowwise(dy, off, elem="e5m2")
    wtd, wts = Q.mxfp8_colwise(w, woff, wpoff)
    assert np.array_equal(host_u8(dyd)[:M], rd[:M])
    assert np.array_equal(host_u8(wq["col_data"]), wtd)
    dt = torch.float32
    out = torch.full((max(rows_cap, 1), N), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_DGRAD_NN, dyd, dys, wq["col_data"], wq["col_scales"],
                           to_dev(off), rows_cap, N, K, out=out, out_dtype=bsg.BSG_OUT_F32,
                           workspace=_workspace(rng))
    ref = GM.mxfp8_dgrad(rd, rs, wtd, wts, off, K, N)
    y = host(out).astype(np.float64)
    for g in range(G):
        if sizes[g]:
            gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], True,
                                 "seed %d group %d" % (seed, g))
    assert np.all(np.isnan(y[M:]))


def _npg(rng, G):
    return [32 * int(rng.integers(1, 9)) for _ in range(G)]


@pytest.mark.parametrize("seed", SEEDS)
def test_random_nvfp4_rowscaled(seed):
    rng = np.random.default_rng(4000 + seed)
    sizes = _sizes(rng, 8, 300)
    G, live = len(sizes), int(sizes.sum())
    npg = _npg(rng, G)
    K = 32 * int(rng.integers(1, 17))
    rows_cap = live + int(rng.integers(1, 40))
    ld = max(npg) + int(rng.integers(0, 9))
    out_f32 = bool(rng.integers(0, 2))
    fused = bool(rng.integers(0, 2))
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    a = bsg.grouped_quantize_nvfp4_rowscaled(bf16_dev(x), to_dev(off))
    b = bsg.grouped_quantize_nvfp4_rowscaled(bf16_dev(w), to_dev(boff))
    ap, asc, at = Q.nvfp4_rowscaled(x, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(w, boff)
    assert np.array_equal(host_u8(a[0])[:live], ap[:live])
    assert np.array_equal(host_u8(b[1]), bsc)
    assert np.array_equal(host(b[2]).view(np.uint32), bt.view(np.uint32))
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((rows_cap, ld), float("nan"), dtype=dt, device=device())
    scratch = None if fused else torch.empty((rows_cap, ld), dtype=torch.float32, device=device())
    bsg.grouped_gemm_nvfp4_rowscaled(a[0], a[1], a[2], to_dev(off), K, b[0], b[1], b[2], npg,
                                     out=out, ld_out=ld,
                                     out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                                     scratch=scratch,
                                     workspace=_workspace(rng) if fused else None)
    y = bf16_out_to_f64(out)
    for g, (rows, r) in enumerate(GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, out_f32, "seed %d group %d" % (seed, g))
            assert np.all(np.isnan(y[rows][:, npg[g]:]))
    assert np.all(np.isnan(y[live:]))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_nvfp4_pertensor(seed):
    rng = np.random.default_rng(5000 + seed)
    sizes = _sizes(rng, 8, 300)
    G, live = len(sizes), int(sizes.sum())
    npg = _npg(rng, G)
    K = 32 * int(rng.integers(1, 17))
    rows_cap = live + int(rng.integers(1, 40))
    ld = max(npg)
    out_f32 = bool(rng.integers(0, 2))
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    a = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(x), to_dev(off))
    b = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(w), to_dev(boff))
    ap, asc, aam = Q.nvfp4_pertensor(x, off)
    bp, bsc, bam = Q.nvfp4_pertensor(w, boff)
    assert np.array_equal(host_u8(a[0])[:live], ap[:live])
    assert np.array_equal(host(b[2]).view(np.uint32), bam.view(np.uint32))
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((rows_cap, ld), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_nvfp4_pertensor(a[0], a[1], a[2], to_dev(off), K, b[0], b[1], b[2], npg,
                                     out=out, ld_out=ld,
                                     out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                                     workspace=_workspace(rng))
    y = bf16_out_to_f64(out)
    for g, (rows, r) in enumerate(GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, out_f32, "seed %d group %d" % (seed, g))
    assert np.all(np.isnan(y[live:]))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_nvfp4_wgrad(seed):
    rng = np.random.default_rng(6000 + seed)
    sizes = _sizes(rng, 6, 300)
    G, M = len(sizes), int(sizes.sum())
    N, K = 32 * int(rng.integers(1, 9)), 32 * int(rng.integers(1, 9))
    out_f32 = bool(rng.integers(0, 2))
    dy = _bits(rng, (max(M, 1), N))
    x = _bits(rng, (max(M, 1), K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    cap = max(M, 1) + 128 * G
    dyc, dys, dyo = bsg.grouped_quantize_nvfp4_rowscaled_colwise(
        bf16_dev(dy), to_dev(off), to_dev(poff), col_rows_cap=cap)
    xc, xs, xo = bsg.grouped_quantize_nvfp4_rowscaled_colwise(
        bf16_dev(x), to_dev(off), to_dev(poff), col_rows_cap=cap)
    wdyc, wdys, wdyo = Q.nvfp4_rowscaled_colwise(dy, off, poff)
    wxc, wxs, wxo = Q.nvfp4_rowscaled_colwise(x, off, poff)
    n = int(poff[-1])
    assert np.array_equal(host_u8(dyc)[:n * N // 2], wdyc)
    assert np.array_equal(host(xo).view(np.uint32), wxo.view(np.uint32))
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((G, N, K), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_nvfp4_rowscaled_wgrad(dyc, dys, dyo, xc, xs, xo, to_dev(poff), N, K,
                                           col_rows_cap=cap, out=out,
                                           out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16)
    ref = GM.nvfp4_rowscaled_wgrad(wdyc, wdys, wdyo, wxc, wxs, wxo, poff, N, K)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g] == 0:
            assert np.all(y[g] == 0.0) and not np.any(np.signbit(y[g]))
        else:
            gemm_tolerance_check(y[g], ref[g], out_f32, "seed %d group %d" % (seed, g))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_mxfp8_fprop_epilogue_terms(seed):
    """grouped_gemm_mxfp8_ex: per-group alpha, beta (0 for some groups, whose
    previous output holds NaN and must not be read) and a bias, random shapes."""
    rng = np.random.default_rng(7000 + seed)
    sizes = _sizes(rng, 10, 300)
    G, live = len(sizes), int(sizes.sum())
    N, K = 32 * int(rng.integers(1, 17)), 32 * int(rng.integers(1, 17))
    rows_cap = live + int(rng.integers(1, 30))
    out_f32 = bool(rng.integers(0, 2))
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (G * N, K), 0.02)
    _, off = O.group_offsets(sizes)
    woff = np.array([0, G * N])
    qa = bsg.grouped_quantize_mxfp8(bf16_dev(x), to_dev(off))
    qb = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(woff))
    ad, asc = Q.mxfp8_rowwise(x, off)
    bd, bsc = Q.mxfp8_rowwise(w, woff)
    s_ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    grp = np.searchsorted(off, np.arange(live), side="right") - 1
    alpha = rng.uniform(-2, 2, G).astype(np.float32)
    beta = np.where(rng.random(G) < 0.5, rng.uniform(0.5, 1.5, G), 0.0).astype(np.float32)
    bias = rng.standard_normal((G, N)).astype(np.float32)
    dt = torch.float32 if out_f32 else torch.bfloat16
    c0 = torch.from_numpy(rng.standard_normal((rows_cap, N)).astype(np.float32)).to(dt)
    c0[:live][torch.from_numpy(beta[grp] == 0)] = float("nan")
    c0[live:] = float("nan")
    out = c0.to(device())
    c_prev = bf16_out_to_f64(out)
    bsg.grouped_gemm_mxfp8_ex(bsg.BSG_FPROP_TN, qa["row_data"], qa["row_scales"], qb["row_data"],
                              qb["row_scales"], to_dev(off), rows_cap, N, K, out,
                              out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                              alpha=to_dev(alpha), beta=to_dev(beta), bias=to_dev(bias))
    ref = GM.epilogue(s_ref[:live], grp, alpha, beta, c_prev[:live], bias)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g]:
            gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32,
                                 "seed %d group %d" % (seed, g))
    assert np.all(np.isnan(y[live:]))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_nvfp4_rowscaled_accumulate(seed):
    """Row-scaled NVFP4 with the accumulate flag (out = out_old + Y), fused or
    through the FP32 scratch, random shapes."""
    rng = np.random.default_rng(8000 + seed)
    sizes = _sizes(rng, 8, 300)
    G, live = len(sizes), int(sizes.sum())
    npg = _npg(rng, G)
    K = 32 * int(rng.integers(1, 17))
    rows_cap = live + int(rng.integers(1, 40))
    ld = max(npg) + int(rng.integers(0, 9))
    fused = bool(rng.integers(0, 2))
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    a = bsg.grouped_quantize_nvfp4_rowscaled(bf16_dev(x), to_dev(off))
    b = bsg.grouped_quantize_nvfp4_rowscaled(bf16_dev(w), to_dev(boff))
    ap, asc, at = Q.nvfp4_rowscaled(x, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(w, boff)
    c0 = rng.standard_normal((rows_cap, ld)).astype(np.float32)
    out = torch.from_numpy(c0).to(device())
    scratch = None if fused else torch.empty((rows_cap, ld), dtype=torch.float32, device=device())
    bsg.grouped_gemm_nvfp4_rowscaled(a[0], a[1], a[2], to_dev(off), K, b[0], b[1], b[2], npg,
                                     out=out, ld_out=ld, out_dtype=bsg.BSG_OUT_F32,
                                     scratch=scratch, accumulate=True,
                                     workspace=_workspace(rng) if fused else None)
    y = host(out).astype(np.float64)
    for g, (rows, r) in enumerate(GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r + c0[rows][:, :npg[g]], True,
                                 "seed %d group %d" % (seed, g))
            assert np.array_equal(y[rows][:, npg[g]:], c0[rows][:, npg[g]:])
    assert np.array_equal(y[live:], c0[live:])


@pytest.mark.parametrize("seed", SEEDS)
def test_random_nvfp4_rht_and_2d_gemm(seed):
    """Per-tensor NVFP4 with the Hadamard transform (a random sign mask) on both
    operands, or with 2-D block scales on the weights: quantized bytes and amax
    bit-exact, the GEMM within the tolerance of the oracle's."""
    rng = np.random.default_rng(9000 + seed)
    sizes = _sizes(rng, 8, 300)
    G, live = len(sizes), int(sizes.sum())
    npg = [16 * int(rng.integers(2, 17)) for _ in range(G)]
    K = 32 * int(rng.integers(1, 17))
    rows_cap = live + int(rng.integers(1, 40))
    out_f32 = bool(rng.integers(0, 2))
    rht = bool(rng.integers(0, 2))
    mask = int(rng.integers(0, 1 << 16))
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    if rht:
        a = bsg.grouped_quantize_nvfp4_pertensor_rht(bf16_dev(x), to_dev(off), mask)
        b = bsg.grouped_quantize_nvfp4_pertensor_rht(bf16_dev(w), to_dev(boff), mask)
        ap, asc, aam = Q.nvfp4_pertensor_rht(x, off, mask)
        bp, bsc, bam = Q.nvfp4_pertensor_rht(w, boff, mask)
    else:
        a = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(x), to_dev(off))
        b = bsg.grouped_quantize_nvfp4_pertensor_2d(bf16_dev(w), to_dev(boff))
        ap, asc, aam = Q.nvfp4_pertensor(x, off)
        bp, bsc, bam = Q.nvfp4_pertensor_2d(w, boff)
    assert np.array_equal(host_u8(a[0])[:live], ap[:live])
    assert np.array_equal(host_u8(a[1])[:live], asc[:live])
    assert np.array_equal(host(a[2]).view(np.uint32), aam.view(np.uint32))
    assert np.array_equal(host_u8(b[0]), bp)
    assert np.array_equal(host_u8(b[1]), bsc)
    assert np.array_equal(host(b[2]).view(np.uint32), bam.view(np.uint32))
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((rows_cap, max(npg)), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_nvfp4_pertensor(a[0], a[1], a[2], to_dev(off), K, b[0], b[1], b[2], npg,
                                     out=out,
                                     out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                                     workspace=_workspace(rng))
    y = bf16_out_to_f64(out)
    for g, (rows, r) in enumerate(GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, out_f32, "seed %d group %d" % (seed, g))
    assert np.all(np.isnan(y[live:]))
