"""GPU parity at the edges of the C-ABI contract and under stress.

* contraction lengths that are any multiple of 32 (not only of the kernels'
  64- or 128-element steps) for the MXFP8 fprop and dgrad and both NVFP4 GEMMs
  ("gemm.py", assert_cublas_requirements: the contracting dim needs only the
  block-size multiple), with the bytes past k made hostile (NaN codes in rows
  no group owns, nonzero padding scale bytes) so that a kernel that reads past
  k fails;
* operands whose 32-element blocks are scaled by 2^U(-20, 20), so that
  neighbouring E8M0 bytes differ and every scale-selection path of the scaled
  MFMA is exercised;
* offsets whose first entry is past row 0 (rows that no group owns stay
  untouched);
* HIP-graph replays with new device sizes for the wgrad, dgrad, row-scaled
  NVFP4 fprop and NVFP4 columnwise + wgrad paths;
* the binding's argument checks (no launch).
"""

import numpy as np
import pytest
import torch

import block_scaled_grouped_amd as bsg
from oracle import formats as F
from oracle import gemm as GM
from oracle import layout as L
from oracle import offsets as O
from oracle import quantize as Q
from gpu_util import (SENTINEL, bf16_dev, bf16_out_to_f64, device, filled_u8,
                      gemm_tolerance_check, host, host_u8, to_dev)

pytestmark = pytest.mark.gpu


def _bits(rng, shape, std=1.0, spread=0, axis=1):
    """bf16 bits of N(0, std^2) values; with spread > 0 every 32-element block
    along `axis` is multiplied by 2^e, e uniform in [-spread, spread]."""
    v = rng.standard_normal(shape) * std
    if spread:
        if axis == 1:
            e = rng.integers(-spread, spread + 1, (shape[0], -(-shape[1] // 32)))
            v = v * np.exp2(np.repeat(e, 32, axis=1)[:, :shape[1]])
        else:
            e = rng.integers(-spread, spread + 1, (-(-shape[0] // 32), shape[1]))
            v = v * np.exp2(np.repeat(e, 32, axis=0)[:shape[0]])
    return F.f32_to_bf16_bits_rne(v.astype(np.float32))


def _stress_scale_padding(stored, n_blk):
    """Sets the E8M0 bytes past the last block of every row (the padding of the
    last 128-element word) to 127: a kernel that masks the data past k still
    multiplies zeros there; one that reads the next row's bytes does not."""
    stored = np.array(stored, copy=True)
    nq = stored.shape[0]
    for pos in range(4):
        if 4 * (nq - 1) + L.MX_PERM[pos] >= n_blk:
            stored[nq - 1, :, pos] = 127
    return stored


def _rows_dev(data, scales, rows_cap, fill=0x7F):
    """Live rows' data [live, K] and scale words [NQ, live, 4] -> device buffers
    of rows_cap rows; rows no group owns hold the E4M3 NaN code."""
    d = np.full((rows_cap, data.shape[1]), fill, np.uint8)
    s = np.full((scales.shape[0], rows_cap, 4), 127, np.uint8)
    d[:data.shape[0]] = data
    s[:, :scales.shape[1]] = scales
    return to_dev(d), to_dev(s)


OUT = {True: bsg.BSG_OUT_F32, False: bsg.BSG_OUT_BF16}


def _out(shape, out_f32):
    return torch.full(shape, float("nan"), dtype=torch.float32 if out_f32 else torch.bfloat16,
                      device=device())


# ---------------------------------------------------------------- MXFP8 fprop, k % 128 != 0

@pytest.mark.parametrize("K", [32, 96, 160, 4128])
@pytest.mark.parametrize("out_f32", [True, False])
def test_fprop_any_k_multiple_of_32(K, out_f32):
    rng = np.random.default_rng(K)
    sizes = np.array([70, 0, 300, 5], np.int32)
    G, N, live = len(sizes), 288, int(sizes.sum())
    rows_cap = live + 40
    x = _bits(rng, (live, K), spread=6)
    w = _bits(rng, (G * N, K), 0.02, spread=6)
    _, off = O.group_offsets(sizes)
    ad, asc = Q.mxfp8_rowwise(x, off)
    bd, bsc = Q.mxfp8_rowwise(w, np.array([0, G * N]))
    ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    nblk = K // 32
    a, a_s = _rows_dev(ad, _stress_scale_padding(asc, nblk), rows_cap)
    b, b_s = to_dev(bd), to_dev(_stress_scale_padding(bsc, nblk))
    out = _out((rows_cap, N), out_f32)
    bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, a_s, b, b_s, to_dev(off), rows_cap, N, K, out=out,
                           out_dtype=OUT[out_f32])
    y = bf16_out_to_f64(out)
    for g in range(G):
        gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32, "group %d" % g)
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


@pytest.mark.parametrize("K", [32, 96, 160])
def test_fprop_any_k_end_to_end(K):
    """GPU quantize (whose scale words past k/32 are 0x00) -> GPU GEMM."""
    rng = np.random.default_rng(5 * K)
    sizes = np.array([33, 200, 0, 64], np.int32)
    G, N, live = len(sizes), 160, int(sizes.sum())
    x = _bits(rng, (live, K))
    w = _bits(rng, (G * N, K), 0.02)
    _, off = O.group_offsets(sizes)
    qa = bsg.grouped_quantize_mxfp8(bf16_dev(x), to_dev(off))
    qb = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(np.array([0, G * N])))
    ad, asc = Q.mxfp8_rowwise(x, off)
    bd, bsc = Q.mxfp8_rowwise(w, np.array([0, G * N]))
    assert np.array_equal(host_u8(qa["row_scales"]), asc)
    assert np.array_equal(host_u8(qb["row_scales"]), bsc)
    out = _out((live, N), True)
    bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, qa["row_data"], qa["row_scales"], qb["row_data"],
                           qb["row_scales"], to_dev(off), live, N, K, out=out,
                           out_dtype=bsg.BSG_OUT_F32)
    ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    y = host(out).astype(np.float64)
    for g in range(G):
        gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], True, "group %d" % g)


# ---------------------------------------------------------------- MXFP8 dgrad, contraction % 128 != 0

@pytest.mark.parametrize("K", [32, 96, 160])
@pytest.mark.parametrize("out_f32", [True, False])
def test_dgrad_any_contraction_multiple_of_32(K, out_f32):
    """dX = dY (E5M2, rowwise along K) x W_g, W from its columnwise copy whose
    experts are padded to roundup(K, 128) tokens."""
    rng = np.random.default_rng(K * 13)
    sizes = np.array([37, 0, 130, 5], np.int32)
    G, M, N = len(sizes), int(sizes.sum()), 288
    rows_cap = M + 17
    kpad = -(-K // 128) * 128
    dy = _bits(rng, (rows_cap, K), spread=6)
    w = _bits(rng, (G * K, N), std=0.05, spread=6, axis=0)
    _, off = O.group_offsets(sizes)
    woff = np.arange(G + 1, dtype=np.int64) * K
    wpoff = np.arange(G + 1, dtype=np.int64) * kpad
    dyd = filled_u8((rows_cap, K), 0x7F)    # rows no group owns: NaN codes
    dys = filled_u8(bsg.mx_scale_shape(rows_cap, K), 127)
    bsg.grouped_quantize_mxfp8_rowwise_e5m2(bf16_dev(dy), to_dev(off), row_data=dyd,
                                            row_scales=dys)
    wq = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(woff), rowwise=False,
                                    padded_offsets=to_dev(wpoff), col_rows_cap=G * kpad)
    rd, rs = Q.mxfp8_rowwise(dy, off, elem="e5m2")
    wtd, wts = Q.mxfp8_colwise(w, woff, wpoff)
    assert np.array_equal(host_u8(dyd)[:M], rd)
    assert np.array_equal(host_u8(wq["col_data"]), wtd)
    assert np.array_equal(host_u8(wq["col_scales"]), wts)
    ref = GM.mxfp8_dgrad(rd, rs, wtd, wts, off, K, N)
    out = _out((rows_cap, N), out_f32)
    bsg.grouped_gemm_mxfp8(bsg.BSG_DGRAD_NN, dyd, dys, wq["col_data"], wq["col_scales"],
                           to_dev(off), rows_cap, N, K, out=out, out_dtype=OUT[out_f32])
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g]:
            gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32,
                                 "group %d" % g)
    assert np.all(np.isnan(y[M:])), "capacity rows untouched"


# ---------------------------------------------------------------- NVFP4, k % 64 != 0

def _nv_rows_dev(a, rows_cap, fill):
    o = np.full((rows_cap,) + a.shape[1:], fill, a.dtype)
    o[:a.shape[0]] = a
    return to_dev(o)


@pytest.mark.parametrize("K", [32, 96, 160, 4128])
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("out_f32", [True, False])
def test_nvfp4_rowscaled_any_k_multiple_of_32(K, fused, out_f32):
    rng = np.random.default_rng(K + 7)
    sizes = np.array([100, 0, 257, 31], np.int32)
    npg = [64, 128, 96, 256]
    live = int(sizes.sum())
    rows_cap = live + 20
    _, off = O.group_offsets(sizes)
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    ap, asc, at = Q.nvfp4_rowscaled(x, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(w, np.array([0, sum(npg)]))
    ld = max(npg) + 8
    out = _out((rows_cap, ld), out_f32)
    scratch = None if fused else torch.empty((rows_cap, ld), dtype=torch.float32, device=device())
    # rows no group owns: E4M3 NaN scales and nonzero codes
    bsg.grouped_gemm_nvfp4_rowscaled(_nv_rows_dev(ap, rows_cap, 0x77),
                                     _nv_rows_dev(asc, rows_cap, 0x7F),
                                     _nv_rows_dev(at, rows_cap, np.float32(1.0)), to_dev(off), K,
                                     to_dev(bp), to_dev(bsc), to_dev(bt), npg, out=out, ld_out=ld,
                                     out_dtype=OUT[out_f32], scratch=scratch)
    y = bf16_out_to_f64(out)
    for g, (rows, r) in enumerate(GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, out_f32, "group %d" % g)
            assert np.all(np.isnan(y[rows][:, npg[g]:]))
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


@pytest.mark.parametrize("K", [32, 96, 4128])
def test_nvfp4_pertensor_any_k_end_to_end(K):
    rng = np.random.default_rng(3 * K + 1)
    sizes = np.array([150, 0, 106], np.int32)
    npg = [128, 256, 96]
    live = int(sizes.sum())
    rows_cap = live + 9
    xb = _bits(rng, (rows_cap, K))
    wb = _bits(rng, (sum(npg), K), 0.02)
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    doff = to_dev(off)
    a = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(xb), doff)
    b = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(wb), to_dev(boff))
    ap, asc, aam = Q.nvfp4_pertensor(xb, off)
    bp, bsc, bam = Q.nvfp4_pertensor(wb, boff)
    assert np.array_equal(host_u8(a[0])[:live], ap) and np.array_equal(host_u8(a[1])[:live], asc)
    out = _out((rows_cap, max(npg)), True)
    bsg.grouped_gemm_nvfp4_pertensor(a[0], a[1], a[2], doff, K, b[0], b[1], b[2], npg, out=out,
                                     out_dtype=bsg.BSG_OUT_F32)
    y = host(out).astype(np.float64)
    for g, (rows, r) in enumerate(GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, True, "group %d" % g)
    assert np.all(np.isnan(y[live:]))


# ---------------------------------------------------------------- scale spread (every E8M0 path)

@pytest.mark.parametrize("out_f32", [True, False])
def test_fprop_scale_spread(out_f32):
    rng = np.random.default_rng(91)
    sizes = np.array([300, 0, 17, 513, 130], np.int32)
    G, K, N, live = len(sizes), 512, 640, int(sizes.sum())
    x = _bits(rng, (live, K), spread=20)
    w = _bits(rng, (G * N, K), 0.02, spread=20)
    _, off = O.group_offsets(sizes)
    ad, asc = Q.mxfp8_rowwise(x, off)
    bd, bsc = Q.mxfp8_rowwise(w, np.array([0, G * N]))
    # the spread reaches the GEMM: neighbouring blocks of a row rarely share a scale
    lg = L.mx_scales_from_gemm_order(asc, K // 32)
    assert np.mean(lg[:, 1:] != lg[:, :-1]) > 0.8
    ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    out = _out((live, N), out_f32)
    bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, to_dev(ad), to_dev(asc), to_dev(bd), to_dev(bsc),
                           to_dev(off), live, N, K, out=out, out_dtype=OUT[out_f32])
    y = bf16_out_to_f64(out)
    for g in range(G):
        gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32, "group %d" % g)


@pytest.mark.parametrize("out_f32", [True, False])
def test_wgrad_scale_spread(out_f32):
    rng = np.random.default_rng(92)
    sizes = np.array([37, 0, 290, 130, 5], np.int32)
    G, M, N, K = len(sizes), int(sizes.sum()), 288, 320
    dy = _bits(rng, (M, N), spread=20, axis=0)
    x = _bits(rng, (M, K), spread=20, axis=0)
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    cap = int(poff[-1])
    q1 = bsg.grouped_quantize_mxfp8(bf16_dev(dy), to_dev(off), rowwise=False,
                                    padded_offsets=to_dev(poff), col_rows_cap=cap)
    q2 = bsg.grouped_quantize_mxfp8(bf16_dev(x), to_dev(off), rowwise=False,
                                    padded_offsets=to_dev(poff), col_rows_cap=cap)
    dyc, dys = Q.mxfp8_colwise(dy, off, poff)
    xc, xs = Q.mxfp8_colwise(x, off, poff)
    assert np.array_equal(host_u8(q1["col_data"]), dyc) and np.array_equal(host_u8(q2["col_scales"]), xs)
    ref = GM.mxfp8_wgrad(dyc, dys, xc, xs, poff, N, K)
    out = _out((G, N, K), out_f32)
    bsg.grouped_gemm_mxfp8(bsg.BSG_WGRAD_NT, q1["col_data"], q1["col_scales"], q2["col_data"],
                           q2["col_scales"], to_dev(poff), cap, N, K, out=out,
                           out_dtype=OUT[out_f32])
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g] == 0:
            assert np.all(y[g] == 0.0) and not np.any(np.signbit(y[g]))
        else:
            gemm_tolerance_check(y[g], ref[g], out_f32, "group %d" % g)


def test_dgrad_scale_spread():
    rng = np.random.default_rng(93)
    sizes = np.array([300, 1, 0, 700], np.int32)
    G, M, K, N = len(sizes), int(sizes.sum()), 384, 256
    dy = _bits(rng, (M, K), spread=20)
    w = _bits(rng, (G * K, N), std=0.05, spread=20, axis=0)
    _, off = O.group_offsets(sizes)
    woff = np.arange(G + 1, dtype=np.int64) * K
    dyd, dys = bsg.grouped_quantize_mxfp8_rowwise_e5m2(bf16_dev(dy), to_dev(off))
    wq = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(woff), rowwise=False,
                                    padded_offsets=to_dev(woff), col_rows_cap=G * K)
    rd, rs = Q.mxfp8_rowwise(dy, off, elem="e5m2")
    wtd, wts = Q.mxfp8_colwise(w, woff, woff)
    assert np.array_equal(host_u8(dys), rs) and np.array_equal(host_u8(wq["col_scales"]), wts)
    ref = GM.mxfp8_dgrad(rd, rs, wtd, wts, off, K, N)
    out = _out((M, N), True)
    bsg.grouped_gemm_mxfp8(bsg.BSG_DGRAD_NN, dyd, dys, wq["col_data"], wq["col_scales"],
                           to_dev(off), M, N, K, out=out, out_dtype=bsg.BSG_OUT_F32)
    y = host(out).astype(np.float64)
    for g in range(G):
        if sizes[g]:
            gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], True, "group %d" % g)


# ---------------------------------------------------------------- offsets[0] > 0

@pytest.mark.parametrize("fused", [True, False])
def test_nvfp4_rowscaled_rows_before_first_offset_untouched(fused):
    rng = np.random.default_rng(61)
    off = np.array([5, 105, 105, 362], np.int64)     # rows 0..4 belong to no group
    npg = [64, 128, 96]
    K, rows_cap = 128, 380
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    ap, asc, at = Q.nvfp4_rowscaled(x, off)          # quantizes rows < offsets[G]
    bp, bsc, bt = Q.nvfp4_rowscaled(w, np.array([0, sum(npg)]))
    ld = max(npg)
    out = _out((rows_cap, ld), True)
    scratch = None if fused else torch.full((rows_cap, ld), 3.0, dtype=torch.float32,
                                            device=device())
    bsg.grouped_gemm_nvfp4_rowscaled(_nv_rows_dev(ap, rows_cap, 0), _nv_rows_dev(asc, rows_cap, 0),
                                     _nv_rows_dev(at, rows_cap, np.float32(0)), to_dev(off), K,
                                     to_dev(bp), to_dev(bsc), to_dev(bt), npg, out=out,
                                     out_dtype=bsg.BSG_OUT_F32, scratch=scratch)
    y = host(out).astype(np.float64)
    for g, (rows, r) in enumerate(GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, True, "group %d" % g)
    assert np.all(np.isnan(y[:5])), "rows before offsets[0] belong to no group"
    assert np.all(np.isnan(y[362:]))


def test_nvfp4_pertensor_rows_before_first_offset():
    """Rows before offsets[0] belong to no group: they do not enter any group's
    amax and the cast leaves them untouched."""
    rng = np.random.default_rng(62)
    off = np.array([7, 100, 100, 300], np.int64)
    K, rows_cap = 96, 320
    x = _bits(rng, (rows_cap, K))
    x[:7] = F.f32_to_bf16_bits_rne(np.full((7, K), 1e4, np.float32))   # would dominate group 0
    rp, rs, ra = Q.nvfp4_pertensor(x[7:], off - 7)
    d = filled_u8((rows_cap, K // 2))
    s = filled_u8((rows_cap, K // 16))
    a = torch.full((3,), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(x), to_dev(off), data=d, block_scales=s, amax=a)
    d, s = host_u8(d), host_u8(s)
    assert np.array_equal(host(a).view(np.uint32), ra.view(np.uint32))
    assert np.array_equal(d[7:300], rp) and np.array_equal(s[7:300], rs)
    assert np.all(d[:7] == SENTINEL) and np.all(s[:7] == SENTINEL)
    assert np.all(d[300:] == SENTINEL) and np.all(s[300:] == SENTINEL)


# ---------------------------------------------------------------- HIP-graph replays with new sizes

def _capture(step):
    step()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    return g


def test_wgrad_hip_graph_replay_with_new_sizes():
    dev = device()
    rng = np.random.default_rng(71)
    G, N, K, rows_cap = 3, 160, 288, 600
    cap = rows_cap + 128 * G
    dyb, xb = _bits(rng, (rows_cap, N)), _bits(rng, (rows_cap, K))
    dy, x = bf16_dev(dyb), bf16_dev(xb)
    sizes = torch.tensor([100, 0, 200], dtype=torch.int32, device=dev)
    off = torch.empty(G + 1, dtype=torch.int64, device=dev)
    poff = torch.empty(G + 1, dtype=torch.int64, device=dev)
    bufs = [filled_u8((cap * c,), 0) for c in (N, K)]
    sbufs = [filled_u8((cap * c // 32,), 0) for c in (N, K)]
    out = torch.empty((G, N, K), dtype=torch.float32, device=dev)

    def step():
        bsg.group_offsets_i32_to_i64(sizes, offsets=off)
        bsg.group_offsets_i32_to_i64(sizes, pad_to=128, offsets=poff)
        for src, d, s in ((dy, bufs[0], sbufs[0]), (x, bufs[1], sbufs[1])):
            bsg.grouped_quantize_mxfp8(src, off, rowwise=False, padded_offsets=poff,
                                       col_rows_cap=cap, col_data=d, col_scales=s)
        bsg.grouped_gemm_mxfp8(bsg.BSG_WGRAD_NT, bufs[0], sbufs[0], bufs[1], sbufs[1], poff, cap,
                               N, K, out=out, out_dtype=bsg.BSG_OUT_F32)

    g = _capture(step)
    for new in ([100, 0, 200], [50, 250, 300], [0, 0, 600], [1, 0, 0], [0, 0, 0]):
        sizes.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _, o = O.group_offsets(np.array(new))
        _, po = O.group_offsets(np.array(new), pad_to=128)
        dyc, dys = Q.mxfp8_colwise(dyb, o, po)
        xc, xs = Q.mxfp8_colwise(xb, o, po)
        ref = GM.mxfp8_wgrad(dyc, dys, xc, xs, po, N, K)
        y = host(out).astype(np.float64)
        for gi in range(G):
            if new[gi] == 0:
                assert np.all(y[gi] == 0.0), new
            else:
                gemm_tolerance_check(y[gi], ref[gi], True, str(new))
        eager = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(eager, out)


def test_dgrad_hip_graph_replay_with_new_sizes():
    dev = device()
    rng = np.random.default_rng(72)
    G, K, N, rows_cap = 3, 256, 160, 500
    dyb = _bits(rng, (rows_cap, K))
    wb = _bits(rng, (G * K, N), std=0.05)
    dy = bf16_dev(dyb)
    woff = np.arange(G + 1, dtype=np.int64) * K
    wq = bsg.grouped_quantize_mxfp8(bf16_dev(wb), to_dev(woff), rowwise=False,
                                    padded_offsets=to_dev(woff), col_rows_cap=G * K)
    wtd, wts = Q.mxfp8_colwise(wb, woff, woff)
    sizes = torch.tensor([100, 0, 200], dtype=torch.int32, device=dev)
    off = torch.empty(G + 1, dtype=torch.int64, device=dev)
    dyd = filled_u8((rows_cap, K), 0)
    dys = filled_u8(bsg.mx_scale_shape(rows_cap, K), 0)
    out = torch.empty((rows_cap, N), dtype=torch.float32, device=dev)

    def step():
        bsg.group_offsets_i32_to_i64(sizes, offsets=off)
        bsg.grouped_quantize_mxfp8_rowwise_e5m2(dy, off, row_data=dyd, row_scales=dys)
        bsg.grouped_gemm_mxfp8(bsg.BSG_DGRAD_NN, dyd, dys, wq["col_data"], wq["col_scales"], off,
                               rows_cap, N, K, out=out, out_dtype=bsg.BSG_OUT_F32)

    g = _capture(step)
    for new in ([100, 0, 200], [50, 250, 200], [0, 0, 500], [500, 0, 0]):
        sizes.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _, o = O.group_offsets(np.array(new))
        rd, rs = Q.mxfp8_rowwise(dyb, o, elem="e5m2")
        ref = GM.mxfp8_dgrad(rd, rs, wtd, wts, o, K, N)
        y = host(out).astype(np.float64)
        live = int(o[-1])
        for gi in range(G):
            if new[gi]:
                gemm_tolerance_check(y[o[gi]:o[gi + 1]], ref[o[gi]:o[gi + 1]], True, str(new))
        assert np.all(np.isnan(y[live:]))
        eager = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(eager[:live], out[:live])


@pytest.mark.parametrize("fused", [True, False])
def test_nvfp4_rowscaled_hip_graph_replay_with_new_sizes(fused):
    dev = device()
    rng = np.random.default_rng(73)
    G, K, rows_cap = 3, 256, 600
    npg = [128, 256, 64]
    xb = _bits(rng, (rows_cap, K))
    wb = _bits(rng, (sum(npg), K), 0.02)
    x = bf16_dev(xb)
    qb = bsg.grouped_quantize_nvfp4_rowscaled(bf16_dev(wb), to_dev(np.array([0, sum(npg)])))
    bp, bsc, bt = Q.nvfp4_rowscaled(wb, np.array([0, sum(npg)]))
    sizes = torch.tensor([100, 0, 200], dtype=torch.int32, device=dev)
    off = torch.empty(G + 1, dtype=torch.int64, device=dev)
    ad = filled_u8((rows_cap, K // 2), 0)
    asc = filled_u8((rows_cap, K // 16), 0)
    ao = torch.zeros(rows_cap, dtype=torch.float32, device=dev)
    ld = max(npg)
    out = torch.empty((rows_cap, ld), dtype=torch.float32, device=dev)
    scratch = None if fused else torch.zeros((rows_cap, ld), dtype=torch.float32, device=dev)

    def step():
        bsg.group_offsets_i32_to_i64(sizes, offsets=off)
        bsg.grouped_quantize_nvfp4_rowscaled(x, off, data=ad, block_scales=asc, outer=ao)
        bsg.grouped_gemm_nvfp4_rowscaled(ad, asc, ao, off, K, qb[0], qb[1], qb[2], npg, out=out,
                                         ld_out=ld, out_dtype=bsg.BSG_OUT_F32, scratch=scratch)

    g = _capture(step)
    for new in ([100, 0, 200], [50, 250, 300], [0, 0, 600], [600, 0, 0], [10, 20, 30]):
        sizes.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _, o = O.group_offsets(np.array(new))
        ap, asn, at = Q.nvfp4_rowscaled(xb, o)
        y = host(out).astype(np.float64)
        for gi, (rows, r) in enumerate(GM.nvfp4_rowscaled_fprop(ap, asn, at, o, bp, bsc, bt, npg, K)):
            if len(rows):
                gemm_tolerance_check(y[rows][:, :npg[gi]], r, True, str(new))
                assert np.all(np.isnan(y[rows][:, npg[gi]:]))
        live = int(o[-1])
        assert np.all(np.isnan(y[live:]))
        eager = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(eager[:live].nan_to_num(7.0), out[:live].nan_to_num(7.0))


def test_nvfp4_colwise_wgrad_hip_graph_replay_with_new_sizes():
    dev = device()
    rng = np.random.default_rng(74)
    G, N, K, rows_cap = 3, 96, 160, 500
    cap = rows_cap + 128 * G
    dyb, xb = _bits(rng, (rows_cap, N)), _bits(rng, (rows_cap, K))
    dy, x = bf16_dev(dyb), bf16_dev(xb)
    sizes = torch.tensor([100, 0, 200], dtype=torch.int32, device=dev)
    off = torch.empty(G + 1, dtype=torch.int64, device=dev)
    poff = torch.empty(G + 1, dtype=torch.int64, device=dev)
    q = [(filled_u8((cap * c // 2,), 0), filled_u8((cap * c // 16,), 0),
          torch.zeros((G, c), dtype=torch.float32, device=dev)) for c in (N, K)]
    out = torch.empty((G, N, K), dtype=torch.float32, device=dev)

    def step():
        bsg.group_offsets_i32_to_i64(sizes, offsets=off)
        bsg.group_offsets_i32_to_i64(sizes, pad_to=128, offsets=poff)
        for src, (d, s, o) in zip((dy, x), q):
            bsg.grouped_quantize_nvfp4_rowscaled_colwise(src, off, poff, col_rows_cap=cap, data=d,
                                                         block_scales=s, outer=o)
        bsg.grouped_gemm_nvfp4_rowscaled_wgrad(q[0][0], q[0][1], q[0][2], q[1][0], q[1][1],
                                               q[1][2], poff, N, K, col_rows_cap=cap, out=out,
                                               out_dtype=bsg.BSG_OUT_F32)

    g = _capture(step)
    for new in ([100, 0, 200], [50, 250, 200], [0, 0, 500], [1, 0, 0]):
        sizes.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _, o = O.group_offsets(np.array(new))
        _, po = O.group_offsets(np.array(new), pad_to=128)
        a = Q.nvfp4_rowscaled_colwise(dyb, o, po)
        b = Q.nvfp4_rowscaled_colwise(xb, o, po)
        n = int(po[-1])
        assert np.array_equal(host_u8(q[0][0])[:n * N // 2], a[0]), new
        assert np.array_equal(host(q[1][2]).view(np.uint32), b[2].view(np.uint32)), new
        ref = GM.nvfp4_rowscaled_wgrad(*a, *b, po, N, K)
        y = host(out).astype(np.float64)
        for gi in range(G):
            if new[gi] == 0:
                assert np.all(y[gi] == 0.0), new
            else:
                gemm_tolerance_check(y[gi], ref[gi], True, str(new))
        eager = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(eager, out)


# ---------------------------------------------------------------- binding checks (nothing launched)

def test_binding_rejects_bad_buffers_before_launch():
    dev = device()
    x = torch.zeros((64, 128), dtype=torch.bfloat16, device=dev)
    off = torch.tensor([0, 64], dtype=torch.int64, device=dev)
    with pytest.raises(ValueError, match="bfloat16"):
        bsg.grouped_quantize_mxfp8(x.float(), off)
    with pytest.raises(ValueError, match="contiguous"):
        bsg.grouped_quantize_mxfp8(torch.zeros((128, 64), dtype=torch.bfloat16, device=dev).t(), off)
    with pytest.raises(ValueError, match="row_data"):
        bsg.grouped_quantize_mxfp8(x, off, row_data=filled_u8((63, 128)))
    with pytest.raises(ValueError, match="offsets"):
        bsg.grouped_quantize_mxfp8(x, off.int(), G=1)
    a = filled_u8((64, 128), 0)
    s = filled_u8(bsg.mx_scale_shape(64, 128), 0)
    b = filled_u8((2, 256, 128), 0)
    bs = filled_u8(bsg.mx_scale_shape(512, 128), 0)
    off2 = torch.tensor([0, 32, 64], dtype=torch.int64, device=dev)
    with pytest.raises(ValueError, match="out"):
        bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, s, b, bs, off2, 64, 256, 128,
                               out=torch.empty((64, 255), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError, match="out"):
        bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, s, b, bs, off2, 64, 256, 128,
                               out=torch.empty((64, 256), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError, match="b holds"):
        bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, s, b[:1].contiguous(), bs, off2, 64, 256, 128)
    with pytest.raises(ValueError, match="a_scales"):
        bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, s[:, :32].contiguous(), b, bs, off2, 64, 256,
                               128)
    nv = filled_u8((64, 64), 0)
    nvs = filled_u8((64, 8), 0)
    nvo = torch.ones(64, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="scratch"):
        bsg.grouped_gemm_nvfp4_rowscaled(nv, nvs, nvo, off2, 128, nv, nvs, nvo, [32, 32],
                                         scratch=torch.empty((64, 31), dtype=torch.float32,
                                                             device=dev))
    with pytest.raises(ValueError, match="b_outer"):
        bsg.grouped_gemm_nvfp4_rowscaled(nv, nvs, nvo, off2, 128, nv, nvs, nvo[:10].contiguous(),
                                         [32, 32])
