"""GPU parity of the grouped GEMMs against the fp64 oracle.

The operands the GPU multiplies are the oracle's own quantized bytes (uploaded),
so the GEMM is checked in isolation; the end-to-end tests chain the GPU
quantize and GPU GEMM and compare with the oracle's quantize + GEMM.  Shapes
span several 256-wide tiles with ragged tails, empty groups and capacity rows.
"""

import numpy as np
import pytest
import torch

import block_scaled_grouped_amd as bsg
from oracle import formats as F
from oracle import gemm as GM
from oracle import offsets as O
from oracle import quantize as Q
import workloads
from gpu_util import (bf16_dev, bf16_out_to_f64, device, gemm_tolerance_check, host, host_u8,
                      to_dev)

pytestmark = pytest.mark.gpu


def _bits(rng, shape, std=1.0):
    return F.f32_to_bf16_bits_rne((rng.standard_normal(shape) * std).astype(np.float32))


def _fprop_operands(rng, sizes, K, N, rows_cap=None):
    sizes = np.array(sizes, np.int32)
    G, live = len(sizes), int(sizes.sum())
    rows_cap = live if rows_cap is None else rows_cap
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (G * N, K), 0.02)
    _, off = O.group_offsets(sizes)
    ad, asc = Q.mxfp8_rowwise(x, off)
    bd, bsc = Q.mxfp8_rowwise(w, np.array([0, G * N]))
    return sizes, off, x, w, ad, asc, bd.reshape(G, N, K), bsc, rows_cap


def _upload_rows(data, scales, rows_cap):
    """Live rows' data [live, K] and scales [NQ, live, 4] -> device buffers of
    rows_cap rows (zero capacity rows)."""
    d = np.zeros((rows_cap, data.shape[1]), np.uint8)
    s = np.zeros((scales.shape[0], rows_cap, 4), np.uint8)
    d[:data.shape[0]] = data
    s[:, :scales.shape[1]] = scales
    return to_dev(d), to_dev(s)


FPROP_CASES = [
    ([300, 0, 17, 513, 130], 512, 640, 1000),
    ([32, 0, 64, 32], 128, 128, 128),
    ([0, 0, 700], 256, 300, 700),
    ([1], 128, 1, 1),
    ([5, 300, 0, 40], 128, 258, 400),   # row stride not a multiple of 4: per-element stores
    ([260, 3], 256, 260, 263),          # a 4-column last tile
    ([(7 * i) % 41 if i % 5 else 0 for i in range(256)], 128, 64, 5200),   # 256 groups (maximum)
]


@pytest.mark.parametrize("sizes,K,N,rows_cap", FPROP_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_fprop_parity(sizes, K, N, rows_cap, out_f32):
    rng = np.random.default_rng(K + N + len(sizes))
    sizes, off, x, w, ad, asc, bd, bsc, rows_cap = _fprop_operands(rng, sizes, K, N, rows_cap)
    ref = GM.mxfp8_fprop(ad, asc, bd, bsc, off, K)
    a, a_s = _upload_rows(ad, asc, rows_cap)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((rows_cap, N), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, a_s, to_dev(bd), to_dev(bsc), to_dev(off), rows_cap,
                           N, K, out=out, out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16)
    y = bf16_out_to_f64(out)
    live = int(off[-1])
    for g in range(len(sizes)):
        gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32, "group %d" % g)
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


WGRAD_CASES = [
    ([37, 0, 130, 5, 300], 160, 96),
    ([2049, 0, 3001, 0], 256, 288),
    ([0, 0], 64, 64),
]


@pytest.mark.parametrize("sizes,N,K", WGRAD_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_wgrad_parity(sizes, N, K, out_f32):
    rng = np.random.default_rng(N * 3 + K)
    sizes = np.array(sizes, np.int32)
    G, M = len(sizes), int(sizes.sum())
    dy = _bits(rng, (max(M, 1), N))
    x = _bits(rng, (max(M, 1), K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    dyc, dys = Q.mxfp8_colwise(dy, off, poff)
    xc, xs = Q.mxfp8_colwise(x, off, poff)
    ref = GM.mxfp8_wgrad(dyc, dys, xc, xs, poff, N, K)
    cap = max(int(poff[-1]), 128)

    def pad(a, n):
        o = np.zeros(n, np.uint8)
        o[:len(a)] = a
        return to_dev(o)

    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((G, N, K), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_WGRAD_NT, pad(dyc, cap * N), pad(dys, cap * N // 32),
                           pad(xc, cap * K), pad(xs, cap * K // 32), to_dev(poff), cap, N, K,
                           out=out, out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g] == 0:
            assert np.all(y[g] == 0.0) and not np.any(np.signbit(y[g])), "empty expert must be +0"
        else:
            gemm_tolerance_check(y[g], ref[g], out_f32, "group %d" % g)


@pytest.mark.parametrize("sizes,N,K", WGRAD_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_wgrad_e5m2_parity(sizes, N, K, out_f32):
    """dW = dY^T X with dY's columnwise copy in E5M2 (GPU quantize, checked
    bit-exact) times X's E4M3 copy."""
    rng = np.random.default_rng(N * 5 + K)
    sizes = np.array(sizes, np.int32)
    G, M = len(sizes), int(sizes.sum())
    dy = _bits(rng, (max(M, 1), N))
    x = _bits(rng, (max(M, 1), K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    cap = max(int(poff[-1]), 128)
    dyc, dys = bsg.grouped_quantize_mxfp8_colwise_e5m2(bf16_dev(dy), to_dev(off), to_dev(poff),
                                                       col_rows_cap=cap)
    wdyc, wdys = Q.mxfp8_colwise(dy, off, poff, elem="e5m2")
    n = int(poff[-1])
    assert np.array_equal(host_u8(dyc)[:n * N], wdyc)
    assert np.array_equal(host_u8(dys)[:n * N // 32], wdys)
    xq = bsg.grouped_quantize_mxfp8(bf16_dev(x), to_dev(off), rowwise=False,
                                    padded_offsets=to_dev(poff), col_rows_cap=cap)
    xc, xs = Q.mxfp8_colwise(x, off, poff)
    ref = GM.mxfp8_wgrad(wdyc, wdys, xc, xs, poff, N, K, elem_a="e5m2")
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((G, N, K), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_WGRAD_NT_E5M2, dyc, dys, xq["col_data"], xq["col_scales"],
                           to_dev(poff), cap, N, K, out=out,
                           out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g] == 0:
            assert np.all(y[g] == 0.0) and not np.any(np.signbit(y[g])), "empty expert must be +0"
        else:
            gemm_tolerance_check(y[g], ref[g], out_f32, "group %d" % g)


def test_fprop_end_to_end_tiny_config():
    """The tiny MoE config: GPU quantize -> GPU GEMM vs oracle quantize -> oracle GEMM."""
    w = workloads.get("tiny")
    t = workloads.tensors(w, device=device())
    xb, wb = workloads.bf16_bits(t["x"]), workloads.bf16_bits(t["w"])
    G, N, K = w.G, w.n, w.k
    _, off = O.group_offsets(w.sizes)
    ad, asc = Q.mxfp8_rowwise(xb, off)
    bd, bsc = Q.mxfp8_rowwise(wb.reshape(G * N, K), np.array([0, G * N]))
    ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)

    _, doff = bsg.group_offsets_i32_to_i64(to_dev(w.sizes))
    qa = bsg.grouped_quantize_mxfp8(t["x"], doff)
    woff = to_dev(np.array([0, G * N]))
    qb = bsg.grouped_quantize_mxfp8(t["w"].view(G * N, K), woff)
    out = torch.full((w.rows_cap, N), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, qa["row_data"], qa["row_scales"], qb["row_data"],
                           qb["row_scales"], doff, w.rows_cap, N, K, out=out,
                           out_dtype=bsg.BSG_OUT_F32)
    y = host(out).astype(np.float64)
    assert np.all(np.isnan(y[int(off[-1]):])), "capacity rows must stay untouched"
    for g in range(G):
        gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], True, "group %d" % g)


def test_grouped_equals_separate_calls_and_determinism():
    rng = np.random.default_rng(31)
    sizes, off, x, w, ad, asc, bd, bsc, rows_cap = _fprop_operands(rng, [257, 0, 90, 400], 384, 512)
    a, a_s = _upload_rows(ad, asc, rows_cap)
    B, Bs, doff = to_dev(bd), to_dev(bsc), to_dev(off)
    y = bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, a_s, B, Bs, doff, rows_cap, 512, 384,
                               out_dtype=bsg.BSG_OUT_F32)
    y2 = bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, a_s, B, Bs, doff, rows_cap, 512, 384,
                                out_dtype=bsg.BSG_OUT_F32)
    assert torch.equal(y, y2)
    for g in range(4):
        if sizes[g] == 0:
            continue
        r0, r1 = int(off[g]), int(off[g + 1])
        one = bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a[r0:r1].contiguous(),
                                     a_s[:, r0:r1].contiguous(), B[g:g + 1].contiguous(),
                                     Bs[:, g * 512:(g + 1) * 512].contiguous(),
                                     to_dev(np.array([0, r1 - r0])), r1 - r0, 512, 384,
                                     out_dtype=bsg.BSG_OUT_F32)
        assert torch.equal(one, y[r0:r1])


def test_all_empty_routing():
    rng = np.random.default_rng(4)
    K, N = 128, 256
    a = to_dev(np.zeros((64, K), np.uint8))
    a_s = to_dev(np.zeros(bsg.mx_scale_shape(64, K), np.uint8))
    b = to_dev(rng.integers(0, 255, (2, N, K)).astype(np.uint8) & 0x77)
    b_s = to_dev(np.full(bsg.mx_scale_shape(2 * N, K), 127, np.uint8))
    out = torch.full((64, N), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, a, a_s, b, b_s, to_dev(np.zeros(3, np.int64)), 64, N, K,
                           out=out, out_dtype=bsg.BSG_OUT_F32)
    assert torch.isnan(out).all()


def test_hip_graph_replay_with_new_sizes():
    """Sizes live on the device: a captured quantize + GEMM replays correctly
    after the sizes change, with no host dependence on them."""
    dev = device()
    rng = np.random.default_rng(8)
    G, K, N, rows_cap = 3, 256, 256, 600
    xb = _bits(rng, (rows_cap, K))
    wb = _bits(rng, (G * N, K), 0.02)
    x, wt = bf16_dev(xb), bf16_dev(wb)
    sizes = torch.tensor([100, 0, 200], dtype=torch.int32, device=dev)
    qb = bsg.grouped_quantize_mxfp8(wt, to_dev(np.array([0, G * N])))
    s64 = torch.empty(G, dtype=torch.int64, device=dev)
    off = torch.empty(G + 1, dtype=torch.int64, device=dev)
    rd = torch.empty((rows_cap, K), dtype=torch.uint8, device=dev)
    rs = torch.empty(bsg.mx_scale_shape(rows_cap, K), dtype=torch.uint8, device=dev)
    out = torch.empty((rows_cap, N), dtype=torch.float32, device=dev)

    def step():
        bsg.group_offsets_i32_to_i64(sizes, sizes_i64=s64, offsets=off)
        bsg.grouped_quantize_mxfp8(x, off, row_data=rd, row_scales=rs)
        bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, rd, rs, qb["row_data"], qb["row_scales"], off,
                               rows_cap, N, K, out=out, out_dtype=bsg.BSG_OUT_F32)

    step()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    bd, bsc = Q.mxfp8_rowwise(wb, np.array([0, G * N]))
    for new in ([100, 0, 200], [50, 250, 300], [0, 0, 600], [600, 0, 0]):
        sizes.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _, o = O.group_offsets(np.array(new))
        ad, asc = Q.mxfp8_rowwise(xb, o)
        ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, o, K)
        y = host(out).astype(np.float64)
        for gi in range(G):
            gemm_tolerance_check(y[o[gi]:o[gi + 1]], ref[o[gi]:o[gi + 1]], True, str(new))
        eager = out.clone()
        step()
        torch.cuda.synchronize()
        assert torch.equal(eager[:int(o[-1])], out[:int(o[-1])])


# ---------------------------------------------------------------- NVFP4

def _nv_operands(rng, sizes, npg, K, rows_cap):
    sizes = np.array(sizes, np.int32)
    _, off = O.group_offsets(sizes)
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    ap, asc, at = Q.nvfp4_rowscaled(x, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(w, np.array([0, sum(npg)]))
    return sizes, off, ap, asc, at, bp, bsc, bt


NV_CASES = [
    ([100, 0, 257, 31], [64, 128, 96, 256], 256, 450),
    ([300, 211], [2048, 4096], 512, 600),
    ([0, 0], [64, 64], 64, 16),
    ([(7 * i) % 41 if i % 5 else 0 for i in range(256)], [32 + 32 * (i % 3) for i in range(256)],
     64, 5200),                          # 256 groups (maximum), three output widths
]


@pytest.mark.parametrize("sizes,npg,K,rows_cap", NV_CASES)
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("out_f32", [True, False])
def test_nvfp4_gemm_parity(sizes, npg, K, rows_cap, fused, out_f32):
    rng = np.random.default_rng(K + rows_cap)
    sizes, off, ap, asc, at, bp, bsc, bt = _nv_operands(rng, sizes, npg, K, rows_cap)
    live = int(off[-1])
    ld = max(npg) + 8

    def pad_rows(a, rows, dtype=None):
        o = np.zeros((rows,) + a.shape[1:], a.dtype)
        o[:a.shape[0]] = a
        return to_dev(o)

    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((rows_cap, ld), float("nan"), dtype=dt, device=device())
    scratch = None if fused else torch.empty((rows_cap, ld), dtype=torch.float32, device=device())
    bsg.grouped_gemm_nvfp4_rowscaled(pad_rows(ap, rows_cap), pad_rows(asc, rows_cap),
                                     pad_rows(at, rows_cap), to_dev(off), K, to_dev(bp),
                                     to_dev(bsc), to_dev(bt), npg, out=out, ld_out=ld,
                                     out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                                     scratch=scratch)
    y = bf16_out_to_f64(out)
    ref = GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)
    for g, (rows, r) in enumerate(ref):
        if len(rows) == 0:
            continue
        gemm_tolerance_check(y[rows][:, :npg[g]], r, out_f32, "group %d" % g)
        assert np.all(np.isnan(y[rows][:, npg[g]:])), "columns past N_g must stay untouched"
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


def test_nvfp4_fused_equals_unfused():
    rng = np.random.default_rng(77)
    sizes, off, ap, asc, at, bp, bsc, bt = _nv_operands(rng, [130, 260], [256, 512], 512, 390)
    args = (to_dev(ap), to_dev(asc), to_dev(at), to_dev(off), 512, to_dev(bp), to_dev(bsc), to_dev(bt),
            [256, 512])
    y1 = bsg.grouped_gemm_nvfp4_rowscaled(*args, ld_out=512)
    scratch = torch.empty((390, 512), dtype=torch.float32, device=device())
    y2 = bsg.grouped_gemm_nvfp4_rowscaled(*args, ld_out=512, scratch=scratch)
    torch.cuda.synchronize()
    assert torch.equal(y1[:130, :256], y2[:130, :256]) and torch.equal(y1[130:], y2[130:])


def test_nvfp4_end_to_end():
    rng = np.random.default_rng(12)
    sizes = np.array([150, 0, 106], np.int32)
    npg = [128, 256, 384]
    K, rows_cap = 256, 300
    xb = _bits(rng, (rows_cap, K))
    wb = _bits(rng, (sum(npg), K), 0.02)
    _, off = O.group_offsets(sizes)
    doff = to_dev(off)
    a = bsg.grouped_quantize_nvfp4_rowscaled(bf16_dev(xb), doff)
    b = bsg.grouped_quantize_nvfp4_rowscaled(bf16_dev(wb), to_dev(np.array([0, sum(npg)])))
    out = torch.full((rows_cap, max(npg)), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_gemm_nvfp4_rowscaled(a[0], a[1], a[2], doff, K, b[0], b[1], b[2], npg, out=out,
                                     out_dtype=bsg.BSG_OUT_F32)
    y = host(out).astype(np.float64)
    assert np.all(np.isnan(y[int(off[-1]):])), "capacity rows must stay untouched"
    ap, asc, at = Q.nvfp4_rowscaled(xb, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(wb, np.array([0, sum(npg)]))
    for g, (rows, r) in enumerate(GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, True, "group %d" % g)


# ---------------------------------------------------------------- NVFP4 per-tensor

NVT_CASES = [
    ([100, 0, 257, 31], [64, 128, 96, 256], 256, 450),
    ([300, 211], [2048, 4096], 512, 600),
    ([0, 0], [64, 64], 64, 16),
    ([(7 * i) % 41 if i % 5 else 0 for i in range(256)], [32 + 32 * (i % 3) for i in range(256)],
     64, 5200),                          # 256 groups (maximum), three output widths
]


@pytest.mark.parametrize("sizes,npg,K,rows_cap", NVT_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_nvfp4_pertensor_gemm_parity(sizes, npg, K, rows_cap, out_f32):
    rng = np.random.default_rng(2 * K + rows_cap)
    sizes = np.array(sizes, np.int32)
    _, off = O.group_offsets(sizes)
    live = int(off[-1])
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    boff = np.concatenate([[0], np.cumsum(npg)])
    ap, asc, aam = Q.nvfp4_pertensor(x, off)
    bp, bsc, bam = Q.nvfp4_pertensor(w, boff)
    ld = max(npg) + 8

    def pad_rows(a, rows):
        o = np.zeros((rows,) + a.shape[1:], a.dtype)
        o[:a.shape[0]] = a
        return to_dev(o)

    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((rows_cap, ld), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_nvfp4_pertensor(pad_rows(ap, rows_cap), pad_rows(asc, rows_cap), to_dev(aam),
                                     to_dev(off), K, to_dev(bp), to_dev(bsc), to_dev(bam), npg,
                                     out=out, ld_out=ld,
                                     out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16)
    y = bf16_out_to_f64(out)
    ref = GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K)
    for g, (rows, r) in enumerate(ref):
        if len(rows) == 0:
            continue
        gemm_tolerance_check(y[rows][:, :npg[g]], r, out_f32, "group %d" % g)
        assert np.all(np.isnan(y[rows][:, npg[g]:])), "columns past N_g must stay untouched"
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


def test_nvfp4_pertensor_end_to_end():
    rng = np.random.default_rng(13)
    sizes = np.array([150, 0, 106], np.int32)
    npg = [128, 256, 384]
    K, rows_cap = 256, 300
    xb = _bits(rng, (rows_cap, K))
    wb = _bits(rng, (sum(npg), K), 0.02)
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    doff = to_dev(off)
    a = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(xb), doff)
    b = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(wb), to_dev(boff))
    out = torch.full((rows_cap, max(npg)), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_gemm_nvfp4_pertensor(a[0], a[1], a[2], doff, K, b[0], b[1], b[2], npg, out=out,
                                     out_dtype=bsg.BSG_OUT_F32)
    y = host(out).astype(np.float64)
    assert np.all(np.isnan(y[int(off[-1]):])), "capacity rows must stay untouched"
    ap, asc, aam = Q.nvfp4_pertensor(xb, off)
    bp, bsc, bam = Q.nvfp4_pertensor(wb, boff)
    for g, (rows, r) in enumerate(GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K)):
        if len(rows):
            gemm_tolerance_check(y[rows][:, :npg[g]], r, True, "group %d" % g)


def test_nvfp4_pertensor_hip_graph_replay_with_new_sizes():
    """The per-tensor path (amax clear kernel, group amax with atomics, cast,
    GEMM) captured once and replayed after the device sizes change: every
    replay equals the oracle and a fresh eager call (the amax is cleared by a
    kernel, not a memset, so replays start from zero)."""
    dev = device()
    rng = np.random.default_rng(18)
    G, K, rows_cap = 3, 256, 600
    npg = [128, 256, 64]
    xb = _bits(rng, (rows_cap, K))
    wb = _bits(rng, (sum(npg), K), 0.02)
    x, wt = bf16_dev(xb), bf16_dev(wb)
    boff = np.concatenate([[0], np.cumsum(npg)])
    qb = bsg.grouped_quantize_nvfp4_pertensor(wt, to_dev(boff))
    sizes = torch.tensor([100, 0, 200], dtype=torch.int32, device=dev)
    off = torch.empty(G + 1, dtype=torch.int64, device=dev)
    ad = torch.empty((rows_cap, K // 2), dtype=torch.uint8, device=dev)
    asc = torch.empty((rows_cap, K // 16), dtype=torch.uint8, device=dev)
    aam = torch.empty(G, dtype=torch.float32, device=dev)
    out = torch.empty((rows_cap, max(npg)), dtype=torch.float32, device=dev)

    def step():
        bsg.group_offsets_i32_to_i64(sizes, offsets=off)
        bsg.grouped_quantize_nvfp4_pertensor(x, off, data=ad, block_scales=asc, amax=aam)
        bsg.grouped_gemm_nvfp4_pertensor(ad, asc, aam, off, K, qb[0], qb[1], qb[2], npg, out=out,
                                         out_dtype=bsg.BSG_OUT_F32)

    step()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step()
    torch.cuda.synchronize()
    bp, bsc, bam = Q.nvfp4_pertensor(wb, boff)
    for new in ([100, 0, 200], [50, 250, 300], [0, 0, 600], [600, 0, 0], [10, 20, 30]):
        sizes.copy_(torch.tensor(new, dtype=torch.int32))
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _, o = O.group_offsets(np.array(new))
        ap, asn, am = Q.nvfp4_pertensor(xb, o)
        assert np.array_equal(host(aam).view(np.uint32), am.view(np.uint32)), new
        y = host(out).astype(np.float64)
        for gi, (rows, r) in enumerate(GM.nvfp4_pertensor_fprop(ap, asn, am, o, bp, bsc, bam, npg, K)):
            if len(rows):
                gemm_tolerance_check(y[rows][:, :npg[gi]], r, True, str(new))
        eager = out.clone()
        step()
        torch.cuda.synchronize()
        live = int(o[-1])
        assert torch.equal(eager[:live].nan_to_num(7.0), out[:live].nan_to_num(7.0))


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("out_f32", [True, False])
def test_nvfp4_gemm_accumulate(fused, out_f32):
    """Copy-or-accumulate of the row-scaled flow: with the accumulate flag the
    live rows and columns n < N_g become previous + Y (added in float32 and
    rounded once); columns past N_g and capacity rows keep their contents."""
    rng = np.random.default_rng(93 + fused)
    sizes, npg, K, rows_cap = [100, 0, 257, 31], [64, 128, 96, 256], 256, 450
    sizes, off, ap, asc, at, bp, bsc, bt = _nv_operands(rng, sizes, npg, K, rows_cap)
    live = int(off[-1])
    ld = max(npg) + 8
    prev = (rng.standard_normal((rows_cap, ld)) * 3).astype(np.float32)
    prev[live:] = np.nan
    for g in range(len(npg)):
        prev[off[g]:off[g + 1], npg[g]:] = np.nan
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.from_numpy(prev).to(dt).to(device())
    c_prev = bf16_out_to_f64(out)
    scratch = None if fused else torch.empty((rows_cap, ld), dtype=torch.float32, device=device())

    def pad_rows(a):
        o = np.zeros((rows_cap,) + a.shape[1:], a.dtype)
        o[:a.shape[0]] = a
        return to_dev(o)

    bsg.grouped_gemm_nvfp4_rowscaled(pad_rows(ap), pad_rows(asc), pad_rows(at), to_dev(off), K,
                                     to_dev(bp), to_dev(bsc), to_dev(bt), npg, out=out, ld_out=ld,
                                     out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                                     scratch=scratch, accumulate=True)
    y = bf16_out_to_f64(out)
    for g, (rows, r) in enumerate(GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)):
        if len(rows) == 0:
            continue
        gemm_tolerance_check(y[rows][:, :npg[g]], r + c_prev[rows][:, :npg[g]], out_f32,
                             "group %d" % g)
        assert np.all(np.isnan(y[rows][:, npg[g]:])), "columns past N_g must stay untouched"
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


@pytest.mark.parametrize("ld_extra", [1, 2])
@pytest.mark.parametrize("accumulate", [False, True])
def test_nvfp4_scratch_postscale_strides_and_tails(ld_extra, accumulate):
    """The two-step flow's post-scale kernel with output widths that are not
    multiples of 4 (its element-wise tail) and a row stride that is (four
    columns per thread) or is not (element-wise throughout)."""
    rng = np.random.default_rng(61 + ld_extra + 2 * accumulate)
    npg = [36, 130, 64]
    sizes, off, ap, asc, at, bp, bsc, bt = _nv_operands(rng, [70, 0, 150], npg, 128, 260)
    live = int(off[-1])
    ld = max(npg) + ld_extra                  # 131: odd stride; 132: multiple of 4
    prev = (rng.standard_normal((260, ld)) * 2).astype(np.float32)
    prev[live:] = np.nan
    for g in range(len(npg)):
        prev[off[g]:off[g + 1], npg[g]:] = np.nan
    out = torch.from_numpy(prev).to(device())
    c_prev = bf16_out_to_f64(out)
    scratch = torch.empty((260, ld), dtype=torch.float32, device=device())

    def pad_rows(a):
        o = np.zeros((260,) + a.shape[1:], a.dtype)
        o[:a.shape[0]] = a
        return to_dev(o)

    bsg.grouped_gemm_nvfp4_rowscaled(pad_rows(ap), pad_rows(asc), pad_rows(at), to_dev(off), 128,
                                     to_dev(bp), to_dev(bsc), to_dev(bt), npg, out=out, ld_out=ld,
                                     out_dtype=bsg.BSG_OUT_F32, scratch=scratch,
                                     accumulate=accumulate)
    y = bf16_out_to_f64(out)
    for g, (rows, r) in enumerate(GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, 128)):
        if len(rows) == 0:
            continue
        want = r + c_prev[rows][:, :npg[g]] if accumulate else r
        gemm_tolerance_check(y[rows][:, :npg[g]], want, True, "group %d" % g)
        assert np.all(np.isnan(y[rows][:, npg[g]:])), "columns past N_g must stay untouched"
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


# ---------------------------------------------------------------- NVFP4 row-scaled wgrad

NVW_CASES = [
    ([37, 0, 130, 5], 96, 160),          # ragged n / k tails (not multiples of 256)
    ([300, 1, 0, 700], 256, 512),
    ([0, 0, 64], 64, 32),
    ([1000], 512, 288),                  # a long contraction (1024 padded tokens)
]


@pytest.mark.parametrize("sizes,N,K", NVW_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_nvfp4_wgrad_parity(sizes, N, K, out_f32):
    rng = np.random.default_rng(N * 7 + K)
    sizes = np.array(sizes, np.int32)
    G, M = len(sizes), int(sizes.sum())
    dy = _bits(rng, (max(M, 1), N))
    x = _bits(rng, (max(M, 1), K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    cap = max(M, 1) + 128 * G
    dyc, dys, dyo = bsg.grouped_quantize_nvfp4_rowscaled_colwise(
        bf16_dev(dy), to_dev(off), to_dev(poff), col_rows_cap=cap)
    xc, xs, xo = bsg.grouped_quantize_nvfp4_rowscaled_colwise(
        bf16_dev(x), to_dev(off), to_dev(poff), col_rows_cap=cap)
    # operands are the oracle's bytes (the quantize itself is pinned bit-exact elsewhere)
    wdyc, wdys, wdyo = Q.nvfp4_rowscaled_colwise(dy, off, poff)
    n = int(poff[-1])
    assert np.array_equal(host_u8(dyc)[:n * N // 2], wdyc)
    assert np.array_equal(host(dyo).view(np.uint32), wdyo.view(np.uint32))
    wxc, wxs, wxo = Q.nvfp4_rowscaled_colwise(x, off, poff)
    ref = GM.nvfp4_rowscaled_wgrad(wdyc, wdys, wdyo, wxc, wxs, wxo, poff, N, K)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((G, N, K), float("nan"), dtype=dt, device=device())
    status = torch.zeros(1, dtype=torch.int32, device=device())
    bsg.grouped_gemm_nvfp4_rowscaled_wgrad(dyc, dys, dyo, xc, xs, xo, to_dev(poff), N, K,
                                           col_rows_cap=cap, out=out, status=status,
                                           out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16)
    y = bf16_out_to_f64(out)
    assert int(host(status)[0]) == 0
    for g in range(G):
        if sizes[g] == 0:
            assert np.all(y[g] == 0.0) and not np.any(np.signbit(y[g])), "empty expert must be +0"
        else:
            gemm_tolerance_check(y[g], ref[g], out_f32, "group %d" % g)


# ---------------------------------------------------------------- MXFP8 dgrad (E5M2 x E4M3)

DGRAD_CASES = [
    ([37, 0, 130, 5], 128, 96),          # n tail (96 < 256), one contraction step pair
    ([300, 1, 0, 700], 384, 256),
    ([64], 1024, 160),
]


@pytest.mark.parametrize("sizes,K,N", DGRAD_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_dgrad_parity(sizes, K, N, out_f32):
    """dX [rows, N] = dY [rows, K] (E5M2) x W_g [K, N] (E4M3 columnwise copy)."""
    rng = np.random.default_rng(K * 11 + N)
    sizes = np.array(sizes, np.int32)
    G, M = len(sizes), int(sizes.sum())
    rows_cap = M + 17
    dy = _bits(rng, (rows_cap, K))
    w = _bits(rng, (G * K, N), std=0.05)
    _, off = O.group_offsets(sizes)
    woff = np.arange(G + 1, dtype=np.int64) * K
    dyd, dys = bsg.grouped_quantize_mxfp8_rowwise_e5m2(bf16_dev(dy), to_dev(off))
    wq = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(woff), rowwise=False,
                                    padded_offsets=to_dev(woff), col_rows_cap=G * K)
    rd, rs = Q.mxfp8_rowwise(dy, off, elem="e5m2")
    wtd, wts = Q.mxfp8_colwise(w, woff, woff)
    assert np.array_equal(host_u8(dyd)[:M], rd)
    assert np.array_equal(host_u8(wq["col_data"]), wtd)
    ref = GM.mxfp8_dgrad(rd, rs, wtd, wts, off, K, N)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((rows_cap, N), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_mxfp8(bsg.BSG_DGRAD_NN, dyd, dys, wq["col_data"], wq["col_scales"],
                           to_dev(off), rows_cap, N, K, out=out,
                           out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g]:
            gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32,
                                 "group %d" % g)
    assert np.all(np.isnan(y[M:])), "capacity rows untouched"


# ---------------------------------------------------------------- epilogue terms (alpha, beta, bias)

EPI_CASES = [
    ([300, 0, 17, 513, 130], 512, 640, 1000),
    ([5, 300, 0, 40], 128, 258, 400),   # odd row stride: the element path
]


@pytest.mark.parametrize("sizes,K,N,rows_cap", EPI_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
@pytest.mark.parametrize("terms", ["all", "bias_only", "alpha_beta"])
def test_fprop_epilogue_parity(sizes, K, N, rows_cap, out_f32, terms):
    rng = np.random.default_rng(K + N + 3 * len(sizes))
    sizes, off, x, w, ad, asc, bd, bsc, rows_cap = _fprop_operands(rng, sizes, K, N, rows_cap)
    G = len(sizes)
    s_ref = GM.mxfp8_fprop(ad, asc, bd, bsc, off, K)
    live = int(off[-1])
    grp = np.searchsorted(off, np.arange(live), side="right") - 1
    alpha = (rng.uniform(-2, 2, G)).astype(np.float32) if terms != "bias_only" else None
    beta = np.where(np.arange(G) % 2 == 0, rng.uniform(0.5, 1.5, G), 0.0).astype(np.float32) \
        if terms != "bias_only" else None
    bias = rng.standard_normal((G, N)).astype(np.float32) if (terms != "alpha_beta" and N % 4 == 0) \
        else None
    dt = torch.float32 if out_f32 else torch.bfloat16
    c0 = torch.from_numpy(rng.standard_normal((rows_cap, N)).astype(np.float32)).to(dt)
    if beta is not None:
        nan_rows = torch.from_numpy(np.repeat(beta[grp] == 0, 1)).to(device())
        c0[:live][nan_rows.cpu()] = float("nan")      # groups with beta 0 must not read it
    c0[live:] = float("nan")
    out = c0.to(device())
    c_prev = bf16_out_to_f64(out)
    a, a_s = _upload_rows(ad, asc, rows_cap)
    bsg.grouped_gemm_mxfp8_ex(bsg.BSG_FPROP_TN, a, a_s, to_dev(bd), to_dev(bsc), to_dev(off),
                              rows_cap, N, K, out,
                              out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                              alpha=None if alpha is None else to_dev(alpha),
                              beta=None if beta is None else to_dev(beta),
                              bias=None if bias is None else to_dev(bias))
    ref = GM.epilogue(s_ref[:live], grp, alpha, beta, c_prev[:live], bias)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g]:
            gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32,
                                 "group %d" % g)
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


@pytest.mark.parametrize("out_f32", [True, False])
def test_wgrad_accumulate_into_main_grad(out_f32):
    """WGRAD with beta = 1 accumulating into an existing dW (the main-grad use),
    alpha per expert, a bias over the k output columns; an empty expert gets
    beta * old + bias (its product is zero)."""
    rng = np.random.default_rng(41)
    sizes = np.array([37, 0, 130, 5], np.int32)
    G, M, N, K = 4, int(sizes.sum()), 160, 96
    dy = _bits(rng, (M, N))
    x = _bits(rng, (M, K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    dyc, dys = Q.mxfp8_colwise(dy, off, poff)
    xc, xs = Q.mxfp8_colwise(x, off, poff)
    s_ref = GM.mxfp8_wgrad(dyc, dys, xc, xs, poff, N, K)
    cap = max(int(poff[-1]), 128)

    def pad(arr, n):
        o = np.zeros(n, np.uint8)
        o[:len(arr)] = arr
        return to_dev(o)

    alpha = rng.uniform(0.5, 2, G).astype(np.float32)
    beta = np.ones(G, np.float32)
    bias = rng.standard_normal((G, K)).astype(np.float32)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.from_numpy(rng.standard_normal((G, N, K)).astype(np.float32)).to(dt).to(device())
    c_prev = bf16_out_to_f64(out)
    bsg.grouped_gemm_mxfp8_ex(bsg.BSG_WGRAD_NT, pad(dyc, cap * N), pad(dys, cap * N // 32),
                              pad(xc, cap * K), pad(xs, cap * K // 32), to_dev(poff), cap, N, K, out,
                              out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                              alpha=to_dev(alpha), beta=to_dev(beta), bias=to_dev(bias))
    y = bf16_out_to_f64(out)
    for g in range(G):
        ref = GM.epilogue(s_ref[g], np.zeros(N, np.int64), alpha[[g]], beta[[g]], c_prev[g],
                          bias[[g]])
        gemm_tolerance_check(y[g], ref, out_f32, "expert %d" % g)


@pytest.mark.parametrize("out_f32", [True, False])
def test_nvfp4_wgrad_accumulate_into_main_grad(out_f32):
    """Row-scaled NVFP4 wgrad with the accumulate flag: dW[g] = previous +
    (S * a_outer) * b_outer, rounded once; an empty expert keeps its block
    exactly."""
    rng = np.random.default_rng(57)
    sizes = np.array([37, 0, 130, 5], np.int32)
    G, M, N, K = 4, int(sizes.sum()), 96, 160
    dy = _bits(rng, (M, N))
    x = _bits(rng, (M, K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    cap = M + 128 * G
    dyc, dys, dyo = bsg.grouped_quantize_nvfp4_rowscaled_colwise(
        bf16_dev(dy), to_dev(off), to_dev(poff), col_rows_cap=cap)
    xc, xs, xo = bsg.grouped_quantize_nvfp4_rowscaled_colwise(
        bf16_dev(x), to_dev(off), to_dev(poff), col_rows_cap=cap)
    wdyc, wdys, wdyo = Q.nvfp4_rowscaled_colwise(dy, off, poff)
    wxc, wxs, wxo = Q.nvfp4_rowscaled_colwise(x, off, poff)
    ref = GM.nvfp4_rowscaled_wgrad(wdyc, wdys, wdyo, wxc, wxs, wxo, poff, N, K)
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.from_numpy(rng.standard_normal((G, N, K)).astype(np.float32)).to(dt).to(device())
    c_prev = bf16_out_to_f64(out)
    bsg.grouped_gemm_nvfp4_rowscaled_wgrad(dyc, dys, dyo, xc, xs, xo, to_dev(poff), N, K,
                                           col_rows_cap=cap, out=out, accumulate=True,
                                           out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16)
    y = bf16_out_to_f64(out)
    for g in range(G):
        if sizes[g] == 0:
            assert np.array_equal(y[g], c_prev[g]), "an empty expert keeps its block"
        else:
            gemm_tolerance_check(y[g], ref[g] + c_prev[g], out_f32, "group %d" % g)
