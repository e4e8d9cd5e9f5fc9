"""GPU checks of the split of the last round of tiles along the contraction
(grouped_gemm_mxfp8_ws): the split tiles' parts, summed in a fixed order by the
second kernel, equal the unsplit GEMM within FP32 rounding and the fp64 oracle
within the GEMM tolerance; the result is deterministic, capacity rows stay
untouched, a workspace left by another call does not matter, the split path
replays correctly from a HIP graph, and WGRAD (never split) is unchanged."""

import numpy as np
import pytest
import torch

import block_scaled_grouped_amd as bsg
from oracle import formats as F
from oracle import gemm as GM
from oracle import offsets as O
from oracle import quantize as Q
from gpu_util import bf16_dev, bf16_out_to_f64, device, gemm_tolerance_check, host, to_dev

pytestmark = pytest.mark.gpu


def _bits(rng, shape, std=1.0):
    return F.f32_to_bf16_bits_rne((rng.standard_normal(shape) * std).astype(np.float32))


def _tiles(sizes, n):
    return sum(-(-int(m) // 256) for m in sizes) * -(-n // 256)


def _fprop(rng, sizes, K, N, rows_cap):
    sizes = np.array(sizes, np.int32)
    G, live = len(sizes), int(sizes.sum())
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (G * N, K), 0.02)
    _, off = O.group_offsets(sizes)
    doff = to_dev(off)
    xq = bsg.grouped_quantize_mxfp8(bf16_dev(x), doff)
    wq = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(np.array([0, G * N])))
    ad, asc = Q.mxfp8_rowwise(x, off)
    bd, bsc = Q.mxfp8_rowwise(w, np.array([0, G * N]))
    ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    args = (bsg.BSG_FPROP_TN, xq["row_data"], xq["row_scales"], wq["row_data"], wq["row_scales"],
            doff, rows_cap, N, K)
    return args, off, ref, live


def _run(args, rows_cap, N, out_f32, ws=None):
    dt = torch.float32 if out_f32 else torch.bfloat16
    out = torch.full((rows_cap, N), float("nan"), dtype=dt, device=device())
    bsg.grouped_gemm_mxfp8(*args, out=out, out_dtype=bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16,
                           workspace=ws)
    torch.cuda.synchronize()
    return out


# (sizes, K, N, rows_cap): every tile split (10 tiles on a grid of 38), the
# same at K = 1056 (9 pairs, the last a quarter full, in 3 parts of 3: the
# last part ends in the contraction tail), and a full round followed by a partial one
# (312 tiles on up to 256 workgroups)
SPLIT_CASES = [
    ([300, 0, 700], 1024, 512, 4096),
    ([300, 0, 700], 1056, 512, 4096),
    ([2560, 1000, 0, 6170], 1024, 2048, 9984),
]


@pytest.mark.parametrize("sizes,K,N,rows_cap", SPLIT_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_split_fprop_matches_unsplit_and_oracle(sizes, K, N, rows_cap, out_f32):
    rng = np.random.default_rng(K + N + rows_cap)
    args, off, ref, live = _fprop(rng, sizes, K, N, rows_cap)
    assert _tiles(sizes, N) % 256 != 0
    ws = bsg.gemm_workspace(device())
    plain = bf16_out_to_f64(_run(args, rows_cap, N, out_f32))
    split = bf16_out_to_f64(_run(args, rows_cap, N, out_f32, ws))
    for g in range(len(sizes)):
        gemm_tolerance_check(split[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], out_f32,
                             "group %d" % g)
    assert np.all(np.isnan(split[live:])), "capacity rows must stay untouched"
    scale = np.max(np.abs(plain[:live]))
    if out_f32:
        # the same FP32 products, summed in a different order
        assert np.max(np.abs(split[:live] - plain[:live])) <= 1e-5 * scale
    else:
        # at most one bf16 rounding step apart
        assert np.all(np.abs(split[:live] - plain[:live]) <= 2.0 ** -7 * np.abs(plain[:live]) + 1e-6 * scale)
    # the split did happen: the workspace header holds the number of split tiles
    # (the partial round's) and the parts per tile
    ntiles = _tiles(sizes, N)
    hdr = host(ws[:8].view(torch.int32))
    assert hdr[0] == ntiles % min(ntiles, 256) or hdr[0] == ntiles, hdr
    assert 2 <= hdr[1] <= 8, hdr


def test_split_is_deterministic_and_ignores_a_stale_workspace():
    rng = np.random.default_rng(5)
    ws = bsg.gemm_workspace(device())
    sizes, K, N, rows_cap = SPLIT_CASES[2]
    args, off, ref, live = _fprop(rng, sizes, K, N, rows_cap)
    first = _run(args, rows_cap, N, True, ws)
    # another call through the same workspace, with another shape and split
    args2, off2, ref2, live2 = _fprop(rng, [300, 0, 700], 1024, 512, 4096)
    other = bf16_out_to_f64(_run(args2, 4096, 512, True, ws))
    for g in range(3):
        gemm_tolerance_check(other[off2[g]:off2[g + 1]], ref2[off2[g]:off2[g + 1]], True)
    again = _run(args, rows_cap, N, True, ws)
    assert torch.equal(first[:live], again[:live])


def test_split_dgrad_matches_oracle():
    """DGRAD (E5M2 dY x E4M3 columnwise W) with a partial last round."""
    rng = np.random.default_rng(9)
    sizes = np.array([2560, 1000, 0, 6170], np.int32)
    K, N = 1024, 2048
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
    ref = GM.mxfp8_dgrad(rd, rs, wtd, wts, off, K, N)
    assert _tiles(sizes, N) % 256 != 0
    args = (bsg.BSG_DGRAD_NN, dyd, dys, wq["col_data"], wq["col_scales"], to_dev(off), rows_cap, N, K)
    ws = bsg.gemm_workspace(device())
    y = bf16_out_to_f64(_run(args, rows_cap, N, True, ws))
    plain = bf16_out_to_f64(_run(args, rows_cap, N, True))
    for g in range(G):
        if sizes[g]:
            gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], True, "group %d" % g)
    assert np.max(np.abs(y[:M] - plain[:M])) <= 1e-5 * np.max(np.abs(plain[:M]))
    assert np.all(np.isnan(y[M:]))


def test_wgrad_with_workspace_is_unchanged():
    rng = np.random.default_rng(13)
    sizes = np.array([2049, 0, 3001, 0], np.int32)
    N, K = 256, 288
    G, M = len(sizes), int(sizes.sum())
    dy = _bits(rng, (M, N))
    x = _bits(rng, (M, K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    cap = int(poff[-1])
    dq = bsg.grouped_quantize_mxfp8(bf16_dev(dy), to_dev(off), rowwise=False,
                                    padded_offsets=to_dev(poff), col_rows_cap=cap)
    xq = bsg.grouped_quantize_mxfp8(bf16_dev(x), to_dev(off), rowwise=False,
                                    padded_offsets=to_dev(poff), col_rows_cap=cap)
    args = (bsg.BSG_WGRAD_NT, dq["col_data"], dq["col_scales"], xq["col_data"], xq["col_scales"],
            to_dev(poff), cap, N, K)
    outs = []
    for ws in (None, bsg.gemm_workspace(device())):
        out = torch.full((G, N, K), float("nan"), dtype=torch.float32, device=device())
        bsg.grouped_gemm_mxfp8(*args, out=out, out_dtype=bsg.BSG_OUT_F32, workspace=ws)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_split_hip_graph_replay_with_new_sizes():
    """The GEMM and the second kernel captured once; replays with other device
    group sizes (so other tiles are split) match eager split calls."""
    rng = np.random.default_rng(17)
    K, N, rows_cap, G = 1024, 2048, 9984, 4
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (G * N, K), 0.02)
    dx = bf16_dev(x)
    wq = bsg.grouped_quantize_mxfp8(bf16_dev(w), to_dev(np.array([0, G * N])))
    off = torch.zeros(G + 1, dtype=torch.int64, device=device())
    ws = bsg.gemm_workspace(device())
    out = torch.zeros((rows_cap, N), dtype=torch.float32, device=device())
    xq = bsg.grouped_quantize_mxfp8(dx, off)

    def step():
        bsg.grouped_quantize_mxfp8(dx, off, row_data=xq["row_data"], row_scales=xq["row_scales"])
        bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, xq["row_data"], xq["row_scales"], wq["row_data"],
                               wq["row_scales"], off, rows_cap, N, K, out=out,
                               out_dtype=bsg.BSG_OUT_F32, workspace=ws)

    off.copy_(to_dev(np.array([0, 2560, 3560, 3560, 9730])))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for new in ([0, 1000, 1000, 7000, 9984], [0, 300, 2900, 2900, 6000], [0, 2560, 3560, 3560, 9730]):
        off.copy_(to_dev(np.array(new)))
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        replayed = out.clone()
        out.zero_()
        step()
        torch.cuda.synchronize()
        live = new[-1]
        assert torch.equal(replayed[:live], out[:live]), new


# ---------------------------------------------------------------- NVFP4
# (sizes, n_per_group, K, rows_cap): every tile split (13 tiles on a grid of
# 126), and a full round followed by a partial one (296 tiles on 256)
NV_SPLIT_CASES = [
    ([300, 0, 700], [512, 256, 768], 1024, 9984),
    ([2560, 1000, 0, 6170], [2048, 1024, 512, 2048], 1024, 9984),
    # k % 64 == 32 (2-byte scale pieces) and a partial last stage in the last part
    ([300, 0, 700], [512, 256, 768], 1056, 9984),
    # 200 groups, every other one empty: 100 tiles of one group each, split 2 ways
    ([(37 * i) % 200 + 1 if i % 2 else 0 for i in range(200)],
     [32 * (1 + i % 8) for i in range(200)], 512, 10500),
]


def _nv_tiles(sizes, npg):
    return sum(-(-int(m) // 256) * -(-int(n) // 256) for m, n in zip(sizes, npg))


def _pad_rows(a, rows):
    o = np.zeros((rows,) + a.shape[1:], a.dtype)
    o[:a.shape[0]] = a
    return to_dev(o)


def _nv_check(y, ref, npg, off, live, out_f32):
    for g, (rows, r) in enumerate(ref):
        if len(rows) == 0:
            continue
        gemm_tolerance_check(y[rows][:, :npg[g]], r, out_f32, "group %d" % g)
        assert np.all(np.isnan(y[rows][:, npg[g]:])), "columns past N_g must stay untouched"
    assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


def _nv_header(ws, sizes, npg):
    ntiles = _nv_tiles(sizes, npg)
    hdr = host(ws[:8].view(torch.int32))
    assert hdr[0] == ntiles % min(ntiles, 256) or hdr[0] == ntiles, hdr
    assert 2 <= hdr[1] <= 8, hdr


@pytest.mark.parametrize("sizes,npg,K,rows_cap", NV_SPLIT_CASES)
@pytest.mark.parametrize("out_f32", [True, False])
def test_nvfp4_pertensor_split_matches_unsplit_and_oracle(sizes, npg, K, rows_cap, out_f32):
    rng = np.random.default_rng(3 * K + rows_cap + out_f32)
    sizes = np.array(sizes, np.int32)
    _, off = O.group_offsets(sizes)
    live = int(off[-1])
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    boff = np.concatenate([[0], np.cumsum(npg)])
    ap, asc, aam = Q.nvfp4_pertensor(x, off)
    bp, bsc, bam = Q.nvfp4_pertensor(w, boff)
    ld = max(npg) + 8
    args = (_pad_rows(ap, rows_cap), _pad_rows(asc, rows_cap), to_dev(aam), to_dev(off), K,
            to_dev(bp), to_dev(bsc), to_dev(bam), npg)
    dt = torch.float32 if out_f32 else torch.bfloat16
    od = bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16
    ws = bsg.gemm_workspace(device())
    outs = []
    for wsx in (None, ws):
        out = torch.full((rows_cap, ld), float("nan"), dtype=dt, device=device())
        bsg.grouped_gemm_nvfp4_pertensor(*args, out=out, ld_out=ld, out_dtype=od, workspace=wsx)
        torch.cuda.synchronize()
        outs.append(bf16_out_to_f64(out))
    plain, split = outs
    _nv_check(split, GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K), npg, off,
              live, out_f32)
    _nv_header(ws, sizes, npg)
    fin = np.isfinite(plain)
    assert np.array_equal(fin, np.isfinite(split))
    scale = np.max(np.abs(plain[fin]))
    if out_f32:
        assert np.max(np.abs(split[fin] - plain[fin])) <= 1e-5 * scale
    else:
        assert np.all(np.abs(split[fin] - plain[fin]) <= 2.0 ** -7 * np.abs(plain[fin]) + 1e-6 * scale)


@pytest.mark.parametrize("sizes,npg,K,rows_cap", NV_SPLIT_CASES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_nvfp4_rowscaled_split_matches_oracle(sizes, npg, K, rows_cap, accumulate):
    """The split's second kernel applies the row and column outer scales, and
    with the accumulate flag adds to the output's previous contents."""
    rng = np.random.default_rng(5 * K + rows_cap + accumulate)
    sizes = np.array(sizes, np.int32)
    _, off = O.group_offsets(sizes)
    live = int(off[-1])
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    ap, asc, at = Q.nvfp4_rowscaled(x, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(w, np.array([0, sum(npg)]))
    ld = max(npg) + 4
    prev = (rng.standard_normal((rows_cap, ld)) * 3).astype(np.float32)
    prev[live:] = np.nan
    for g in range(len(npg)):
        prev[off[g]:off[g + 1], npg[g]:] = np.nan
    out = torch.from_numpy(prev if accumulate else np.full_like(prev, np.nan)).to(device())
    c_prev = bf16_out_to_f64(out)
    ws = bsg.gemm_workspace(device())
    bsg.grouped_gemm_nvfp4_rowscaled(_pad_rows(ap, rows_cap), _pad_rows(asc, rows_cap),
                                     _pad_rows(at, rows_cap), to_dev(off), K, to_dev(bp),
                                     to_dev(bsc), to_dev(bt), npg, out=out, ld_out=ld,
                                     out_dtype=bsg.BSG_OUT_F32, accumulate=accumulate,
                                     workspace=ws)
    torch.cuda.synchronize()
    y = bf16_out_to_f64(out)
    ref = GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)
    if accumulate:
        ref = [(rows, r + c_prev[rows][:, :npg[g]]) for g, (rows, r) in enumerate(ref)]
    _nv_check(y, ref, npg, off, live, True)
    _nv_header(ws, sizes, npg)


def test_nvfp4_split_is_deterministic_and_graph_safe():
    """Two split calls give the same bits (also with another call through the
    same workspace between them), and a captured split call replays them."""
    rng = np.random.default_rng(41)
    sizes, npg, K, rows_cap = NV_SPLIT_CASES[1]
    sizes = np.array(sizes, np.int32)
    _, off = O.group_offsets(sizes)
    live = int(off[-1])
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    boff = np.concatenate([[0], np.cumsum(npg)])
    a = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(x), to_dev(off))
    b = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(w), to_dev(boff))
    ws = bsg.gemm_workspace(device())
    ld = max(npg)
    out = torch.zeros((rows_cap, ld), dtype=torch.float32, device=device())
    doff = to_dev(off)

    def step():
        bsg.grouped_gemm_nvfp4_pertensor(a[0], a[1], a[2], doff, K, b[0], b[1], b[2], npg, out=out,
                                         out_dtype=bsg.BSG_OUT_F32, workspace=ws)

    step()
    torch.cuda.synchronize()
    first = out.clone()
    # another call through the workspace (all of its tiles split)
    s2, n2, k2, r2 = NV_SPLIT_CASES[0]
    _, o2 = O.group_offsets(np.array(s2, np.int32))
    x2 = _bits(rng, (r2, k2))
    w2 = _bits(rng, (sum(n2), k2), 0.02)
    a2 = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(x2), to_dev(o2))
    b2 = bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(w2), to_dev(np.concatenate([[0], np.cumsum(n2)])))
    bsg.grouped_gemm_nvfp4_pertensor(a2[0], a2[1], a2[2], to_dev(o2), k2, b2[0], b2[1], b2[2], n2,
                                     out_dtype=bsg.BSG_OUT_F32, workspace=ws)
    out.zero_()
    step()
    torch.cuda.synchronize()
    assert torch.equal(first[:live], out[:live])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(first[:live], out[:live])


@pytest.mark.parametrize("accumulate", [False, True])
def test_nvfp4_split_bf16_odd_row_stride(accumulate):
    """The second kernel's element-wise stores: bf16 output with a row stride
    that is not a multiple of 4 (with and without the accumulate flag)."""
    rng = np.random.default_rng(71 + accumulate)
    sizes, npg, K, rows_cap = NV_SPLIT_CASES[0]
    sizes = np.array(sizes, np.int32)
    _, off = O.group_offsets(sizes)
    live = int(off[-1])
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    ap, asc, at = Q.nvfp4_rowscaled(x, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(w, np.array([0, sum(npg)]))
    ld = max(npg) + 3
    prev = (rng.standard_normal((rows_cap, ld)) * 3).astype(np.float32)
    prev[live:] = np.nan
    for g in range(len(npg)):
        prev[off[g]:off[g + 1], npg[g]:] = np.nan
    start = prev if accumulate else np.full_like(prev, np.nan)
    out = torch.from_numpy(start).to(torch.bfloat16).to(device())
    c_prev = bf16_out_to_f64(out)
    ws = bsg.gemm_workspace(device())
    bsg.grouped_gemm_nvfp4_rowscaled(_pad_rows(ap, rows_cap), _pad_rows(asc, rows_cap),
                                     _pad_rows(at, rows_cap), to_dev(off), K, to_dev(bp),
                                     to_dev(bsc), to_dev(bt), npg, out=out, ld_out=ld,
                                     out_dtype=bsg.BSG_OUT_BF16, accumulate=accumulate,
                                     workspace=ws)
    torch.cuda.synchronize()
    y = bf16_out_to_f64(out)
    ref = GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)
    if accumulate:
        ref = [(rows, r + c_prev[rows][:, :npg[g]]) for g, (rows, r) in enumerate(ref)]
    _nv_check(y, ref, npg, off, live, False)
    _nv_header(ws, sizes, npg)
