"""Full-size parity in the launch configuration bench.py times.

Each MoE workload is built and stepped exactly as the benchmark does (same
case objects, same buffers, same calls); then sampled outputs are compared
with the oracle, which recomputes only what those samples need: rowwise
quantization is row-local and columnwise quantization column-local within a
group, so a sampled output needs only its own rows / columns quantized.
"""

import numpy as np
import pytest
import torch

import bench
from oracle import formats as F
from oracle import gemm as GM
from oracle import offsets as O
from oracle import quantize as Q
from oracle import rht as R
import workloads
from gpu_util import bf16_out_to_f64, device, gemm_tolerance_check, host_u8

pytestmark = pytest.mark.gpu


def _sample_rows(off, rng, per_group=3):
    rows = []
    for g in range(len(off) - 1):
        a, b = int(off[g]), int(off[g + 1])
        if b > a:
            rows += [a, b - 1] + list(rng.integers(a, b, per_group))
    return np.unique(np.array(rows, dtype=np.int64))


def _check_fprop_case(name):
    dev = device()
    case = bench.make_case(name, dev)
    case.y.fill_(float("nan"))
    case.step()
    torch.cuda.synchronize()
    w = case.w
    G, N, K = w.G, w.n, w.k
    _, off = O.group_offsets(w.sizes)
    rng = np.random.default_rng(2024)
    rows = _sample_rows(off, rng)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 30)]))
    xb = workloads.bf16_bits(case.x[torch.from_numpy(rows).to(dev)])
    ad, asc = Q.mxfp8_rowwise(xb, np.array([0, len(rows)]))
    gx = host_u8(case.xr)[rows]
    gxs = host_u8(case.xrs)[:, rows, :]
    assert np.array_equal(gx, ad) and np.array_equal(gxs, asc), "activation quantize"
    grp = np.searchsorted(off, rows, side="right") - 1
    y = bf16_out_to_f64(case.y)
    wq, wqs = host_u8(case.wq), host_u8(case.wqs)
    for g in np.unique(grp):
        wrows = g * N + cols
        wb = workloads.bf16_bits(case.wt.view(G * N, K)[torch.from_numpy(wrows).to(dev)])
        bd, bsc = Q.mxfp8_rowwise(wb, np.array([0, len(cols)]))
        assert np.array_equal(wq[wrows], bd) and np.array_equal(wqs[:, wrows, :], bsc), \
            "weight quantize"
        sel = np.nonzero(grp == g)[0]
        ref = GM.mxfp8_fprop(ad[sel], asc[:, sel], bd.reshape(1, len(cols), K), bsc,
                             np.array([0, len(sel)]), K)
        gemm_tolerance_check(y[rows[sel]][:, cols], ref, False, "%s group %d" % (name, g))
    assert not np.isnan(y[:int(off[-1])]).any(), "every live output row written"
    return case, off


def test_full_fprop_headline():
    """8 experts, 16384 rows, K=4096, N=14336 (rowwise + columnwise X)."""
    case, off = _check_fprop_case("fprop")
    # the columnwise copy of the activations (used by the wgrad), on sampled columns
    w = case.w
    K = w.k
    _, poff = O.group_offsets(w.sizes, pad_to=128)
    c0 = 32 * 37
    xb = workloads.bf16_bits(case.x[:, c0:c0 + 32])
    cd, cs = Q.mxfp8_colwise(xb, off, poff)
    gd, gs = host_u8(case.xc), host_u8(case.xcs)
    for g in range(w.G):
        mp = int(poff[g + 1] - poff[g])
        if mp == 0:
            continue
        blk = gd[poff[g] * K:poff[g + 1] * K].reshape(K, mp)[c0:c0 + 32]
        want = cd[poff[g] * 32:poff[g + 1] * 32].reshape(32, mp)
        assert np.array_equal(blk, want), g
        sblk = gs[poff[g] * K // 32:poff[g + 1] * K // 32].reshape(mp // 128, K, 4)[:, c0:c0 + 32]
        swant = cs[poff[g]:poff[g + 1]].reshape(mp // 128, 32, 4)
        assert np.array_equal(sblk, swant), g


def test_full_zipf_64_experts():
    """64 experts (4 empty), 32768 Zipf-routed rows, K=7168, N=2048."""
    _check_fprop_case("zipf")


def test_full_tiny_all_outputs():
    dev = device()
    case = bench.make_case("tiny", dev)
    case.step()
    torch.cuda.synchronize()
    w = case.w
    G, N, K = w.G, w.n, w.k
    _, off = O.group_offsets(w.sizes)
    ad, asc = Q.mxfp8_rowwise(workloads.bf16_bits(case.x), off)
    bd, bsc = Q.mxfp8_rowwise(workloads.bf16_bits(case.wt).reshape(G * N, K), np.array([0, G * N]))
    ref = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    y = bf16_out_to_f64(case.y)
    for g in range(G):
        gemm_tolerance_check(y[off[g]:off[g + 1]], ref[off[g]:off[g + 1]], False, "group %d" % g)


@pytest.mark.parametrize("flow", ["wgrad", "wgrad_e5m2"])
def test_full_wgrad(flow):
    """8 experts (2 empty), 16384 ragged tokens, dW [8, 4096, 4096]; dY's
    columnwise copy in E4M3, or in E5M2 (wgrad_e5m2)."""
    dev = device()
    case = bench.make_case(flow, dev)
    elem = "e5m2" if flow == "wgrad_e5m2" else "e4m3"
    case.dw.fill_(float("nan"))
    case.step()
    torch.cuda.synchronize()
    w = case.w
    G, N, K = w.G, w.n, w.k
    _, off = O.group_offsets(w.sizes)
    _, poff = O.group_offsets(w.sizes, pad_to=128)
    rng = np.random.default_rng(7)
    i0, j0 = 32 * int(rng.integers(0, N // 32)), 32 * int(rng.integers(0, K // 32))
    dyb = workloads.bf16_bits(case.dy[:, i0:i0 + 32])
    xb = workloads.bf16_bits(case.x[:, j0:j0 + 32])
    dyc, dys = Q.mxfp8_colwise(dyb, off, poff, elem=elem)
    xc, xs = Q.mxfp8_colwise(xb, off, poff)
    ref = GM.mxfp8_wgrad(dyc, dys, xc, xs, poff, 32, 32, elem_a=elem)
    gd = host_u8(case.dyc)
    dw = case.dw
    for g in range(G):
        mp = int(poff[g + 1] - poff[g])
        if w.sizes[g] == 0:
            assert bool((dw[g] == 0).all()), "empty expert %d must get zeros" % g
            continue
        blk = gd[poff[g] * N:poff[g + 1] * N].reshape(N, mp)[i0:i0 + 32]
        assert np.array_equal(blk, dyc[poff[g] * 32:poff[g + 1] * 32].reshape(32, mp)), g
        y = dw[g, i0:i0 + 32, j0:j0 + 32].float().cpu().numpy().astype(np.float64)
        gemm_tolerance_check(y, ref[g], False, "%s group %d" % (flow, g))
    assert not torch.isnan(dw).any()


@pytest.mark.parametrize("flow", ["nvfp4", "nvfp4_scratch"])
def test_full_nvfp4_rowscaled(flow):
    """8 experts, 16384 live rows of 18432, K=4096, N_e in {2048, 4096}; fused
    outer-scale epilogue, and the FP32-scratch + post-scale flow."""
    dev = device()
    case = bench.make_case(flow, dev)
    case.y.fill_(float("nan"))
    case.step()
    torch.cuda.synchronize()
    w = case.w
    K, npg = w.k, case.npg
    _, off = O.group_offsets(w.sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    rng = np.random.default_rng(11)
    rows = _sample_rows(off, rng)
    xb = workloads.bf16_bits(case.x[torch.from_numpy(rows).to(dev)])
    ap, asc, at = Q.nvfp4_rowscaled(xb, np.array([0, len(rows)]))
    assert np.array_equal(host_u8(case.xd)[rows], ap)
    assert np.array_equal(host_u8(case.xs)[rows], asc)
    assert np.array_equal(case.xo.cpu().numpy()[rows].view(np.uint32), at.view(np.uint32))
    grp = np.searchsorted(off, rows, side="right") - 1
    y = bf16_out_to_f64(case.y)
    for g in np.unique(grp):
        cols = np.unique(np.concatenate([[0, npg[g] - 1], rng.integers(0, npg[g], 24)]))
        wrows = boff[g] + cols
        wb = workloads.bf16_bits(case.wt[torch.from_numpy(wrows).to(dev)])
        bp, bsc, bt = Q.nvfp4_rowscaled(wb, np.array([0, len(cols)]))
        assert np.array_equal(host_u8(case.wd)[wrows], bp)
        sel = np.nonzero(grp == g)[0]
        (_, ref), = GM.nvfp4_rowscaled_fprop(ap[sel], asc[sel], at[sel], np.array([0, len(sel)]),
                                             bp, bsc, bt, [len(cols)], K)
        gemm_tolerance_check(y[rows[sel]][:, cols], ref, False, "nvfp4 group %d" % g)
        if npg[g] < case.ld:
            assert np.isnan(y[rows[sel]][:, npg[g]:]).all(), "columns past N_g untouched"
    live = int(off[-1])
    assert np.isnan(y[live:]).all(), "capacity rows untouched"
    assert not np.isnan(y[:live, :min(npg)]).any()


def test_full_nvfp4_wgrad():
    """Row-scaled NVFP4 wgrad: 8 experts (2 empty), 16384 ragged tokens, dW
    [8, 4096, 4096]; a sampled 32 x 32 block of every expert's dW, and the
    columnwise copies of its 32 dY and 32 X columns."""
    dev = device()
    case = bench.make_case("nvfp4_wgrad", dev)
    case.dw.fill_(float("nan"))
    case.step()
    torch.cuda.synchronize()
    w = case.w
    G, N, K = w.G, w.n, w.k
    _, off = O.group_offsets(w.sizes)
    _, poff = O.group_offsets(w.sizes, pad_to=128)
    rng = np.random.default_rng(9)
    i0, j0 = 32 * int(rng.integers(0, N // 32)), 32 * int(rng.integers(0, K // 32))
    dyb = workloads.bf16_bits(case.dy[:, i0:i0 + 32])
    xb = workloads.bf16_bits(case.x[:, j0:j0 + 32])
    dyc, dys, dyo = Q.nvfp4_rowscaled_colwise(dyb, off, poff)
    xc, xs, xo = Q.nvfp4_rowscaled_colwise(xb, off, poff)
    ref = GM.nvfp4_rowscaled_wgrad(dyc, dys, dyo, xc, xs, xo, poff, 32, 32)
    gd, gs = host_u8(case.dyc), host_u8(case.dys)
    go = case.dyo.cpu().numpy()
    assert np.array_equal(go[:, i0:i0 + 32].view(np.uint32), dyo.view(np.uint32))
    assert np.array_equal(case.xo.cpu().numpy()[:, j0:j0 + 32].view(np.uint32), xo.view(np.uint32))
    dw = case.dw
    for g in range(G):
        mp = int(poff[g + 1] - poff[g])
        if w.sizes[g] == 0:
            assert bool((dw[g] == 0).all()), "empty expert %d must get zeros" % g
            continue
        blk = gd[poff[g] * N // 2:poff[g + 1] * N // 2].reshape(N, mp // 2)[i0:i0 + 32]
        assert np.array_equal(blk, dyc[poff[g] * 16:poff[g + 1] * 16].reshape(32, mp // 2)), g
        sblk = gs[poff[g] * N // 16:poff[g + 1] * N // 16].reshape(N, mp // 16)[i0:i0 + 32]
        assert np.array_equal(sblk, dys[poff[g] * 2:poff[g + 1] * 2].reshape(32, mp // 16)), g
        y = dw[g, i0:i0 + 32, j0:j0 + 32].float().cpu().numpy().astype(np.float64)
        gemm_tolerance_check(y, ref[g], False, "nvfp4 wgrad group %d" % g)
    assert not torch.isnan(dw).any()


def test_full_dgrad():
    """MoE dgrad at the fprop shapes: dX [16384, 4096] = dY [16384, 14336] (E5M2)
    x W_g [14336, 4096] (E4M3 columnwise copy); sampled rows of every expert
    and sampled columns, the E5M2 rows and the weights' columns checked
    bit-exact on the way."""
    dev = device()
    case = bench.make_case("dgrad", dev)
    case.dx.fill_(float("nan"))
    case.step()
    torch.cuda.synchronize()
    w = case.w
    G, N, K = w.G, w.n, w.k
    _, off = O.group_offsets(w.sizes)
    rng = np.random.default_rng(12)
    rows = _sample_rows(off, rng, per_group=2)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 14)]))
    dyb = workloads.bf16_bits(case.dy[torch.from_numpy(rows).to(dev)])
    ad, asc = Q.mxfp8_rowwise(dyb, np.array([0, len(rows)]), elem="e5m2")
    assert np.array_equal(host_u8(case.dyd)[rows], ad)
    assert np.array_equal(host_u8(case.dys)[:, rows, :], asc)
    grp = np.searchsorted(off, rows, side="right") - 1
    y = bf16_out_to_f64(case.dx)
    wcd, wcs = host_u8(case.wc), host_u8(case.wcs)
    nq = K // 128
    for g in np.unique(grp):
        wb = workloads.bf16_bits(case.wt[g][:, torch.from_numpy(cols).to(dev)])    # [K, len(cols)]
        bd, bs = Q.mxfp8_colwise(wb, np.array([0, K]), np.array([0, K]))
        blk = wcd[g * K * N:(g + 1) * K * N].reshape(N, K)[cols]
        assert np.array_equal(blk, bd.reshape(len(cols), K)), "weight copy, expert %d" % g
        sblk = wcs[g * K * N // 32:(g + 1) * K * N // 32].reshape(nq, N, 4)[:, cols, :]
        assert np.array_equal(sblk, bs.reshape(nq, len(cols), 4)), "weight scales, expert %d" % g
        sel = np.nonzero(grp == g)[0]
        ref = GM.mxfp8_dgrad(ad[sel], asc[:, sel], bd, bs, np.array([0, len(sel)]), K, len(cols))
        gemm_tolerance_check(y[rows[sel]][:, cols], ref, False, "dgrad group %d" % g)
    assert not np.isnan(y[:int(off[-1])]).any(), "every live output row written"


@pytest.mark.parametrize("flow", ["nvfp4_pertensor", "nvfp4_rht", "nvfp4_2d"])
def test_full_nvfp4_pertensor(flow):
    """Per-tensor NVFP4: 8 experts, 16384 live rows of 18432, K=4096, N_e in
    {2048, 4096}; each expert's activations and each expert's weight carry one
    amax.  The amax is checked against a plain max over the whole group (of
    the transformed rows with RHT); the sampled rows are quantized by the
    oracle together with one added row that holds the group's amax, so the
    oracle sees the same tensor scale.  "nvfp4_rht": both operands through the
    randomized Hadamard transform (same signs); "nvfp4_2d": weights with 16 x
    16 block scales, sampled by whole block rows."""
    dev = device()
    case = bench.make_case(flow, dev)
    case.y.fill_(float("nan"))
    case.step()
    torch.cuda.synchronize()
    w = case.w
    K, npg, G = w.k, case.npg, w.G
    _, off = O.group_offsets(w.sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    xa, wa = case.xa.cpu().numpy(), case.wa.cpu().numpy()
    rht = flow == "nvfp4_rht"
    mask = case.rht_mask

    def values(t, lo, hi):
        v = t[lo:hi].float()
        if rht:   # the transform of whole rows, in the oracle's float32 steps
            v = torch.from_numpy(R.rht16(v.cpu().numpy(), mask))
        return v

    def group_amax(t, lo, hi):
        if hi <= lo:
            return np.float32(0)
        return np.float32(values(t, lo, hi).abs().max().item())

    for g in range(G):
        assert xa[g] == group_amax(case.x, int(off[g]), int(off[g + 1])), g
        assert wa[g] == group_amax(case.wt, int(boff[g]), int(boff[g + 1])), g

    def quantize_sample(t, rows, amax):
        xb = workloads.bf16_bits(t[torch.from_numpy(rows).to(dev)])
        if rht:
            v = R.rht16(F.bf16_bits_to_f64(xb).astype(np.float32), mask)
            extra = np.zeros((1, K), np.float32)
            extra[0, 0] = amax
            p, s, a = Q.nvfp4_pertensor_values(np.concatenate([v, extra]),
                                               np.array([0, len(rows) + 1]))
        else:
            extra = np.zeros((1, K), np.float32)
            extra[0, 0] = amax
            xb = np.concatenate([xb, F.f32_to_bf16_bits_rne(extra)])
            p, s, a = Q.nvfp4_pertensor(xb, np.array([0, len(rows) + 1]))
        assert a[0] == amax
        return p[:-1], s[:-1]

    rng = np.random.default_rng(17)
    rows = _sample_rows(off, rng)
    grp = np.searchsorted(off, rows, side="right") - 1
    y = bf16_out_to_f64(case.y)
    gd, gs, gwd, gws = host_u8(case.xd), host_u8(case.xs), host_u8(case.wd), host_u8(case.ws)
    for g in np.unique(grp):
        sel = rows[grp == g]
        ap, asc = quantize_sample(case.x, sel, xa[g])
        assert np.array_equal(gd[sel], ap) and np.array_equal(gs[sel], asc)
        if flow == "nvfp4_2d":
            # two whole block rows of the expert's weight (16 output columns each)
            nbr = (npg[g] + 15) // 16
            brs = np.unique(np.array([0, nbr - 1, int(rng.integers(0, nbr))]))
            cols = np.concatenate([np.arange(16 * b, min(16 * b + 16, npg[g])) for b in brs])
            wrows = boff[g] + cols
            # the oracle's 2-D quantize of each sampled block row, after a block
            # row whose only nonzero is the expert's amax (so S is the expert's)
            pieces = []
            for b in brs:
                r = boff[g] + np.arange(16 * b, min(16 * b + 16, npg[g]))
                blk = F.bf16_bits_to_f64(workloads.bf16_bits(case.wt[torch.from_numpy(r).to(dev)]))
                pieces.append(blk)
            bp_list, bs_list = [], []
            for blk in pieces:
                v = blk.astype(np.float32)
                extra = np.zeros((16, K), np.float32)
                extra[0, 0] = wa[g]
                p, s, a = Q.nvfp4_pertensor_2d(
                    F.f32_to_bf16_bits_rne(np.concatenate([extra, v])), np.array([0, 16 + len(v)]))
                assert a[0] == wa[g]
                bp_list.append(p[16:])
                bs_list.append(s[16:])
            bp, bsc = np.concatenate(bp_list), np.concatenate(bs_list)
        else:
            cols = np.unique(np.concatenate([[0, npg[g] - 1], rng.integers(0, npg[g], 24)]))
            wrows = boff[g] + cols
            bp, bsc = quantize_sample(case.wt, wrows, wa[g])
        assert np.array_equal(gwd[wrows], bp) and np.array_equal(gws[wrows], bsc)
        one = np.array([0, len(sel)])
        aam, bam = np.array([xa[g]], np.float32), np.array([wa[g]], np.float32)
        (_, ref), = GM.nvfp4_pertensor_fprop(ap, asc, aam, one, bp, bsc, bam, [len(cols)], K)
        gemm_tolerance_check(y[sel][:, cols], ref, False, "%s group %d" % (flow, g))
        if npg[g] < case.ld:
            assert np.isnan(y[sel][:, npg[g]:]).all(), "columns past N_g untouched"
    live = int(off[-1])
    assert np.isnan(y[live:]).all(), "capacity rows untouched"
    assert not np.isnan(y[:live, :min(npg)]).any()
