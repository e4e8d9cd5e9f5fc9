"""Pins of the oracle's grouped GEMMs (CPU only).

* exact integer arithmetic: inputs whose quantization is lossless (small
  integers), so every grouped product must equal the integer per-expert
  product of the raw inputs -- this catches a wrong group, a transposed
  operand, a wrong contraction range or a dropped padding rule;
* correctly rounded sums (math.fsum over exact fp64 products) of the test's
  own decode of the stored bytes;
* grouped == per-expert calls on slices.
"""

import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import gemm as GM
from oracle import offsets as O
from oracle import quantize as Q
import workloads


def _int_bits(rng, shape, lo=-3, hi=3):
    v = rng.integers(lo, hi + 1, shape).astype(np.float32)
    return F.f32_to_bf16_bits_rne(v), v.astype(np.int64)


def test_fprop_exact_on_lossless_inputs():
    rng = np.random.default_rng(21)
    sizes = np.array([32, 0, 64, 32], np.int32)
    K, N, G = 128, 48, 4
    xb, xi = _int_bits(rng, (128, K))
    wb, wi = _int_bits(rng, (G * N, K))
    _, off = O.group_offsets(sizes)
    ad, asc = Q.mxfp8_rowwise(xb, off)
    bd, bsc = Q.mxfp8_rowwise(wb, np.array([0, G * N]))
    y = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    for g in range(G):
        want = xi[off[g]:off[g + 1]] @ wi[g * N:(g + 1) * N].T
        assert np.array_equal(y[off[g]:off[g + 1]], want.astype(np.float64))


@pytest.mark.parametrize("elem", ["e4m3", "e5m2"])
def test_wgrad_exact_on_lossless_inputs(elem):
    """Small integers are exact in E4M3 and E5M2 under any MX scale: dW must be
    the exact per-expert integer product, whichever element format dY uses."""
    rng = np.random.default_rng(22)
    sizes = np.array([37, 0, 130, 5], np.int32)
    M, N, K = int(sizes.sum()), 40, 64
    dyb, dyi = _int_bits(rng, (M, N))
    xb, xi = _int_bits(rng, (M, K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    dyc, dys = Q.mxfp8_colwise(dyb, off, poff, elem=elem)
    xc, xs = Q.mxfp8_colwise(xb, off, poff)
    dw = GM.mxfp8_wgrad(dyc, dys, xc, xs, poff, N, K, elem_a=elem)
    for g in range(4):
        want = dyi[off[g]:off[g + 1]].T @ xi[off[g]:off[g + 1]]
        assert np.array_equal(dw[g], want.astype(np.float64)), g
    assert np.all(dw[1] == 0)


def _decode_rows_fsum_check(data, stored, k):
    """The test's own decode: bit fields -> value, scale order undone by hand."""
    rows = data.shape[0]
    vals = np.zeros((rows, k))
    for r in range(rows):
        logical = []
        for q in range(stored.shape[0]):          # word (q, r): b0, b2, b1, b3
            s0, s2, s1, s3 = stored[q, r]
            logical += [s0, s1, s2, s3]
        for j in range(k):
            c = int(data[r, j])
            e, m = (c >> 3) & 15, c & 7
            v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
            if c & 0x80:
                v = -v
            vals[r, j] = v * 2.0 ** (int(logical[j // 32]) - 127)
    return vals


def test_fprop_fsum_on_tiny_config():
    w = workloads.get("tiny")
    t = workloads.tensors(w)
    xb, wb = workloads.bf16_bits(t["x"]), workloads.bf16_bits(t["w"])
    K, N, G = w.k, w.n, w.G
    _, off = O.group_offsets(w.sizes)
    ad, asc = Q.mxfp8_rowwise(xb, off)
    bd, bsc = Q.mxfp8_rowwise(wb.reshape(G * N, K), np.array([0, G * N]))
    y = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    a = _decode_rows_fsum_check(ad, asc, K)
    b = _decode_rows_fsum_check(bd, bsc, K)
    for r in range(0, 128, 5):
        g = int(np.searchsorted(off, r, side="right") - 1)
        for n in range(0, N, 3):
            ref = math.fsum(a[r] * b[g * N + n])
            assert abs(y[r, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_grouped_equals_per_expert_gemm():
    rng = np.random.default_rng(23)
    sizes = np.array([10, 0, 33, 21], np.int32)
    K, N, G = 96, 24, 4
    xb = F.f32_to_bf16_bits_rne(rng.standard_normal((64, K)).astype(np.float32))
    wb = F.f32_to_bf16_bits_rne(rng.standard_normal((G * N, K)).astype(np.float32))
    _, off = O.group_offsets(sizes)
    ad, asc = Q.mxfp8_rowwise(xb, off)
    bd, bsc = Q.mxfp8_rowwise(wb, np.array([0, G * N]))
    bd = bd.reshape(G, N, K)
    y = GM.mxfp8_fprop(ad, asc, bd, bsc, off, K)
    for g in range(G):
        one = GM.mxfp8_fprop(ad[off[g]:off[g + 1]], asc[:, off[g]:off[g + 1]], bd[g:g + 1],
                             bsc[:, g * N:(g + 1) * N], np.array([0, sizes[g]]), K)
        assert np.array_equal(y[off[g]:off[g + 1]], one)
    sub = GM.mxfp8_fprop(ad, asc, bd, bsc, off, K, rows=np.array([5, 40, 63]))
    assert np.array_equal(sub, y[[5, 40, 63]])


@pytest.mark.parametrize("K", [64, 32, 96])
def test_nvfp4_exact_on_lossless_inputs_and_widths(K):
    """Values on the E2M1 grid with row max 6: S = 448, every block scale 448,
    enc = 1, so the codes are the values; Y must equal the integer product times
    the two outer scales, per group over its own N_g columns (K = 32 and 96 end
    in half a 64-element step)."""
    rng = np.random.default_rng(24 + K)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6])
    sizes = np.array([3, 0, 5], np.int32)
    npg = [8, 16, 24]

    def mk(rows):
        v = rng.choice(grid, (rows, K))
        v[:, ::16] = 6.0                  # every block's max is 6
        return F.f32_to_bf16_bits_rne(v.astype(np.float32)), v

    xb, xv = mk(int(sizes.sum()) + 2)     # 2 capacity rows
    wb, wv = mk(sum(npg))
    _, off = O.group_offsets(sizes)
    ap, asc, at = Q.nvfp4_rowscaled(xb, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(wb, np.array([0, sum(npg)]))
    assert np.all(asc == 0x7E) and np.all(bsc == 0x7E)
    res = GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)
    boff = np.concatenate([[0], np.cumsum(npg)])
    for g in range(3):
        rows, y = res[g]
        assert list(rows) == list(range(off[g], off[g + 1]))
        assert y.shape == (sizes[g], npg[g])
        if sizes[g] == 0:
            continue
        exact = (xv[rows] @ wv[boff[g]:boff[g + 1]].T) * 448.0 * 448.0
        want = exact * at[rows].astype(np.float64)[:, None] * bt[boff[g]:boff[g + 1]].astype(np.float64)
        assert np.allclose(y, want, rtol=1e-14, atol=0)
        # and this is the raw product within float32 rounding of the outer scales
        assert np.allclose(y, xv[rows] @ wv[boff[g]:boff[g + 1]].T, rtol=1e-6, atol=1e-9)


def test_nvfp4_wgrad_exact_on_lossless_inputs():
    """Values on the E2M1 grid times a per-column power of two 2^-e_c, with a
    +-6 * 2^-e_c in every 16-token block of every column of every expert: then
    S = 448 * 2^e_c, every block scale is 448, enc = 2^e_c and the codes are the
    grid values, so quantization is lossless and dW must equal the exact
    per-expert product of the raw inputs.  The per-column powers make every
    column's outer scale different (an outer scale taken by the wrong index, or
    a transposed operand, fails); the experts' token counts are not multiples of
    16 (padding must encode to zero) and one expert is empty (dW = 0)."""
    rng = np.random.default_rng(25)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -.5, -1, -1.5, -2, -3, -4, -6])
    sizes = np.array([21, 0, 40, 3], np.int32)
    M, N, K = int(sizes.sum()), 32, 64
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)

    def mk(cols):
        v = rng.choice(grid, (M, cols))
        for g in range(len(sizes)):
            v[off[g]:off[g + 1]:16] = rng.choice([6.0, -6.0], v[off[g]:off[g + 1]:16].shape)
        v = v * 2.0 ** -rng.integers(0, 6, (1, cols))
        return F.f32_to_bf16_bits_rne(v.astype(np.float32)), v

    dyb, dyv = mk(N)
    xb, xv = mk(K)
    dyc, dys, dyo = Q.nvfp4_rowscaled_colwise(dyb, off, poff)
    xc, xs, xo = Q.nvfp4_rowscaled_colwise(xb, off, poff)
    for g in (0, 2, 3):
        m = int(sizes[g])
        ns = dys[poff[g] * N // 16:poff[g + 1] * N // 16].reshape(N, -1)[:, :(m + 15) // 16]
        assert np.all(ns == 0x7E)
    assert len(set(np.round(np.log2(dyo[0] * 2688 / 6)))) > 1
    dw = GM.nvfp4_rowscaled_wgrad(dyc, dys, dyo, xc, xs, xo, poff, N, K)
    for g in range(len(sizes)):
        want = dyv[off[g]:off[g + 1]].T @ xv[off[g]:off[g + 1]]
        # the outer scales are float32 roundings of amax / 2688
        assert np.allclose(dw[g], want, rtol=2e-7, atol=0), g
    assert np.all(dw[1] == 0)
    # exact once the float32 outer scales are divided back out
    g = 2
    s = dw[g] / dyo[g].astype(np.float64)[:, None] / xo[g].astype(np.float64)[None, :]
    exact = (dyv[off[g]:off[g + 1]].T @ xv[off[g]:off[g + 1]]) * 448.0 * 448.0 * \
        (6.0 / (np.abs(dyv[off[g]:off[g + 1]]).max(axis=0)))[:, None] * \
        (6.0 / (np.abs(xv[off[g]:off[g + 1]]).max(axis=0)))[None, :]
    assert np.allclose(s, exact, rtol=1e-12, atol=0)
    # restricted evaluation agrees with the full one
    part = GM.nvfp4_rowscaled_wgrad(dyc, dys, dyo, xc, xs, xo, poff, N, K, groups=[3, 0],
                                    out_rows=[5, 1])
    assert np.array_equal(part[0], dw[3][[5, 1]]) and np.array_equal(part[1], dw[0][[5, 1]])


@pytest.mark.parametrize("N,K", [(256, 96), (160, 64), (32, 96)])
def test_dgrad_exact_on_lossless_inputs(N, K):
    """dY and W small integers: lossless in E5M2 (dY) and E4M3 (W) under any MX
    scale, so dX must equal the exact per-expert integer product dY_g @ W_g.
    n != k catches a transposed W copy; an empty expert and uneven row counts
    catch a wrong group range; a contraction n that is not a multiple of 128
    uses the columnwise copy whose experts are padded to 128 tokens (a wrong
    expert stride or a padding read as data fails)."""
    rng = np.random.default_rng(26 + N)
    sizes = np.array([9, 0, 40, 3], np.int32)
    G, M = len(sizes), int(sizes.sum())
    npad = -(-N // 128) * 128
    dyb, dyi = _int_bits(rng, (M, N))
    wb, wi = _int_bits(rng, (G * N, K))
    _, off = O.group_offsets(sizes)
    dyd, dys = Q.mxfp8_rowwise(dyb, off, elem="e5m2")
    woff = np.arange(G + 1, dtype=np.int64) * N
    wtd, wts = Q.mxfp8_colwise(wb, woff, np.arange(G + 1, dtype=np.int64) * npad)
    dx = GM.mxfp8_dgrad(dyd, dys, wtd, wts, off, N, K)
    for g in range(G):
        want = dyi[off[g]:off[g + 1]] @ wi[g * N:(g + 1) * N]
        assert np.array_equal(dx[off[g]:off[g + 1]], want.astype(np.float64)), g
    part = GM.mxfp8_dgrad(dyd, dys, wtd, wts, off, N, K, rows=[50, 0])
    assert np.array_equal(part, dx[[50, 0]])


def test_dgrad_e5m2_rounding_is_visible():
    """Non-integer gradients: E5M2 keeps 2 mantissa bits, so dX differs from the
    bf16 product by the E5M2 rounding, within the format's relative error 2^-3
    per element (bounded per row by sum |dy_i w_ij| * 2^-3 plus the weights'
    E4M3 error 2^-4)."""
    rng = np.random.default_rng(27)
    sizes = np.array([64], np.int32)
    N, K = 128, 32
    dy = rng.standard_normal((64, N)).astype(np.float32)
    w = rng.standard_normal((N, K)).astype(np.float32)
    dyb, wb = F.f32_to_bf16_bits_rne(dy), F.f32_to_bf16_bits_rne(w)
    _, off = O.group_offsets(sizes)
    dyd, dys = Q.mxfp8_rowwise(dyb, off, elem="e5m2")
    woff = np.array([0, N])
    wtd, wts = Q.mxfp8_colwise(wb, woff, woff)
    dx = GM.mxfp8_dgrad(dyd, dys, wtd, wts, off, N, K)
    dyv, wv = F.bf16_bits_to_f64(dyb), F.bf16_bits_to_f64(wb)
    exact = dyv @ wv
    bound = np.abs(dyv) @ np.abs(wv) * (2.0 ** -3 + 2.0 ** -4 + 2.0 ** -7)
    assert np.all(np.abs(dx - exact) <= bound)
    assert np.abs(dx - exact).max() > 0          # the gradient really is E5M2


def test_wgrad_e5m2_rounding_is_visible():
    """The E5M2 wgrad equals the product of dY's E5M2 codes decoded by their
    bit fields (sign, 5 exponent bits with bias 15, 2 mantissa bits) times the
    block scales read from the words by hand, and differs from the E4M3 wgrad
    (values with more significant bits than E5M2 keeps)."""
    rng = np.random.default_rng(27)
    sizes = np.array([64, 40], np.int32)
    M, N, K = int(sizes.sum()), 32, 32
    dyb = F.f32_to_bf16_bits_rne(rng.standard_normal((M, N)).astype(np.float32))
    xb, xi = _int_bits(rng, (M, K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    c5, s5 = Q.mxfp8_colwise(dyb, off, poff, elem="e5m2")
    c4, s4 = Q.mxfp8_colwise(dyb, off, poff)
    xc, xs = Q.mxfp8_colwise(xb, off, poff)
    dw5 = GM.mxfp8_wgrad(c5, s5, xc, xs, poff, N, K, elem_a="e5m2")
    dw4 = GM.mxfp8_wgrad(c4, s4, xc, xs, poff, N, K)
    for g in range(2):
        mp = int(poff[g + 1] - poff[g])
        codes = c5[poff[g] * N:poff[g + 1] * N].reshape(N, mp)
        words = s5[poff[g] * N // 32:poff[g + 1] * N // 32].reshape(mp // 128, N, 4)
        dq = np.zeros((N, mp))
        for c in range(N):
            for t in range(mp):
                code = int(codes[c, t])
                e, m = (code >> 2) & 31, code & 3
                v = m / 4 * 2.0 ** -14 if e == 0 else (1 + m / 4) * 2.0 ** (e - 15)
                if code & 0x80:
                    v = -v
                blk = t // 32
                stored = words[blk // 4, c]              # bytes b0, b2, b1, b3
                byte = int(stored[[0, 2, 1, 3].index(blk % 4)])
                dq[c, t] = v * 2.0 ** (byte - 127)
        want = dq[:, :sizes[g]] @ xi[off[g]:off[g + 1]]
        assert np.allclose(dw5[g], want, rtol=1e-12, atol=0), g
        assert not np.allclose(dw5[g], dw4[g])


def test_epilogue_exact_on_lossless_inputs():
    """alpha, beta and bias values that are exact in fp64 and distinct per
    group, on lossless integer operands: the fprop output must equal
    alpha_g * (X_g W_g^T) + beta_g * C + bias_g exactly, row by row in its own
    group; beta = 0 must not read C (NaN there stays out of the result)."""
    rng = np.random.default_rng(28)
    sizes = np.array([5, 0, 9], np.int32)
    G, M, N, K = 3, 14, 40, 128
    xb, xi = _int_bits(rng, (M, K))
    wb, wi = _int_bits(rng, (G * N, K))
    _, off = O.group_offsets(sizes)
    ad, asc = Q.mxfp8_rowwise(xb, off)
    bd, bsc = Q.mxfp8_rowwise(wb, np.array([0, G * N]))
    s = GM.mxfp8_fprop(ad, asc, bd.reshape(G, N, K), bsc, off, K)
    grp = np.searchsorted(off, np.arange(M), side="right") - 1
    alpha = np.array([0.5, 3.0, -2.0])
    beta = np.array([1.0, 0.0, 0.0])
    c = rng.integers(-9, 10, (M, N)).astype(np.float64)
    c[grp == 2] = np.nan                       # beta 0: never read
    bias = rng.integers(-4, 5, (G, N)).astype(np.float64) * 0.25
    y = GM.epilogue(s, grp, alpha, beta, c, bias)
    for r in range(M):
        g = grp[r]
        want = alpha[g] * (xi[r] @ wi[g * N:(g + 1) * N].T) + bias[g]
        if beta[g] != 0:
            want = want + beta[g] * c[r]
        assert np.array_equal(y[r], want), r
    # the defaults are the plain product
    assert np.array_equal(GM.epilogue(s, grp), s)


def test_nvfp4_pertensor_exact_on_lossless_inputs():
    """Per-tensor NVFP4 on lossless operands: every 16-block holds E2M1 grid
    values times 2^j with a block maximum of exactly 6 * 2^j, and each group's
    (expert's) largest block reaches 2688 * 2^p, so tsi = 2^p, every scale is a
    power of two (or 448) and the codes reproduce the inputs exactly.  Y must
    then equal the exact per-expert product of the raw inputs, over each
    group's own N_g columns."""
    rng = np.random.default_rng(26)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, -.5, -1, -1.5, -2, -3, -4])
    sizes = np.array([3, 0, 5, 2], np.int32)
    npg = [8, 16, 24, 8]
    K = 64

    def mk(group_rows, p):
        v = rng.choice(grid, (group_rows, K))
        j = rng.integers(-6, 3, (group_rows, K // 16))
        v[:, ::16] = rng.choice([6.0, -6.0], (group_rows, K // 16))   # block max 6 * 2^j
        v = v * np.exp2(np.repeat(j, 16, axis=1))
        v[0, 16:32] *= 448 / 2.0 ** j[0, 1]          # one block at 2688: tsi = 1 before 2^p
        return v * 2.0 ** p

    xs = [mk(int(m), p) for m, p in zip(sizes, [-3, 0, 4, 1]) if m > 0]
    xv = np.concatenate(xs + [np.zeros((2, K))])             # 2 capacity rows
    wv = np.concatenate([mk(n, p) for n, p in zip(npg, [0, -2, 1, 3])])
    _, off = O.group_offsets(sizes)
    boff = np.concatenate([[0], np.cumsum(npg)])
    xb, wb = F.f32_to_bf16_bits_rne(xv.astype(np.float32)), F.f32_to_bf16_bits_rne(wv.astype(np.float32))
    assert np.array_equal(F.bf16_bits_to_f64(xb), xv) and np.array_equal(F.bf16_bits_to_f64(wb), wv)
    ap, asc, aam = Q.nvfp4_pertensor(xb, off)
    bp, bsc, bam = Q.nvfp4_pertensor(wb, boff)
    for g, p in zip((0, 2, 3), (-3, 4, 1)):
        assert Q.nvfp4_tensor_scale_inv(aam)[g] == 2.0 ** p
    # lossless: dequant reproduces the inputs
    dq = Q.nvfp4_dequant(ap, asc, Q.nvfp4_tensor_scale_inv(aam)[np.repeat(np.arange(4), sizes)], K)
    assert np.array_equal(dq, xv[:off[-1]])
    res = GM.nvfp4_pertensor_fprop(ap, asc, aam, off, bp, bsc, bam, npg, K)
    for g in range(4):
        rows, y = res[g]
        assert list(rows) == list(range(off[g], off[g + 1]))
        assert y.shape == (sizes[g], npg[g])
        if sizes[g]:
            assert np.array_equal(y, xv[rows] @ wv[boff[g]:boff[g + 1]].T)


# ---------------------------------------------------------------- properties over random shapes

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=30, deadline=None)
@given(sizes=st.lists(st.integers(0, 70), min_size=1, max_size=6),
       kq=st.integers(1, 8), n=st.integers(1, 40), spare=st.integers(0, 5),
       seed=st.integers(0, 2 ** 31 - 1))
def test_fprop_lossless_property(sizes, kq, n, spare, seed):
    """Any ragged grouping (empty groups, capacity rows past the live ones),
    any K that is a multiple of 32: on small-integer operands, which every MX
    block holds exactly, the grouped fprop equals the exact per-expert integer
    product."""
    rng = np.random.default_rng(seed)
    sizes = np.array(sizes, np.int32)
    G, K, rows = len(sizes), 32 * kq, int(sizes.sum()) + spare
    xb, xi = _int_bits(rng, (rows, K))
    wb, wi = _int_bits(rng, (G * n, K))
    _, off = O.group_offsets(sizes)
    ad, asc = Q.mxfp8_rowwise(xb, off)
    bd, bsc = Q.mxfp8_rowwise(wb, np.array([0, G * n]))
    y = GM.mxfp8_fprop(ad, asc, bd.reshape(G, n, K), bsc, off, K)
    for g in range(G):
        want = xi[off[g]:off[g + 1]] @ wi[g * n:(g + 1) * n].T
        assert np.array_equal(y[off[g]:off[g + 1]], want.astype(np.float64))


@settings(max_examples=20, deadline=None)
@given(sizes=st.lists(st.integers(0, 200), min_size=1, max_size=5),
       nq=st.integers(1, 3), kq=st.integers(1, 3), seed=st.integers(0, 2 ** 31 - 1))
def test_wgrad_lossless_property(sizes, nq, kq, seed):
    """Any ragged token split (sizes not multiples of 32, empty experts): the
    columnwise copies padded per expert to 128 tokens give dW[g] = dY_g^T X_g
    exactly on small-integer operands, and exact zeros for an empty expert."""
    rng = np.random.default_rng(seed)
    sizes = np.array(sizes, np.int32)
    G, N, K, M = len(sizes), 32 * nq, 32 * kq, int(sizes.sum())
    dyb, dyi = _int_bits(rng, (M, N))
    xb, xi = _int_bits(rng, (M, K))
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    dyc, dys = Q.mxfp8_colwise(dyb, off, poff)
    xc, xs = Q.mxfp8_colwise(xb, off, poff)
    dw = GM.mxfp8_wgrad(dyc, dys, xc, xs, poff, N, K)
    for g in range(G):
        want = dyi[off[g]:off[g + 1]].T @ xi[off[g]:off[g + 1]]
        assert np.array_equal(dw[g], want.astype(np.float64)), g
