"""Grouped GEMMs as per-expert dense products of dequantized operands, in fp64
(oracle; test infrastructure only).

The grouped GEMM equals, group by group, a dense GEMM of the dequantized
operands: the pure-JAX fallback ("gemm.py", ``_jax_scaled_matmul``: TN, data
(B, M, K) x (B, N, K) with scales (B, M, K/block)) and the parity tests of
"[Common][PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM"
(per-expert dense GEMM over byte-identical operands) define it that way.
Each product of two decoded elements is exact in fp64 and the K-sums carry
only fp64 rounding, far below the GEMM tolerance.
"""

import numpy as np

from .quantize import mxfp8_dequant_rows, nvfp4_block_dequant, mx_scale_words, MX_BLOCK


def _group_of_rows(offsets, rows):
    off = np.asarray(offsets, dtype=np.int64)
    return np.searchsorted(off, np.asarray(rows), side="right") - 1


def mxfp8_fprop(a_data, a_scales, b_data, b_scales, offsets, k, rows=None):
    """FPROP (TN, ragged rows; "gemm.py", ``grouped_gemm`` with lhs first dims
    ragged, rhs [G, N, K]):
        Y[r, n] = sum_k dq(A)[r, k] * dq(B)[g, n, k]  for r in [off[g], off[g+1]).

    a_data [R_a, k] with scales [NQ, R_a, 4] (rowwise, R_a >= live rows);
    b_data [G, N, k] with scales [NQ, G * N, 4] (the weights quantized as G * N
    rows).  ``rows`` (optional) selects live rows to compute; default all live
    rows.  Returns float64 [len(rows), N]."""
    off = np.asarray(offsets, dtype=np.int64)
    G, N = b_data.shape[0], b_data.shape[1]
    nq = mx_scale_words(k)
    if rows is None:
        rows = np.arange(int(off[-1]))
    rows = np.asarray(rows, dtype=np.int64)
    a_data = np.asarray(a_data).reshape(-1, k)
    a_scales = np.asarray(a_scales).reshape(nq, -1, 4)
    b_scales = np.asarray(b_scales).reshape(nq, G * N, 4)
    out = np.zeros((len(rows), N), dtype=np.float64)
    grp = _group_of_rows(off, rows)
    for g in range(G):
        sel = np.nonzero(grp == g)[0]
        if len(sel) == 0:
            continue
        dqa = mxfp8_dequant_rows(a_data[rows[sel]], a_scales[:, rows[sel], :], k)
        dqb = mxfp8_dequant_rows(np.asarray(b_data[g]).reshape(N, k),
                                 b_scales[:, g * N:(g + 1) * N, :], k)
        out[sel] = dqa @ dqb.T
    return out


def mxfp8_wgrad(dy_col, dy_col_scales, x_col, x_col_scales, padded_offsets, n, k, groups=None,
                out_rows=None, elem_a="e4m3"):
    """WGRAD (NT, ragged contraction; "gemm.py", ``grouped_gemm`` with rhs first
    dims ragged, uniform (G, ...) output):
        dW[g, i, j] = sum_{t < m_g} dq(dY)[off[g] + t, i] * dq(X)[off[g] + t, j]
    with dY's elements E4M3, or E5M2 (``elem_a``; an E5M2 gradient times E4M3
    activations, a pairing ``_compatible_fp8_gemm_dtypes`` accepts)

    taken from the columnwise copies (group g: dY^T block [n, m~_g], X^T block
    [k, m~_g], zero padding beyond m_g; scales [m~_g/128, n or k, 4] words).  An empty group gives dW[g] = 0.
    ``groups`` / ``out_rows`` optionally restrict the computed groups / rows i.
    Returns float64 [len(groups), len(out_rows), k]."""
    poff = np.asarray(padded_offsets, dtype=np.int64)
    G = len(poff) - 1
    groups = list(range(G)) if groups is None else list(groups)
    out_rows = np.arange(n) if out_rows is None else np.asarray(out_rows, dtype=np.int64)
    out = np.zeros((len(groups), len(out_rows), k), dtype=np.float64)
    for gi, g in enumerate(groups):
        mp = int(poff[g + 1] - poff[g])
        if mp == 0:
            continue
        nq = mx_scale_words(mp)
        a = np.asarray(dy_col[poff[g] * n:poff[g + 1] * n]).reshape(n, mp)[out_rows]
        a_s = np.asarray(dy_col_scales[poff[g] * n // MX_BLOCK:poff[g + 1] * n // MX_BLOCK]
                         ).reshape(nq, n, 4)[:, out_rows, :]
        b = np.asarray(x_col[poff[g] * k:poff[g + 1] * k]).reshape(k, mp)
        b_s = np.asarray(x_col_scales[poff[g] * k // MX_BLOCK:poff[g + 1] * k // MX_BLOCK]
                         ).reshape(nq, k, 4)
        out[gi] = mxfp8_dequant_rows(a, a_s, mp, elem=elem_a) @ mxfp8_dequant_rows(b, b_s, mp).T
    return out


def nvfp4_rowscaled_fprop(a_packed, a_bscales, a_tsi, offsets, b_packed, b_bscales, b_tsi,
                          n_per_group, k, rows=None):
    """Row-scaled NVFP4 FPROP ("[Common][PyTorch] Add row-scaled NVFP4 support to
    grouped-tensor GEMM": the outer scales are neutralized in the GEMM, the
    product goes to an FP32 scratch, and the outer scales are applied afterwards
    over each group's own rows and columns):
        S[r, n] = sum_k (e2m1(A) * sd_A)[r, k] * (e2m1(B_g) * sd_B)[n, k]
        Y[r, n] = S[r, n] * tsi_A[r] * tsi_B_g[n]   for live r in g, n < N_g.

    B holds the experts' [N_g, k] weights one after another (rows
    sum(N_g)); b_tsi is indexed the same way.  Returns a list, per group, of
    (row indices, float64 [len(rows in g), N_g])."""
    off = np.asarray(offsets, dtype=np.int64)
    npg = [int(v) for v in n_per_group]
    boff = np.concatenate([[0], np.cumsum(npg)]).astype(np.int64)
    if rows is None:
        rows = np.arange(int(off[-1]))
    rows = np.asarray(rows, dtype=np.int64)
    grp = _group_of_rows(off, rows)
    a_packed = np.asarray(a_packed).reshape(-1, k // 2)
    a_bscales = np.asarray(a_bscales).reshape(-1, k // 16)
    b_packed = np.asarray(b_packed).reshape(-1, k // 2)
    b_bscales = np.asarray(b_bscales).reshape(-1, k // 16)
    result = []
    for g in range(len(npg)):
        sel = rows[grp == g]
        if len(sel) == 0 or npg[g] == 0:
            result.append((sel, np.zeros((len(sel), npg[g]))))
            continue
        a = nvfp4_block_dequant(a_packed[sel], a_bscales[sel], k)
        b = nvfp4_block_dequant(b_packed[boff[g]:boff[g + 1]], b_bscales[boff[g]:boff[g + 1]], k)
        s = a @ b.T
        y = s * np.asarray(a_tsi, np.float64)[sel][:, None] * \
            np.asarray(b_tsi, np.float64)[boff[g]:boff[g + 1]][None, :]
        result.append((sel, y))
    return result


def nvfp4_pertensor_fprop(a_packed, a_bscales, a_amax, offsets, b_packed, b_bscales, b_amax,
                          n_per_group, k, rows=None):
    """Per-tensor NVFP4 FPROP over groups ("gemm.py": for NVFP4 operands the
    GEMM's alpha is the product of the two operands' tensor scales
    ``_get_nvfp4_tensor_scale_inv(amax)``, and the product is scaled by it; the
    graph-safe grouped GEMM takes one alpha per group):
        S[r, n] = sum_k (e2m1(A) * sd_A)[r, k] * (e2m1(B_g) * sd_B)[n, k]
        alpha_g = float32(tsi(amax_A[g]) * tsi(amax_B[g]))
        Y[r, n] = alpha_g * S[r, n]      for live r in g, n < N_g.

    B holds the experts' [N_g, k] weights one after another, each expert one
    tensor with its amax b_amax[g].  Returns a list, per group, of (row
    indices, float64 [len(rows in g), N_g])."""
    from .quantize import nvfp4_tensor_scale_inv
    off = np.asarray(offsets, dtype=np.int64)
    npg = [int(v) for v in n_per_group]
    boff = np.concatenate([[0], np.cumsum(npg)]).astype(np.int64)
    if rows is None:
        rows = np.arange(int(off[-1]))
    rows = np.asarray(rows, dtype=np.int64)
    grp = _group_of_rows(off, rows)
    a_packed = np.asarray(a_packed).reshape(-1, k // 2)
    a_bscales = np.asarray(a_bscales).reshape(-1, k // 16)
    b_packed = np.asarray(b_packed).reshape(-1, k // 2)
    b_bscales = np.asarray(b_bscales).reshape(-1, k // 16)
    alpha = np.float32(nvfp4_tensor_scale_inv(a_amax)) * np.float32(nvfp4_tensor_scale_inv(b_amax))
    alpha = np.asarray(alpha, dtype=np.float32)
    result = []
    for g in range(len(npg)):
        sel = rows[grp == g]
        if len(sel) == 0 or npg[g] == 0:
            result.append((sel, np.zeros((len(sel), npg[g]))))
            continue
        a = nvfp4_block_dequant(a_packed[sel], a_bscales[sel], k)
        b = nvfp4_block_dequant(b_packed[boff[g]:boff[g + 1]], b_bscales[boff[g]:boff[g + 1]], k)
        result.append((sel, float(alpha[g]) * (a @ b.T)))
    return result


def nvfp4_rowscaled_wgrad(dy_col, dy_bscales, dy_outer, x_col, x_bscales, x_outer,
                          padded_offsets, n, k, groups=None, out_rows=None):
    """Row-scaled NVFP4 WGRAD (NT, contraction over each expert's ragged
    tokens), from the columnwise copies of ``quantize.nvfp4_rowscaled_colwise``
    ("[Common][PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM":
    the outer scales are neutralized in the GEMM and applied afterwards per
    expert -- the discrete-out wgrad path -- over each expert's own rows and
    columns):
        S[g, i, j]  = sum_{t < m~_g} (e2m1 * sd)(dY^T_g)[i, t] * (e2m1 * sd)(X^T_g)[j, t]
        dW[g, i, j] = S[g, i, j] * tsi_dY[g, i] * tsi_X[g, j]
    Padding tokens encode to zero, so the sum over m~_g equals the sum over the
    expert's m_g tokens; an empty expert gives dW[g] = 0.  ``groups`` /
    ``out_rows`` optionally restrict the computed experts / rows i.  Returns
    float64 [len(groups), len(out_rows), k]."""
    poff = np.asarray(padded_offsets, dtype=np.int64)
    G = len(poff) - 1
    groups = list(range(G)) if groups is None else list(groups)
    out_rows = np.arange(n) if out_rows is None else np.asarray(out_rows, dtype=np.int64)
    dy_outer = np.asarray(dy_outer, dtype=np.float64).reshape(G, n)
    x_outer = np.asarray(x_outer, dtype=np.float64).reshape(G, k)
    out = np.zeros((len(groups), len(out_rows), k), dtype=np.float64)
    for gi, g in enumerate(groups):
        mp = int(poff[g + 1] - poff[g])
        if mp == 0:
            continue
        a = np.asarray(dy_col[poff[g] * n // 2:poff[g + 1] * n // 2]).reshape(n, mp // 2)[out_rows]
        a_s = np.asarray(dy_bscales[poff[g] * n // 16:poff[g + 1] * n // 16]
                         ).reshape(n, mp // 16)[out_rows]
        b = np.asarray(x_col[poff[g] * k // 2:poff[g + 1] * k // 2]).reshape(k, mp // 2)
        b_s = np.asarray(x_bscales[poff[g] * k // 16:poff[g + 1] * k // 16]).reshape(k, mp // 16)
        s = nvfp4_block_dequant(a, a_s, mp) @ nvfp4_block_dequant(b, b_s, mp).T
        out[gi] = s * dy_outer[g][out_rows][:, None] * x_outer[g][None, :]
    return out


def mxfp8_dgrad(dy_data, dy_scales, wt_data, wt_scales, offsets, n, k, rows=None):
    """MoE DGRAD (NN, "gemm.py", ``grouped_gemm``; E5M2 gradient times E4M3
    weight, a pairing ``_compatible_fp8_gemm_dtypes`` accepts):
        dX[r, j] = sum_{i < n} dq_E5M2(dY)[r, i] * dq_E4M3(W_g)[i, j]
    for rows r of expert g.  dY is the rowwise E5M2 quantize of the
    [rows, n] gradient (``quantize.mxfp8_rowwise(..., elem="e5m2")``); W is
    taken from its columnwise copy (``quantize.mxfp8_colwise`` of the
    [G * n, k] weights with expert offsets g * n and padded offsets g * n~,
    n~ = n rounded up to a multiple of 128: every columnwise copy pads a group's
    tokens to a multiple of 128), i.e. per expert the transposed [k, n~] block
    quantized along n (zero padding past n), with [n~ / 128, k, 4] scale words.
    ``rows`` optionally restricts the output rows.  Returns float64 [len(rows), k]."""
    off = np.asarray(offsets, dtype=np.int64)
    G = len(off) - 1
    if rows is None:
        rows = np.arange(int(off[-1]))
    rows = np.asarray(rows, dtype=np.int64)
    grp = _group_of_rows(off, rows)
    nq = mx_scale_words(n)
    npad = 4 * MX_BLOCK * nq          # the expert's padded token count n~
    dy_data = np.asarray(dy_data).reshape(-1, n)
    dy_scales = np.asarray(dy_scales).reshape(nq, -1, 4)
    out = np.zeros((len(rows), k), dtype=np.float64)
    for g in range(G):
        sel = np.nonzero(grp == g)[0]
        if len(sel) == 0:
            continue
        a = mxfp8_dequant_rows(dy_data[rows[sel]], dy_scales[:, rows[sel], :], n, elem="e5m2")
        wt = np.asarray(wt_data[g * npad * k:(g + 1) * npad * k]).reshape(k, npad)
        ws = np.asarray(wt_scales[g * npad * k // MX_BLOCK:(g + 1) * npad * k // MX_BLOCK]
                        ).reshape(nq, k, 4)
        out[sel] = a @ mxfp8_dequant_rows(wt, ws, npad)[:, :n].T
    return out


def epilogue(s, groups, alpha=None, beta=None, c_old=None, bias=None):
    """Per-group epilogue of the grouped GEMM ("gemm.py", ``grouped_gemm``: bias
    of shape (num_gemms, N) over the output columns; the graph-safe grouped
    primitive's per-group float32 alpha and beta, defaults 1 and 0; "[Common]
    [PyTorch] Add row-scaled NVFP4 support to grouped-tensor GEMM": copy or
    accumulate into the output):
        Y[r, j] = alpha[g] * S[r, j] + beta[g] * C[r, j] + bias[g, j]
    with g the group of output row r (``groups``, one entry per row of S), C
    the output's previous contents, read only where beta[g] != 0.  Reading:
    the three terms are combined before the single rounding to the output
    type.  Returns float64 like S."""
    s = np.asarray(s, dtype=np.float64)
    g = np.asarray(groups, dtype=np.int64)
    a = 1.0 if alpha is None else np.asarray(alpha, dtype=np.float64)[g][:, None]
    y = a * s
    if beta is not None:
        b = np.asarray(beta, dtype=np.float64)[g]
        if np.any(b != 0):
            c = np.asarray(c_old, dtype=np.float64)
            y = y + np.where(b[:, None] != 0, b[:, None] * np.where(b[:, None] != 0, c, 0.0), 0.0)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)[g]
    return y
