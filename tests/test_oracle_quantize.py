"""Pins of the oracle's offsets, layouts and grouped quantizers (CPU only).

The grouped quantizers are checked against a per-element pure-Python
re-derivation on tiny inputs (its own table search and its own block walk, no
shared helpers), against the concatenation of per-expert calls, and against the
invariants the pages state (sum of sizes vs rows)."""

import math
import os

import numpy as np
import pytest

from oracle import formats as F
from oracle import layout as L
from oracle import offsets as O
from oracle import quantize as Q
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- offsets

def test_offsets_formula_and_pad():
    sizes = np.array([32, 0, 64, 32], np.int32)
    s64, off = O.group_offsets(sizes)
    assert list(off) == [0, 32, 32, 96, 128] and list(s64) == [32, 0, 64, 32]
    s64, off = O.group_offsets(np.array([2049, 0, 3001, 1], np.int32), pad_to=128)
    assert list(off) == [0, 2176, 2176, 2176 + 3072, 2176 + 3072 + 128]
    s64, off = O.group_offsets(np.array([3, 5], np.int32), multiplier=4096)
    assert list(s64) == [3 * 4096, 5 * 4096] and list(off) == [0, 3 * 4096, 8 * 4096]
    with pytest.raises(ValueError):
        O.group_offsets(np.array([1, -1], np.int32))


@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
def test_workload_size_invariants(name):
    w = workloads.get(name)
    _, off = O.group_offsets(w.sizes)
    assert off[-1] == np.sum(w.sizes.astype(np.int64))
    assert O.check_capacity(off, w.rows_cap)
    if name in ("tiny", "fprop", "wgrad", "zipf", "nvfp4_wgrad", "dgrad"):
        assert off[-1] == w.rows_cap
    else:
        assert off[-1] < w.rows_cap
    if name in ("fprop", "dgrad"):
        assert np.all(w.sizes % 128 == 0) and len(set(w.sizes.tolist())) > 1
    if name in ("wgrad", "nvfp4_wgrad"):
        assert np.sum(w.sizes == 0) == 2 and np.all(w.sizes[w.sizes > 0] % 32 != 0)
    if name == "zipf":
        assert np.sum(w.sizes == 0) >= 4 and w.G == 64


# ---------------------------------------------------------------- layout

def test_mx_scale_order_hand_example_and_inverse():
    logical = np.array([[10, 11, 12, 13, 14, 15]], np.uint8)
    stored = L.mx_scales_to_gemm_order(logical)
    assert stored.reshape(-1).tolist() == [10, 12, 11, 13, 14, 0, 15, 0]
    # two rows, two 128-element groups: words ordered group-major, then row
    two = np.array([[1, 2, 3, 4, 5, 6, 7, 8], [11, 12, 13, 14, 15, 16, 17, 18]], np.uint8)
    assert L.mx_scales_to_gemm_order(two).reshape(-1).tolist() == \
        [1, 3, 2, 4, 11, 13, 12, 14, 5, 7, 6, 8, 15, 17, 16, 18]
    rng = np.random.default_rng(0)
    for nb in (1, 3, 4, 7, 8, 128):
        lg = rng.integers(0, 255, (5, nb)).astype(np.uint8)
        assert np.array_equal(L.mx_scales_from_gemm_order(L.mx_scales_to_gemm_order(lg), nb), lg)


def test_fp4_pack_order():
    codes = np.array([[1, 2, 3, 4]], np.uint8)
    assert L.fp4_pack(codes).tolist() == [[0x21, 0x43]]
    assert np.array_equal(L.fp4_unpack(L.fp4_pack(codes)), codes)


# ---------------------------------------------------------------- brute-force re-derivation

_E4M3_TABLE = None


def _e4m3_table():
    global _E4M3_TABLE
    if _E4M3_TABLE is None:
        vals = []
        for code in range(0x7F):
            e, m = code >> 3, code & 7
            vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
        _E4M3_TABLE = vals
    return _E4M3_TABLE


def _slow_e4m3(v):
    a = abs(v)
    best = (math.inf, 0)
    for code, g in enumerate(_e4m3_table()):
        d = abs(a - g)
        if d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | (0x80 if math.copysign(1.0, v) < 0 else 0)


def _slow_scale_byte(block):
    amax = max(abs(v) for v in block)
    if amax == 0:
        return 0
    e = math.floor(math.log2(amax))
    while 2.0 ** e > amax:
        e -= 1
    while 2.0 ** (e + 1) <= amax:
        e += 1
    return min(max(e - 8 + 127, 0), 254)


def _slow_mx_block(block):
    b = _slow_scale_byte(block)
    return b, [_slow_e4m3(v / 2.0 ** (b - 127)) for v in block]


def _tiny_bits(rng, rows, cols):
    x = (rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-3, 4, (rows, 1)))).astype(np.float32)
    x[rng.random((rows, cols)) < 0.02] *= 40
    x[0, :32] = 0.0
    return F.f32_to_bf16_bits_rne(x)


def test_rowwise_matches_slow_rederivation():
    rng = np.random.default_rng(11)
    bits = _tiny_bits(rng, 9, 160)              # 5 blocks per row (a short scale group)
    xv = F.bf16_bits_to_f64(bits)
    off = np.array([0, 3, 3, 7])                # 7 live rows of 9
    data, scales = Q.mxfp8_rowwise(bits, off)
    assert data.shape == (7, 160) and scales.shape == (2, 7, 4)
    for r in range(7):
        logical = []
        for blk in range(5):
            b, codes = _slow_mx_block(list(xv[r, blk * 32:(blk + 1) * 32]))
            logical.append(b)
            assert list(data[r, blk * 32:(blk + 1) * 32]) == codes
        stored = [logical[0], logical[2], logical[1], logical[3], logical[4], 0, 0, 0]
        assert list(scales[:, r, :].reshape(-1)) == stored


def test_colwise_matches_slow_rederivation():
    rng = np.random.default_rng(12)
    sizes = np.array([37, 0, 130, 5], np.int32)
    bits = _tiny_bits(rng, 200, 64)
    xv = F.bf16_bits_to_f64(bits)
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    data, scales = Q.mxfp8_colwise(bits, off, poff)
    C = 64
    assert len(data) == poff[-1] * C and len(scales) == poff[-1] * C // 32
    for g in range(4):
        m, mp = int(sizes[g]), int(poff[g + 1] - poff[g])
        blk_data = data[poff[g] * C:poff[g + 1] * C].reshape(C, mp)
        blk_sc = scales[poff[g] * C // 32:poff[g + 1] * C // 32].reshape(mp // 128, C, 4)
        for c in range(0, C, 7):
            col = [xv[off[g] + t, c] if t < m else 0.0 for t in range(mp)]
            logical = []
            for b in range(mp // 32):
                sb, codes = _slow_mx_block(col[b * 32:(b + 1) * 32])
                logical.append(sb)
                assert list(blk_data[c, b * 32:(b + 1) * 32]) == codes, (g, c, b)
            want = []
            for q in range(0, len(logical), 4):
                grp = logical[q:q + 4]
                want += [grp[0], grp[2], grp[1], grp[3]]
            assert list(blk_sc[:, c, :].reshape(-1)) == want
        assert np.all(blk_data[:, m:] == 0)


def test_grouped_equals_per_expert_concatenation():
    rng = np.random.default_rng(13)
    sizes = np.array([40, 0, 90, 7], np.int32)
    bits = _tiny_bits(rng, 150, 96)
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    d_all, s_all = Q.mxfp8_rowwise(bits, off)
    cd_all, cs_all = Q.mxfp8_colwise(bits, off, poff)
    n_all, ns_all, nt_all = Q.nvfp4_rowscaled(bits, off)
    for g in range(4):
        part = bits[off[g]:off[g + 1]]
        one = np.array([0, sizes[g]])
        d, s = Q.mxfp8_rowwise(part, one)
        assert np.array_equal(d, d_all[off[g]:off[g + 1]])
        assert np.array_equal(s, s_all[:, off[g]:off[g + 1]])
        _, p1 = O.group_offsets(sizes[g:g + 1], pad_to=128)
        cd, cs = Q.mxfp8_colwise(part, one, p1)
        assert np.array_equal(cd, cd_all[poff[g] * 96:poff[g + 1] * 96])
        assert np.array_equal(cs, cs_all[poff[g] * 96 // 32:poff[g + 1] * 96 // 32])
        n, ns, nt = Q.nvfp4_rowscaled(part, one)
        assert np.array_equal(n, n_all[off[g]:off[g + 1]])
        assert np.array_equal(ns, ns_all[off[g]:off[g + 1]])
        assert np.array_equal(nt, nt_all[off[g]:off[g + 1]])


def test_capacity_rows_not_read():
    rng = np.random.default_rng(14)
    bits = _tiny_bits(rng, 10, 64)
    bits[6:] = workloads.BF16_NAN_BITS
    d, s = Q.mxfp8_rowwise(bits, np.array([0, 2, 6]))
    assert d.shape[0] == 6
    n, ns, nt = Q.nvfp4_rowscaled(bits, np.array([0, 6]))
    assert n.shape[0] == 6 and np.all(np.isfinite(nt))
    with pytest.raises(ValueError):
        Q.mxfp8_rowwise(bits, np.array([0, 11]))


def _slow_e2m1(v):
    grid = [0, .5, 1, 1.5, 2, 3, 4, 6]
    a = abs(v)
    best = (math.inf, 0)
    for code, g in enumerate(grid):
        d = abs(a - g)
        if d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | (8 if math.copysign(1.0, v) < 0 else 0)


def test_nvfp4_matches_slow_rederivation():
    rng = np.random.default_rng(15)
    bits = _tiny_bits(rng, 6, 64)
    xv = F.bf16_bits_to_f64(bits)
    packed, s8, tsi = Q.nvfp4_rowscaled(bits, np.array([0, 6]))
    f = np.float32
    for r in range(6):
        amax = f(max(abs(v) for v in xv[r]))
        S = f(f(2688) / amax) if amax > 0 else f(1)
        assert tsi[r] == f(amax / f(2688))
        for b in range(4):
            blk = xv[r, b * 16:(b + 1) * 16]
            bmax = f(max(abs(v) for v in blk))
            sf = f(f(bmax / f(6)) * S)
            code8 = _slow_e4m3(float(sf))
            assert s8[r, b] == code8
            sd = f(_e4m3_table()[code8 & 0x7F])
            enc = f(S / sd) if sd != 0 else f(0)
            for i in range(16):
                j = b * 16 + i
                q = _slow_e2m1(float(f(f(blk[i]) * enc)))
                got = (packed[r, j // 2] >> (4 * (j % 2))) & 0xF
                assert got == q, (r, j)


def test_nvfp4_colwise_golden_per_expert_columns():
    """tests/golden/nvfp4_cols.txt: each expert's columns get their own outer
    scale, blocks run along the expert's tokens, padding encodes to zero."""
    lines = [ln.split("#")[0].split() for ln in open(os.path.join(GOLDEN, "nvfp4_cols.txt"))]
    lines = [ln for ln in lines if ln]
    sizes = np.array([3, 2], np.int32)
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    x = np.zeros((5, 32), np.float32)
    for g, c, vals, *_ in lines:
        v = [float(t) for t in vals.split(",")]
        x[off[int(g)]:off[int(g)] + len(v), int(c)] = v
    data, bsc, outer = Q.nvfp4_rowscaled_colwise(F.f32_to_bf16_bits_rne(x), off, poff)
    assert data.shape == (256 * 32 // 2,) and bsc.shape == (256 * 32 // 16,)
    assert outer.shape == (2, 32) and np.all(outer[:, 2:] == 0)
    for g, c, vals, amax, s8, packed in lines:
        g, c = int(g), int(c)
        blk = data[poff[g] * 32 // 2:poff[g + 1] * 32 // 2].reshape(32, 64)
        sc = bsc[poff[g] * 32 // 16:poff[g + 1] * 32 // 16].reshape(32, 8)
        assert outer[g, c] == np.float32(np.float32(amax) / np.float32(2688))
        assert sc[c, 0] == int(s8, 16) and np.all(sc[c, 1:] == 0)
        want = [int(b, 16) for b in packed.split(",")]
        assert list(blk[c, :len(want)]) == want
        assert np.all(blk[c, len(want):] == 0)
    # the all-zero columns: scale 0, codes 0
    for g in range(2):
        blk = data[poff[g] * 32 // 2:poff[g + 1] * 32 // 2].reshape(32, 64)
        assert np.all(blk[2:] == 0)


def test_nvfp4_colwise_dequant_within_format_error():
    """Invariant: e2m1 * block scale * outer scale reproduces every live token
    of every column within NVFP4's error (half an E2M1 step of the block scale
    times the outer scale, plus the E4M3 rounding of the scale), and an empty
    expert writes nothing."""
    rng = np.random.default_rng(31)
    sizes = np.array([40, 0, 17, 128], np.int32)
    M, C = int(sizes.sum()), 64
    x = rng.standard_normal((M, C)).astype(np.float32) * np.exp(rng.uniform(-3, 3, (1, C)))
    xb = F.f32_to_bf16_bits_rne(x)
    xv = F.bf16_bits_to_f64(xb)
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    data, bsc, outer = Q.nvfp4_rowscaled_colwise(xb, off, poff)
    assert np.all(outer[1] == 0)
    for g in (0, 2, 3):
        m, mp = int(sizes[g]), int(poff[g + 1] - poff[g])
        blk = data[poff[g] * C // 2:poff[g + 1] * C // 2].reshape(C, mp // 2)
        sc = bsc[poff[g] * C // 16:poff[g + 1] * C // 16].reshape(C, mp // 16)
        dq = Q.nvfp4_dequant(blk, sc, outer[g], mp)
        ref = xv[off[g]:off[g + 1]].T
        assert np.all(dq[:, m:] == 0)
        amax = np.abs(ref).max(axis=1)
        assert np.allclose(outer[g], (amax / 2688).astype(np.float32), rtol=1e-7, atol=0)
        # per block: |err| <= 0.25 * 2 (E2M1 step at 6 is 2, half of it 1; scaled
        # by sd * tsi ~ bmax / 6) -> |err| <= bmax / 6 plus 1/16 relative scale error
        for b in range((m + 15) // 16):
            seg = slice(16 * b, min(16 * b + 16, m))
            bmax = np.abs(ref[:, seg]).max(axis=1, keepdims=True)
            assert np.all(np.abs(dq[:, seg] - ref[:, seg]) <= bmax / 6 * 1.07 + 1e-30)


# ---------------------------------------------------------------- per-tensor NVFP4

def test_nvfp4_pertensor_golden():
    """tests/golden/nvfp4_pertensor.txt: every row of a group takes the group's
    amax (a row whose own amax is smaller gets a smaller block scale than the
    row-scaled cast would give it), an empty group has amax 0."""
    lines = [ln.split("#")[0].split() for ln in open(os.path.join(GOLDEN, "nvfp4_pertensor.txt"))]
    lines = [ln for ln in lines if ln]
    sizes = np.array([2, 1, 0, 1], np.int32)
    _, off = O.group_offsets(sizes)
    x = np.zeros((4, 32), np.float32)
    for r, (g, vals, *_rest) in enumerate(lines):
        v = [float(t) for t in vals.split(",")]
        x[r, :len(v)] = v
    packed, s8, amax = Q.nvfp4_pertensor(F.f32_to_bf16_bits_rne(x), off)
    assert packed.shape == (4, 16) and s8.shape == (4, 2) and amax.shape == (4,)
    assert amax[2] == 0.0
    for r, (g, vals, am, sc, pk) in enumerate(lines):
        assert amax[int(g)] == np.float32(float(am))
        assert s8[r, 0] == int(sc, 16) and s8[r, 1] == 0
        want = [int(b, 16) for b in pk.split(",")]
        assert list(packed[r, :len(want)]) == want and np.all(packed[r, len(want):] == 0)
    assert Q.nvfp4_tensor_scale_inv(amax)[0] == np.float32(np.float32(6) / np.float32(2688))


def test_nvfp4_pertensor_matches_slow_rederivation():
    rng = np.random.default_rng(17)
    bits = _tiny_bits(rng, 7, 64)
    xv = F.bf16_bits_to_f64(bits)
    off = np.array([0, 3, 3, 7])
    packed, s8, amax = Q.nvfp4_pertensor(bits, off)
    f = np.float32
    for g in range(3):
        rows = range(off[g], off[g + 1])
        am = f(max((abs(v) for r in rows for v in xv[r]), default=0.0))
        assert amax[g] == am
        S = f(f(2688) / am) if am > 0 else f(1)
        for r in rows:
            for b in range(4):
                blk = xv[r, b * 16:(b + 1) * 16]
                sf = f(f(f(max(abs(v) for v in blk)) / f(6)) * S)
                code8 = _slow_e4m3(float(sf))
                assert s8[r, b] == code8
                sd = f(_e4m3_table()[code8 & 0x7F])
                enc = f(S / sd) if sd != 0 else f(0)
                for i in range(16):
                    j = b * 16 + i
                    q = _slow_e2m1(float(f(f(blk[i]) * enc)))
                    assert (packed[r, j // 2] >> (4 * (j % 2))) & 0xF == q, (r, j)


def test_nvfp4_pertensor_equals_rowscaled_when_rows_share_amax():
    """Special case: when every row of a group reaches the group's amax, the
    per-tensor cast is the row-scaled cast (same bytes, tsi_g = tsi_r)."""
    rng = np.random.default_rng(19)
    x = rng.standard_normal((9, 96)).astype(np.float32)
    x[:4, 5] = 7.5
    x[4:, 40] = -0.3125 * 64
    xb = F.f32_to_bf16_bits_rne(x)
    off = np.array([0, 4, 4, 9])
    p1, s1, amax = Q.nvfp4_pertensor(xb, off)
    p2, s2, tsi = Q.nvfp4_rowscaled(xb, off)
    assert np.array_equal(p1, p2) and np.array_equal(s1, s2)
    tsi_g = Q.nvfp4_tensor_scale_inv(amax)
    assert np.all(tsi[:4] == tsi_g[0]) and np.all(tsi[4:] == tsi_g[2]) and amax[1] == 0


def test_nvfp4_pertensor_grouped_equals_per_expert_concatenation():
    rng = np.random.default_rng(23)
    bits = _tiny_bits(rng, 11, 128)
    sizes = np.array([4, 0, 6, 1], np.int32)
    _, off = O.group_offsets(sizes)
    p_all, s_all, a_all = Q.nvfp4_pertensor(bits, off)
    for g in range(4):
        part = bits[off[g]:off[g + 1]]
        p, s, a = Q.nvfp4_pertensor(part, np.array([0, sizes[g]]))
        assert np.array_equal(p, p_all[off[g]:off[g + 1]])
        assert np.array_equal(s, s_all[off[g]:off[g + 1]])
        assert a[0] == a_all[g]


# ---------------------------------------------------------------- properties over random groupings

from hypothesis import given, settings, strategies as st  # noqa: E402


@settings(max_examples=25, deadline=None)
@given(sizes=st.lists(st.integers(0, 150), min_size=1, max_size=5),
       cq=st.integers(1, 3), seed=st.integers(0, 2 ** 31 - 1))
def test_colwise_grouped_equals_per_expert_property(sizes, cq, seed):
    """The grouped columnwise copy is, byte for byte, the concatenation of each
    expert quantized alone (blocks restart at every expert's first token,
    padding to 128 tokens encodes to zero), for any token split."""
    rng = np.random.default_rng(seed)
    sizes = np.array(sizes, np.int32)
    C = 32 * cq
    bits = _tiny_bits(rng, max(int(sizes.sum()), 1), C)
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    data, scales = Q.mxfp8_colwise(bits, off, poff)
    for g in range(len(sizes)):
        m = int(sizes[g])
        d1, s1 = Q.mxfp8_colwise(bits[off[g]:off[g + 1]].reshape(m, C), np.array([0, m]),
                                 O.group_offsets(np.array([m], np.int32), pad_to=128)[1])
        assert np.array_equal(data[poff[g] * C:poff[g + 1] * C], d1)
        assert np.array_equal(scales[poff[g] * C // 32:poff[g + 1] * C // 32], s1)


@settings(max_examples=25, deadline=None)
@given(sizes=st.lists(st.integers(0, 40), min_size=1, max_size=6),
       cq=st.integers(1, 4), seed=st.integers(0, 2 ** 31 - 1))
def test_nvfp4_pertensor_grouped_equals_per_expert_property(sizes, cq, seed):
    rng = np.random.default_rng(seed)
    sizes = np.array(sizes, np.int32)
    C = 32 * cq
    bits = _tiny_bits(rng, max(int(sizes.sum()), 1), C)
    _, off = O.group_offsets(sizes)
    p_all, s_all, a_all = Q.nvfp4_pertensor(bits, off)
    for g in range(len(sizes)):
        p, s, a = Q.nvfp4_pertensor(bits[off[g]:off[g + 1]], np.array([0, sizes[g]]))
        assert np.array_equal(p, p_all[off[g]:off[g + 1]])
        assert np.array_equal(s, s_all[off[g]:off[g + 1]])
        assert a[0] == a_all[g]
