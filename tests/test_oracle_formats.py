"""Pins of the oracle's codecs against hand-worked vectors, an independent
library cast (torch CPU float8), brute-force nearest-grid search, and closed
forms.  CPU only."""

import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quantize as Q

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _val(tok):
    tok = tok.strip()
    if "*2^" in tok:
        m, e = tok.split("*2^")
        return math.ldexp(float(m), int(e))
    return float(tok)


def _rows(name):
    out = []
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            out.append(line.split())
    return out


# ---------------------------------------------------------------- hand-worked vectors

def test_mx_hand_blocks():
    rows = _rows("mxfp8_blocks.txt")
    assert len(rows) >= 15
    for amax_s, val_s, sb_s, code_s in rows:
        amax, val = _val(amax_s), _val(val_s)
        block = np.zeros(32)
        block[0] = amax
        block[1] = val
        if val_s.startswith("-") and val == 0.0:
            block[1] = -0.0
        bits = F.f32_to_bf16_bits_rne(block.astype(np.float32))
        assert np.array_equal(F.bf16_bits_to_f64(bits), block), "fixture value not bf16-exact"
        data, scales = Q.mxfp8_rowwise(bits.reshape(1, 32), np.array([0, 1]))
        assert scales[0, 0, 0] == int(sb_s, 16), (amax_s, val_s)
        assert data[0, 1] == int(code_s, 16), (amax_s, val_s, hex(data[0, 1]))


def test_e2m1_hand_values():
    rows = _rows("e2m1_values.txt")
    vals = np.array([_val(r[0]) for r in rows])
    want = np.array([int(r[1], 16) for r in rows], dtype=np.uint8)
    assert np.array_equal(F.e2m1_encode(vals), want)


def test_nvfp4_hand_rows():
    for amax_s, vals_s, s8_s, codes_s in _rows("nvfp4_rows.txt"):
        amax = _val(amax_s)
        row = np.zeros(32)
        row[16:16 + 1] = amax          # the amax lives in the second block
        vals = [_val(v) for v in vals_s.split(",")]
        row[:len(vals)] = vals
        if amax == 0.0:
            row[:] = 0.0
        bits = F.f32_to_bf16_bits_rne(row.astype(np.float32)).reshape(1, 32)
        packed, s8, tsi = Q.nvfp4_rowscaled(bits, np.array([0, 1]))
        codes = np.zeros(32, dtype=np.uint8)
        codes[0::2] = packed[0] & 0xF
        codes[1::2] = packed[0] >> 4
        assert s8[0, 0] == int(s8_s, 16), (amax_s, vals_s, hex(s8[0, 0]))
        want = [int(c, 16) for c in codes_s.split(",")]
        assert list(codes[:len(want)]) == want, (vals_s, codes[:len(want)])
        assert np.float32(tsi[0]) == np.float32(np.float32(amax) / np.float32(2688.0))
    # the first fixture's first packed byte
    row = np.zeros(32, np.float32)
    row[:5] = [6, 3, 1.5, 0.75, -5]
    packed, _, _ = Q.nvfp4_rowscaled(F.f32_to_bf16_bits_rne(row).reshape(1, 32), np.array([0, 1]))
    assert packed[0, 0] == 0x57


# ---------------------------------------------------------------- independent library casts

def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_bits_to_f64(bits)
    return v[np.isfinite(v)]


def test_e4m3_matches_torch_cast_all_bf16_times_all_scales():
    """Every finite bf16 value divided by every E8M0 scale, clamped to +-448,
    against torch's float8_e4m3fn cast (round to nearest even)."""
    x = _all_finite_bf16()
    for byte in range(0, 255, 1):
        v = x / F.e8m0_decode(byte)
        clamped = np.clip(v, -448.0, 448.0)
        ours = F.e4m3_encode(clamped)
        ref = torch.from_numpy(clamped.astype(np.float32)).to(torch.float8_e4m3fn)
        ref = ref.view(torch.uint8).numpy()
        # float32 conversion of tiny values may lose the sign of zero only for exact zeros
        assert np.array_equal(ours, ref), byte
        # saturation: the unclamped encoder gives the same codes
        assert np.array_equal(F.e4m3_encode(v), ours)


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = F.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e8m0_decode_matches_torch():
    b = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(F.e8m0_decode(b), ref)


# ---------------------------------------------------------------- brute force

def _nearest_code_bruteforce(values, table):
    """Nearest grid value by exhaustive search over a code table (codes ordered by
    magnitude), ties to the even code; saturate beyond the table."""
    out = []
    for v in values:
        a = abs(v)
        best = None
        for code, g in enumerate(table):
            d = abs(a - g)
            if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
                best = (d, code)
        out.append(best[1])
    return np.array(out)


def test_e4m3_bruteforce_near_grid_points():
    table = [float(F.e4m3_decode(c)) for c in range(0x7F)]
    pts = []
    for i, g in enumerate(table):
        for cand in [g] + ([0.5 * (g + table[i + 1])] if i + 1 < len(table) else []):
            f = np.float32(cand)
            pts.append(float(f))
            lo = hi = f
            for _ in range(3):
                lo = np.nextafter(lo, np.float32(-1))
                hi = np.nextafter(hi, np.float32(1e30))
                pts.extend([float(lo), float(hi)])
    pts = np.array([p for p in pts if p >= 0.0] + [450.0, 463.9, 464.0, 470.0, 1e6])
    want = _nearest_code_bruteforce(pts, table)
    got = F.e4m3_encode(pts)
    assert np.array_equal(got, want)
    assert np.array_equal(F.e4m3_encode(-pts), want | 0x80)


def test_e2m1_bruteforce():
    table = [0, .5, 1, 1.5, 2, 3, 4, 6]
    rng = np.random.default_rng(5)
    pts = np.concatenate([rng.uniform(0, 8, 20000).astype(np.float32).astype(np.float64),
                          np.arange(0, 7.01, 0.125)])
    want = _nearest_code_bruteforce(pts, table)
    assert np.array_equal(F.e2m1_encode(pts), want)
    assert np.array_equal(F.e2m1_decode(want), np.minimum(
        np.array([table[c] for c in want]), 6.0))


# ---------------------------------------------------------------- closed forms / invariants

def test_e8m0_closed_form_bracket():
    rng = np.random.default_rng(1)
    amax = np.abs(rng.standard_normal(100000)) * np.exp2(rng.integers(-60, 60, 100000))
    amax = F.bf16_bits_to_f64(F.f32_to_bf16_bits_rne(amax.astype(np.float32)))
    amax = amax[amax > 0]
    b = F.e8m0_from_amax(amax).astype(np.int64)
    s = np.ldexp(1.0, b - 127)
    assert np.all(amax >= 256 * s) and np.all(amax < 512 * s)


def test_mx_roundtrip_bound_and_block_max_code():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    x[3, :40] = 0.0
    bits = F.f32_to_bf16_bits_rne(x)
    xv = F.bf16_bits_to_f64(bits)
    data, scales = Q.mxfp8_rowwise(bits, np.array([0, 64]))
    dq = Q.mxfp8_dequant_rows(data, scales, 256)
    from oracle.layout import mx_scales_from_gemm_order
    sb = mx_scales_from_gemm_order(scales, 8).astype(np.int64)
    s = np.repeat(np.ldexp(1.0, sb - 127), 32, axis=1)
    v = np.abs(xv) / s
    # |v| <= 448: error at most half an E4M3 step at v's binade; above: saturated to 448
    e = np.maximum(np.floor(np.log2(np.maximum(v, 1e-300))), -6)
    step = np.exp2(e - 3)
    inrange = v <= 448
    assert np.all(np.abs(xv - dq)[inrange] <= (0.5 * step * s)[inrange])
    assert np.all(np.abs(dq[~inrange]) == (448 * s)[~inrange])
    # every nonzero block's largest code magnitude lies in 0x78..0x7E
    mags = (data & 0x7F).reshape(64, 8, 32).max(axis=2)
    nz = np.abs(xv).reshape(64, 8, 32).max(axis=2) > 0
    assert np.all((mags[nz] >= 0x78) & (mags[nz] <= 0x7E))
    assert np.all(sb[~nz] == 0)


def test_nvfp4_encode_bound():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((32, 128)) * np.exp2(rng.integers(-10, 10, (32, 1)))).astype(np.float32)
    bits = F.f32_to_bf16_bits_rne(x)
    xv = F.bf16_bits_to_f64(bits)
    packed, s8, tsi = Q.nvfp4_rowscaled(bits, np.array([0, 32]))
    amax = np.abs(xv).max(axis=1)
    assert np.array_equal(tsi, (amax.astype(np.float32) / np.float32(2688)).astype(np.float32))
    dq_inner = Q.nvfp4_block_dequant(packed, s8, 128)
    # the encoded magnitudes x*enc lie within the E2M1 rounding bound of q
    S = np.float32(2688) / amax.astype(np.float32)
    sd = F.e4m3_decode(s8)
    enc = (S[:, None].astype(np.float32) / sd.astype(np.float32)).astype(np.float32)
    xe = (xv.reshape(32, 8, 16).astype(np.float32) * enc[..., None]).astype(np.float64)
    q = dq_inner.reshape(32, 8, 16) / sd[..., None]
    a = np.abs(xe)
    bound = np.where(a < 2, 0.25, np.where(a < 4, 0.5, np.where(a <= 6, 1.0, a - 6)))
    assert np.all(np.abs(np.abs(q) - a) <= bound + 1e-12)
    # relative reconstruction error of the block maximum stays within the E4M3 + E2M1 steps
    dq = dq_inner * tsi[:, None].astype(np.float64)
    assert np.max(np.abs(dq - xv)) <= 0.25 * np.max(np.abs(xv))


def test_e5m2_hand_values():
    """E5M2: bias 15, 2 mantissa bits, subnormal step 2^-16, largest 57344."""
    cases = [(1.0, 0x3C), (57344.0, 0x7B), (2.0 ** -16, 0x01), (2.0 ** -14, 0x04),
             (1.25, 0x3D), (1.375, 0x3E),      # the tie 1.375 goes to the even mantissa (1.5)
             (1.125, 0x3C), (-3.0, 0xC2), (61440.0, 0x7B), (1e9, 0x7B),   # saturation
             (0.0, 0x00), (-0.0, 0x80), (3 * 2.0 ** -17, 0x02)]           # 1.5 steps -> 2 (even)
    for v, code in cases:
        assert int(F.e5m2_encode(np.array([v]))[0]) == code, (v, hex(code))
    assert F.e5m2_decode(np.array([0x7C]))[0] == np.inf and np.isnan(F.e5m2_decode(np.array([0x7D]))[0])


def test_e5m2_is_the_rounded_top_byte_of_fp16():
    """Every fp16-representable value: the E5M2 code is the fp16 bit pattern
    rounded to its upper byte (round half to even on the value, which for
    same-sign IEEE patterns is integer rounding of the pattern), saturating at
    0x7B -- numpy's float16 is the independent reference."""
    bits = np.arange(0x7C00, dtype=np.uint16)                  # all finite non-negative fp16
    vals = bits.view(np.float16).astype(np.float64)
    low, high = bits & 0xFF, (bits >> 8).astype(np.int64)
    up = (low > 0x80) | ((low == 0x80) & (high & 1 == 1))
    want = np.minimum(high + up, 0x7B)
    got = F.e5m2_encode(vals).astype(np.int64)
    assert np.array_equal(got, want)
    assert np.array_equal(F.e5m2_encode(-vals[1:]).astype(np.int64), want[1:] | 0x80)
    # and decoding every finite code is exact
    codes = np.arange(0x7C)
    assert np.array_equal(F.e5m2_encode(F.e5m2_decode(codes)), codes.astype(np.uint8))


def test_e8m0_rule_for_e5m2():
    """scale exponent = floor(log2 amax) - 15 for E5M2 (OCP MX), biased by 127."""
    assert int(F.e8m0_from_amax(np.array([1.0]), F.E5M2_EMAX)[0]) == 112
    assert int(F.e8m0_from_amax(np.array([57344.0]), F.E5M2_EMAX)[0]) == 127
    assert int(F.e8m0_from_amax(np.array([1.0]))[0]) == 119          # E4M3: - 8
