"""GPU parity of the offsets scan and the grouped quantizers against the CPU
oracle: bit-exact bytes and scales, untouched capacity / padding regions."""

import numpy as np
import pytest
import torch

import block_scaled_grouped_amd as bsg
from oracle import formats as F
from oracle import offsets as O
from oracle import quantize as Q
import workloads
from gpu_util import (SENTINEL, bf16_dev, device, filled_u8, host, host_u8, to_dev)

pytestmark = pytest.mark.gpu


def _bits(rng, rows, cols, spread=4, outliers=0.01):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-spread, spread + 1, (rows, 1))).astype(np.float32)
    x[rng.random((rows, cols)) < outliers] *= 20
    return F.f32_to_bf16_bits_rne(x)


# ---------------------------------------------------------------- offsets

@pytest.mark.parametrize("name", workloads.CONFIG_NAMES)
@pytest.mark.parametrize("mult,pad", [(1, 1), (1, 128), (4096, 1)])
def test_offsets_match_oracle(name, mult, pad):
    sizes = workloads.group_sizes(name)
    s64, off = bsg.group_offsets_i32_to_i64(to_dev(sizes), multiplier=mult, pad_to=pad)
    ws, wo = O.group_offsets(sizes, mult, pad)
    assert np.array_equal(host(s64), ws) and np.array_equal(host(off), wo)


def test_offsets_256_groups_and_status():
    rng = np.random.default_rng(7)
    sizes = rng.integers(0, 5000, 256).astype(np.int32)
    s64, off = bsg.group_offsets_i32_to_i64(to_dev(sizes), pad_to=128)
    assert np.array_equal(host(off), O.group_offsets(sizes, 1, 128)[1])
    status = torch.zeros(1, dtype=torch.int32, device=device())
    bad = np.array([5, -3, 7], np.int32)
    s64, off = bsg.group_offsets_i32_to_i64(to_dev(bad), capacity=10, status=status)
    assert list(host(off)) == [0, 5, 5, 12]
    assert list(host(s64)) == [5, 0, 7]
    assert int(host(status)[0]) == bsg.DEV_NEGATIVE_SIZE | bsg.DEV_OVER_CAPACITY


# ---------------------------------------------------------------- MXFP8 rowwise

ROW_CASES = [
    # rows_cap, cols, sizes
    (128, 128, [32, 0, 64, 32]),
    (700, 4224, [300, 0, 17, 300]),      # 5 partial 1024-chunks, 83 dead rows
    (64, 160, [10, 20, 30]),             # a short last scale group
    (2049, 7168, [1, 2047]),
]


@pytest.mark.parametrize("rows_cap,cols,sizes", ROW_CASES)
def test_rowwise_bit_exact(rows_cap, cols, sizes):
    rng = np.random.default_rng(rows_cap + cols)
    bits = _bits(rng, rows_cap, cols)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS
    _, off = O.group_offsets(sizes)
    want_d, want_s = Q.mxfp8_rowwise(bits, off)
    d = filled_u8((rows_cap, cols))
    s = filled_u8(bsg.mx_scale_shape(rows_cap, cols))
    out = bsg.grouped_quantize_mxfp8(bf16_dev(bits), to_dev(off), row_data=d, row_scales=s)
    d, s = host_u8(out["row_data"]), host_u8(out["row_scales"])
    assert np.array_equal(d[:live], want_d)
    assert np.array_equal(s[:, :live], want_s)
    assert np.all(d[live:] == SENTINEL) and np.all(s[:, live:] == SENTINEL)


def test_rowwise_codec_sweep_every_exponent():
    """Blocks whose amax walks every bf16 binade (subnormals included), with the
    other 31 elements drawn from every magnitude below it, both signs, zeros
    and saturating values: all element codes and scale bytes bit-exact."""
    rng = np.random.default_rng(99)
    nblk = 1 << 15
    exp_amax = rng.integers(-133, 128, nblk)
    man = rng.integers(0, 128, (nblk, 32))
    exps = exp_amax[:, None] - rng.integers(0, 40, (nblk, 32))
    exps[:, 0] = exp_amax
    vals = np.ldexp(1.0 + man / 128.0, exps)
    vals[rng.random((nblk, 32)) < 0.05] = 0.0
    vals *= np.where(rng.random((nblk, 32)) < 0.5, -1.0, 1.0)
    vals[rng.random((nblk, 32)) < 0.01] = -0.0
    vals = np.clip(vals, -3.0e38, 3.0e38)
    bits = F.f32_to_bf16_bits_rne(vals.astype(np.float32)).reshape(-1, 1024)
    rows = bits.shape[0]
    off = np.array([0, rows])
    want_d, want_s = Q.mxfp8_rowwise(bits, off)
    out = bsg.grouped_quantize_mxfp8(bf16_dev(bits), to_dev(off))
    assert np.array_equal(host_u8(out["row_data"]), want_d)
    assert np.array_equal(host_u8(out["row_scales"]), want_s)


@pytest.mark.parametrize("rows_cap,cols,sizes", ROW_CASES)
def test_rowwise_e5m2_bit_exact(rows_cap, cols, sizes):
    rng = np.random.default_rng(rows_cap + cols + 1)
    bits = _bits(rng, rows_cap, cols)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS
    _, off = O.group_offsets(sizes)
    want_d, want_s = Q.mxfp8_rowwise(bits, off, elem="e5m2")
    d = filled_u8((rows_cap, cols))
    s = filled_u8(bsg.mx_scale_shape(rows_cap, cols))
    bsg.grouped_quantize_mxfp8_rowwise_e5m2(bf16_dev(bits), to_dev(off), row_data=d, row_scales=s)
    d, s = host_u8(d), host_u8(s)
    assert np.array_equal(d[:live], want_d)
    assert np.array_equal(s[:, :live], want_s)
    assert np.all(d[live:] == SENTINEL) and np.all(s[:, live:] == SENTINEL)


def test_rowwise_e5m2_codec_sweep_every_exponent():
    """As the E4M3 sweep, for E5M2 elements: every binade, subnormals, zeros,
    and block members in the top binade that round past 57344 (saturation)."""
    rng = np.random.default_rng(98)
    nblk = 1 << 15
    exp_amax = rng.integers(-133, 128, nblk)
    man = rng.integers(0, 128, (nblk, 32))
    exps = exp_amax[:, None] - rng.integers(0, 40, (nblk, 32))
    exps[:, 0] = exp_amax
    exps[:, 1] = exp_amax                     # a second top-binade element
    man[:, 1] = rng.integers(112, 128, nblk)  # near the top: rounds past 1.75 * 2^15 after scaling
    vals = np.ldexp(1.0 + man / 128.0, exps)
    vals[rng.random((nblk, 32)) < 0.05] = 0.0
    vals *= np.where(rng.random((nblk, 32)) < 0.5, -1.0, 1.0)
    vals = np.clip(vals, -3.0e38, 3.0e38)
    bits = F.f32_to_bf16_bits_rne(vals.astype(np.float32)).reshape(-1, 1024)
    rows = bits.shape[0]
    off = np.array([0, rows])
    want_d, want_s = Q.mxfp8_rowwise(bits, off, elem="e5m2")
    assert np.any((want_d & 0x7F) == 0x7B)    # saturation is exercised
    d, s = bsg.grouped_quantize_mxfp8_rowwise_e5m2(bf16_dev(bits), to_dev(off))
    assert np.array_equal(host_u8(d), want_d)
    assert np.array_equal(host_u8(s), want_s)


# ---------------------------------------------------------------- MXFP8 columnwise (+ fused rowwise)

COL_CASES = [
    (200, 96, [37, 0, 130, 5]),
    (800, 4096, [2049 - 1600, 0, 301, 0, 50]),
    (128, 128, [32, 0, 64, 32]),
]


@pytest.mark.parametrize("rows_cap,cols,sizes", COL_CASES)
@pytest.mark.parametrize("with_rows", [False, True])
def test_colwise_bit_exact(rows_cap, cols, sizes, with_rows):
    rng = np.random.default_rng(rows_cap * 7 + cols)
    bits = _bits(rng, rows_cap, cols)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    want_d, want_s = Q.mxfp8_colwise(bits, off, poff)
    G = len(sizes)
    cap = rows_cap + 128 * G
    cd = filled_u8((cap * cols,))
    cs = filled_u8((cap * cols // 32,))
    kw = {}
    if with_rows:
        kw = dict(row_data=filled_u8((rows_cap, cols)),
                  row_scales=filled_u8(bsg.mx_scale_shape(rows_cap, cols)))
    out = bsg.grouped_quantize_mxfp8(bf16_dev(bits), to_dev(off), rowwise=with_rows,
                                     padded_offsets=to_dev(poff), col_rows_cap=cap, col_data=cd,
                                     col_scales=cs, **kw)
    d, s = host_u8(out["col_data"]), host_u8(out["col_scales"])
    n = int(poff[-1]) * cols
    assert np.array_equal(d[:n], want_d)
    assert np.array_equal(s[:n // 32], want_s)
    assert np.all(d[n:] == SENTINEL) and np.all(s[n // 32:] == SENTINEL)
    if with_rows:
        rd, rs = Q.mxfp8_rowwise(bits, off)
        assert np.array_equal(host_u8(out["row_data"])[:live], rd)
        assert np.array_equal(host_u8(out["row_scales"])[:, :live], rs)
        assert np.all(host_u8(out["row_scales"])[:, live:] == SENTINEL)
        assert np.all(host_u8(out["row_data"])[live:] == SENTINEL)


@pytest.mark.parametrize("rows_cap,cols,sizes", COL_CASES)
def test_colwise_e5m2_bit_exact(rows_cap, cols, sizes):
    """The gradient's E5M2 columnwise copy, with values spread over many
    binades (including blocks past the E5M2 range after scaling)."""
    rng = np.random.default_rng(rows_cap * 13 + cols)
    bits = _bits(rng, rows_cap, cols, spread=12, outliers=0.05)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    want_d, want_s = Q.mxfp8_colwise(bits, off, poff, elem="e5m2")
    G = len(sizes)
    cap = rows_cap + 128 * G
    cd = filled_u8((cap * cols,))
    cs = filled_u8((cap * cols // 32,))
    bsg.grouped_quantize_mxfp8_colwise_e5m2(bf16_dev(bits), to_dev(off), to_dev(poff),
                                            col_rows_cap=cap, col_data=cd, col_scales=cs)
    d, s = host_u8(cd), host_u8(cs)
    n = int(poff[-1]) * cols
    assert np.array_equal(d[:n], want_d)
    assert np.array_equal(s[:n // 32], want_s)
    assert np.all(d[n:] == SENTINEL) and np.all(s[n // 32:] == SENTINEL)


def test_colwise_bad_padding_flagged():
    bits = _bits(np.random.default_rng(3), 64, 64)
    off = np.array([0, 10, 64])
    poff = np.array([0, 64, 192])          # group 0 padded to 64, not 128
    status = torch.zeros(1, dtype=torch.int32, device=device())
    bsg.grouped_quantize_mxfp8(bf16_dev(bits), to_dev(off), rowwise=False,
                               padded_offsets=to_dev(poff), col_rows_cap=256, status=status)
    torch.cuda.synchronize()
    assert int(host(status)[0]) & bsg.DEV_BAD_PADDING


# ---------------------------------------------------------------- NVFP4 row-scaled

NV_CASES = [
    (400, 4096, [100, 0, 157, 43]),
    (64, 160, [17, 0, 30]),
    (40, 16384, [33]),
    (128, 128, [32, 0, 64, 32]),
    (12, 16416, [3, 0, 5]),              # longer than a thread's registers hold: read twice
    (6, 32768, [4]),
]


@pytest.mark.parametrize("rows_cap,cols,sizes", NV_CASES)
def test_nvfp4_quantize_bit_exact(rows_cap, cols, sizes):
    rng = np.random.default_rng(rows_cap + 3 * cols)
    bits = _bits(rng, rows_cap, cols, spread=8)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS
    bits[0] = 0                             # an all-zero row
    _, off = O.group_offsets(sizes)
    wd, ws, wt = Q.nvfp4_rowscaled(bits, off)
    d = filled_u8((rows_cap, cols // 2))
    s = filled_u8((rows_cap, cols // 16))
    t = torch.full((rows_cap,), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_quantize_nvfp4_rowscaled(bf16_dev(bits), to_dev(off), data=d, block_scales=s, outer=t)
    d, s, t = host_u8(d), host_u8(s), host(t)
    assert np.array_equal(d[:live], wd)
    assert np.array_equal(s[:live], ws)
    assert np.array_equal(t[:live].view(np.uint32), wt.view(np.uint32))
    assert np.all(d[live:] == SENTINEL) and np.all(s[live:] == SENTINEL)
    assert np.all(np.isnan(t[live:]))


# ---------------------------------------------------------------- NVFP4 per-tensor

NVT_CASES = [
    (400, 4096, [100, 0, 157, 43]),
    (64, 160, [17, 0, 30]),
    (40, 16384, [33]),
    (300, 96, [0, 5, 0, 250, 1]),          # leading empty group, a one-row group
    (16, 32, [0]),                         # empty routing: only the amax is written (0)
    (3000, 64, [i % 23 for i in range(256)]),   # 256 groups (the maximum), empty ones among them
    (12, 16416, [3, 0, 5]),                # rows read twice by the cast
    (7, 32768, [2, 3]),
]


@pytest.mark.parametrize("rows_cap,cols,sizes", NVT_CASES)
def test_nvfp4_pertensor_bit_exact(rows_cap, cols, sizes):
    rng = np.random.default_rng(rows_cap + 5 * cols)
    bits = _bits(rng, rows_cap, cols, spread=8)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS
    if live:
        bits[0] = 0                         # an all-zero row
    _, off = O.group_offsets(sizes)
    wd, ws, wa = Q.nvfp4_pertensor(bits, off)
    d = filled_u8((rows_cap, cols // 2))
    s = filled_u8((rows_cap, cols // 16))
    a = torch.full((len(sizes),), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(bits), to_dev(off), data=d, block_scales=s,
                                         amax=a)
    d, s, a = host_u8(d), host_u8(s), host(a)
    assert np.array_equal(a.view(np.uint32), wa.view(np.uint32))
    assert np.array_equal(d[:live], wd)
    assert np.array_equal(s[:live], ws)
    assert np.all(d[live:] == SENTINEL) and np.all(s[live:] == SENTINEL)


def test_nvfp4_pertensor_two_calls_reuse_amax():
    """The amax buffer is cleared by every call: a second call with smaller
    values and other group sizes must not keep the first call's maxima."""
    rng = np.random.default_rng(44)
    bits = _bits(rng, 256, 128, spread=2)
    small = F.f32_to_bf16_bits_rne(F.bf16_bits_to_f64(bits).astype(np.float32) * np.float32(1e-3))
    a = torch.empty(3, dtype=torch.float32, device=device())
    for b, sizes in ((bits, [100, 56, 100]), (small, [10, 0, 200])):
        _, off = O.group_offsets(np.array(sizes, np.int32))
        bsg.grouped_quantize_nvfp4_pertensor(bf16_dev(b), to_dev(off), amax=a)
        assert np.array_equal(host(a).view(np.uint32), Q.nvfp4_pertensor(b, off)[2].view(np.uint32))


NVCOL_CASES = [
    (200, 96, [37, 0, 130, 5]),          # a 32-column last slab, an empty expert
    (800, 4096, [449, 0, 301, 0, 50]),
    (300, 160, [257, 1]),                # three 128-token tiles, a one-token expert
    (64, 32, [0, 0, 64]),                # leading empty experts
    (12, 16416, [3, 0, 5]),              # more than 16384 columns
    (5, 32768, [4]),
]


@pytest.mark.parametrize("rows_cap,cols,sizes", NVCOL_CASES)
def test_nvfp4_colwise_bit_exact(rows_cap, cols, sizes):
    rng = np.random.default_rng(rows_cap * 5 + cols)
    bits = _bits(rng, rows_cap, cols, spread=8)
    sizes = np.array(sizes, np.int32)
    live = int(sizes.sum())
    bits[live:] = workloads.BF16_NAN_BITS       # capacity rows: never read
    bits[:, 1] = 0                              # an all-zero column
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    wd, ws, wo = Q.nvfp4_rowscaled_colwise(bits, off, poff)
    G = len(sizes)
    cap = rows_cap + 128 * G
    d = filled_u8((cap * cols // 2,))
    sc = filled_u8((cap * cols // 16,))
    o = torch.full((G, cols), float("nan"), dtype=torch.float32, device=device())
    bsg.grouped_quantize_nvfp4_rowscaled_colwise(bf16_dev(bits), to_dev(off), to_dev(poff),
                                                 col_rows_cap=cap, data=d, block_scales=sc,
                                                 outer=o)
    d, sc, o = host_u8(d), host_u8(sc), host(o)
    n = int(poff[-1]) * cols
    assert np.array_equal(d[:n // 2], wd)
    assert np.array_equal(sc[:n // 16], ws)
    assert np.array_equal(o.view(np.uint32), wo.view(np.uint32))
    assert np.all(d[n // 2:] == SENTINEL) and np.all(sc[n // 16:] == SENTINEL)


def test_nvfp4_colwise_bad_padding_flagged():
    bits = _bits(np.random.default_rng(4), 64, 64)
    off = np.array([0, 10, 64])
    poff = np.array([0, 64, 192])          # expert 0 padded to 64, not 128
    status = torch.zeros(1, dtype=torch.int32, device=device())
    bsg.grouped_quantize_nvfp4_rowscaled_colwise(bf16_dev(bits), to_dev(off), to_dev(poff),
                                                 col_rows_cap=256, status=status)
    torch.cuda.synchronize()
    assert int(host(status)[0]) & bsg.DEV_BAD_PADDING


def test_determinism_two_runs():
    rng = np.random.default_rng(5)
    bits = _bits(rng, 512, 4096)
    off = to_dev(np.array([0, 200, 512]))
    a = bsg.grouped_quantize_mxfp8(bf16_dev(bits), off)
    b = bsg.grouped_quantize_mxfp8(bf16_dev(bits), off)
    assert torch.equal(a["row_data"], b["row_data"]) and torch.equal(a["row_scales"], b["row_scales"])


def test_nan_inf_inputs_stay_in_bounds():
    """NaN and Inf inputs are outside the contract (their codes are
    unspecified), but every quantizer must still write only its live outputs:
    the capacity rows and the bytes past the padded outputs keep their
    sentinels."""
    rng = np.random.default_rng(46)
    rows_cap, cols = 300, 128
    sizes = np.array([100, 0, 57, 43], np.int32)
    live = int(sizes.sum())
    bits = _bits(rng, rows_cap, cols)
    bits[::7, ::5] = 0x7FC0                      # NaN
    bits[3::11, 1::9] = 0x7F80                   # +Inf
    bits[5::13, 2::7] = 0xFF80                   # -Inf
    _, off = O.group_offsets(sizes)
    _, poff = O.group_offsets(sizes, pad_to=128)
    x, doff, dpoff = bf16_dev(bits), to_dev(off), to_dev(poff)
    cap = rows_cap + 128 * len(sizes)
    rd = filled_u8((rows_cap, cols))
    rs = filled_u8(bsg.mx_scale_shape(rows_cap, cols))
    cd = filled_u8((cap * cols,))
    cs = filled_u8((cap * cols // 32,))
    bsg.grouped_quantize_mxfp8(x, doff, row_data=rd, row_scales=rs, padded_offsets=dpoff,
                               col_rows_cap=cap, col_data=cd, col_scales=cs)
    nd = filled_u8((rows_cap, cols // 2))
    ns = filled_u8((rows_cap, cols // 16))
    no = torch.full((rows_cap,), 7.0, dtype=torch.float32, device=device())
    bsg.grouped_quantize_nvfp4_rowscaled(x, doff, data=nd, block_scales=ns, outer=no)
    td = filled_u8((rows_cap, cols // 2))
    ts = filled_u8((rows_cap, cols // 16))
    bsg.grouped_quantize_nvfp4_pertensor(x, doff, data=td, block_scales=ts)
    cd2 = filled_u8((cap * cols // 2,))
    cs2 = filled_u8((cap * cols // 16,))
    bsg.grouped_quantize_nvfp4_rowscaled_colwise(x, doff, dpoff, col_rows_cap=cap, data=cd2,
                                                 block_scales=cs2)
    torch.cuda.synchronize()
    n = int(poff[-1]) * cols
    assert np.all(host_u8(rd)[live:] == SENTINEL)
    assert np.all(host_u8(rs)[:, live:] == SENTINEL)
    assert np.all(host_u8(cd)[n:] == SENTINEL) and np.all(host_u8(cs)[n // 32:] == SENTINEL)
    assert np.all(host_u8(nd)[live:] == SENTINEL) and np.all(host_u8(ns)[live:] == SENTINEL)
    assert np.all(host(no)[live:] == 7.0)
    assert np.all(host_u8(td)[live:] == SENTINEL) and np.all(host_u8(ts)[live:] == SENTINEL)
    assert np.all(host_u8(cd2)[n // 2:] == SENTINEL) and np.all(host_u8(cs2)[n // 16:] == SENTINEL)
