"""The no-allocation entry point grouped_gemm_nvfp4_rowscaled_noalloc (the
two-step FP32-S flow with S in the library's static device scratch), checked
against the existing entry point grouped_gemm_nvfp4_rowscaled with a caller
scratch, on two calls in a row (the second smaller, so the shared scratch still
holds the first call's values) and against the fp64 oracle."""

import ctypes

import numpy as np
import pytest
import torch

import block_scaled_grouped_amd as bsg
from oracle import formats as F
from oracle import gemm as GM
from oracle import offsets as O
from oracle import quantize as Q
from gpu_util import device, gemm_tolerance_check, host, to_dev

pytestmark = pytest.mark.gpu


def _bits(rng, shape, std=1.0):
    return F.f32_to_bf16_bits_rne((rng.standard_normal(shape) * std).astype(np.float32))


def _case(seed, sizes, npg, K, rows_cap):
    rng = np.random.default_rng(seed)
    _, off = O.group_offsets(np.array(sizes, np.int32))
    x = _bits(rng, (rows_cap, K))
    w = _bits(rng, (sum(npg), K), 0.02)
    ap, asc, at = Q.nvfp4_rowscaled(x, off)
    bp, bsc, bt = Q.nvfp4_rowscaled(w, np.array([0, sum(npg)]))

    def rows(a):
        o = np.zeros((rows_cap,) + a.shape[1:], a.dtype)
        o[:a.shape[0]] = a
        return to_dev(o)

    dev_args = (rows(ap), rows(asc), rows(at), to_dev(off), K, to_dev(bp), to_dev(bsc), to_dev(bt),
                list(npg))
    ref = GM.nvfp4_rowscaled_fprop(ap, asc, at, off, bp, bsc, bt, npg, K)
    return dev_args, ref, int(off[-1])


@pytest.mark.parametrize("out_f32", [False, True])
def test_noalloc_equals_caller_scratch_on_two_calls(out_f32):
    dev = device()
    odt = bsg.BSG_OUT_F32 if out_f32 else bsg.BSG_OUT_BF16
    tdt = torch.float32 if out_f32 else torch.bfloat16
    cases = [
        (5, [300, 0, 257, 131], [256, 512, 128, 384], 512, 720),   # the larger call first
        (6, [40, 90, 0], [96, 64, 160], 96, 150),                  # then a smaller one (k % 64 == 32)
    ]
    for seed, sizes, npg, K, rows_cap in cases:
        args, ref, live = _case(seed, sizes, npg, K, rows_cap)
        ld = max(npg) + 4
        want = torch.full((rows_cap, ld), float("nan"), dtype=tdt, device=dev)
        scratch = torch.empty((rows_cap, ld), dtype=torch.float32, device=dev)
        bsg.grouped_gemm_nvfp4_rowscaled(*args, out=want, ld_out=ld, out_dtype=odt,
                                         scratch=scratch)
        got = torch.full((rows_cap, ld), float("nan"), dtype=tdt, device=dev)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated(dev)
        bsg.grouped_gemm_nvfp4_rowscaled_noalloc(*args, out=got, ld_out=ld, out_dtype=odt)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated(dev) == before, "the no-alloc call allocated"
        # bit-identical to the existing entry point, untouched entries included
        assert torch.equal(got.view(torch.int16 if not out_f32 else torch.int32),
                           want.view(torch.int16 if not out_f32 else torch.int32)), (seed, K)
        y = host(got.float()).astype(np.float64)
        for g, (rows, r) in enumerate(ref):
            if len(rows):
                gemm_tolerance_check(y[rows][:, :npg[g]], r, out_f32, "group %d" % g)
                assert np.all(np.isnan(y[rows][:, npg[g]:]))
        assert np.all(np.isnan(y[live:])), "capacity rows must stay untouched"


def test_noalloc_rejects_sizes_past_its_scratch():
    """rows_cap * ld_out * 4 above the static scratch: a clear error from the
    C-ABI, nothing launched."""
    dev = device()
    lib = bsg.load_library()
    rows_cap, ld_out, k = 4097, 4096, 32          # 4097 * 4096 * 4 bytes > 64 MiB
    assert rows_cap * ld_out * 4 > bsg.BSG_NOALLOC_SCRATCH_BYTES
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device=dev)
    p = ctypes.c_void_p(buf.data_ptr())
    npg = (ctypes.c_int64 * 1)(ld_out)
    rc = lib.grouped_gemm_nvfp4_rowscaled_noalloc(1, p, p, p, p, rows_cap, k, p, p, p,
                                                  ctypes.cast(npg, ctypes.c_void_p), p, ld_out,
                                                  bsg.BSG_OUT_BF16, None, None)
    assert rc == 2, rc
    assert b"static scratch" in lib.bsg_last_error()
    assert torch.count_nonzero(buf).item() == 0
    # at the limit the call is accepted (a small live range keeps it cheap)
    rows_cap = bsg.BSG_NOALLOC_SCRATCH_BYTES // (4 * ld_out)
    a = torch.zeros((rows_cap, k // 2), dtype=torch.uint8, device=dev)
    asc = torch.zeros((rows_cap, k // 16), dtype=torch.uint8, device=dev)
    ao = torch.ones(rows_cap, dtype=torch.float32, device=dev)
    off = torch.tensor([0, 3], dtype=torch.int64, device=dev)
    b = torch.zeros((ld_out, k // 2), dtype=torch.uint8, device=dev)
    bs = torch.zeros((ld_out, k // 16), dtype=torch.uint8, device=dev)
    bo = torch.ones(ld_out, dtype=torch.float32, device=dev)
    out = torch.full((rows_cap, ld_out), float("nan"), dtype=torch.bfloat16, device=dev)
    bsg.grouped_gemm_nvfp4_rowscaled_noalloc(a, asc, ao, off, k, b, bs, bo, [ld_out], out=out)
    torch.cuda.synchronize()
    assert torch.all(out[:3] == 0) and torch.isnan(out[3:]).all()
