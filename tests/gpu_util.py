"""Shared helpers of the GPU tests: device tensors from host arrays, the HIP
binding, and the GEMM tolerance."""

import numpy as np
import torch

import block_scaled_grouped_amd as bsg

SENTINEL = 0xAB


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    bsg.load_library()          # fails loudly when the HIP library is missing
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device())


def bf16_dev(bits):
    return to_dev(np.asarray(bits, np.uint16).view(np.int16), torch.bfloat16)


def host(t):
    return t.detach().cpu().numpy()


def host_u8(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def filled_u8(shape, value=SENTINEL):
    return torch.full(shape, value, dtype=torch.uint8, device=device())


def gemm_tolerance_check(y, ref, out_f32, what=""):
    """Max relative error 1e-3 against the fp64 oracle, read per group:
    f32 out: max|y - r| <= 1e-3 * max|r|;  bf16 out: |y - r| <= 2^-8 |r| + 1e-3 max|r|
    elementwise (bf16's own rounding is 2^-9 relative).  Returns the max relative
    error max|y - r| / max|r|."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    assert y.shape == ref.shape, (what, y.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(y)), what
    scale = np.max(np.abs(ref))
    err = np.abs(y - ref)
    if scale == 0:
        assert np.all(err == 0), what
        return 0.0
    if out_f32:
        assert err.max() <= 1e-3 * scale, (what, err.max() / scale)
    else:
        bad = err > 2.0 ** -8 * np.abs(ref) + 1e-3 * scale
        assert not bad.any(), (what, int(bad.sum()), err.max() / scale)
    return float(err.max() / scale)


def bf16_out_to_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)
