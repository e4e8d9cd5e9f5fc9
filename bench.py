"""Benchmark of the grouped block-scaled quantize + grouped GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

One step = one pass of the MoE expert-product hot path over one batch of
seeded synthetic input, inputs already resident in HBM:

  fprop (8 experts, 16384 routed rows, K = 4096, N = 14336; the headline):
      int32 sizes -> int64 offsets (live, and 128-padded)
      -> MXFP8 quantize of the activations, rowwise + columnwise in one pass
      -> MXFP8 quantize of the expert weights (rowwise)
      -> grouped MXFP8 GEMM, fprop TN, bf16 out.

The other MoE shapes (tiny, wgrad, 64-expert Zipf, row-scaled NVFP4) are timed
the same way and reported under "configs".  Before every timed step a 512 MiB
buffer is read (a reduction over it), so the 256 MB MALL holds none of the
step's inputs (cold numbers) and no dirty lines whose write-back would land in
the first kernel's time; per-kernel times come from HIP events recorded on the
stream the kernels run on, around each launch.

Prints ONE JSON line on stdout (details go to stderr).
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

import block_scaled_grouped_amd as bsg
import workloads

HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
# HBM bytes per fprop GEMM launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (scaled by a copy of
# known size), recorded with the hash of the kernel source they were taken with
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemm_mxfp8_fprop_moe_8exp_16384x4096x14336_traffic.json")
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp4": 10100.0, "bf16": 2500.0}
METRIC = "MXFP8 grouped GEMM TFLOP/s + grouped quantize GB/s (1 MI355X, % roofline)"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- cases

class Case:
    """Allocates a workload's buffers on the device and launches one step."""

    kernels = ()

    def step(self, ev=None):
        raise NotImplementedError

    def _rec(self, ev, i):
        if ev is not None:
            ev[i].record()


class MxFprop(Case):
    """offsets -> quantize X (row [+ col]) -> quantize W -> grouped GEMM fprop."""

    def __init__(self, name, dev, with_colwise=True):
        self.name = name
        self.w = w = workloads.get(name)
        t = workloads.tensors(w, device=dev)
        self.x, self.wt = t["x"], t["w"]
        G, N, K, R = w.G, w.n, w.k, w.rows_cap
        self.G, self.N, self.K, self.R = G, N, K, R
        self.sizes = torch.from_numpy(w.sizes).to(dev)
        self.s64 = torch.empty(G, dtype=torch.int64, device=dev)
        self.off = torch.empty(G + 1, dtype=torch.int64, device=dev)
        self.with_colwise = with_colwise
        self.poff = torch.empty(G + 1, dtype=torch.int64, device=dev)
        self.col_cap = R + 128 * G
        self.xr = torch.empty((R, K), dtype=torch.uint8, device=dev)
        self.xrs = torch.empty(bsg.mx_scale_shape(R, K), dtype=torch.uint8, device=dev)
        if with_colwise:
            self.xc = torch.empty(self.col_cap * K, dtype=torch.uint8, device=dev)
            self.xcs = torch.empty(self.col_cap * K // 32, dtype=torch.uint8, device=dev)
        self.woff = torch.tensor([0, G * N], dtype=torch.int64, device=dev)
        self.wq = torch.empty((G * N, K), dtype=torch.uint8, device=dev)
        self.wqs = torch.empty(bsg.mx_scale_shape(G * N, K), dtype=torch.uint8, device=dev)
        self.y = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
        self.ws = bsg.gemm_workspace(dev)  # lets the GEMM split a partly filled last round
        self.kernels = ("offsets", "quantize_x", "quantize_w", "gemm")
        live = w.live_rows
        self.flops = 2.0 * live * N * K
        per_dir = 1.0 + 1.0 / 32
        self.bytes = {
            "offsets": 0.0,
            "quantize_x": live * K * (2.0 + per_dir * (2 if with_colwise else 1)),
            "quantize_w": G * N * K * (2.0 + per_dir),
            "gemm": (live * K * per_dir + sum(N * K * per_dir for s in w.sizes if s > 0)
                     + live * N * 2.0),
        }

    def step(self, ev=None):
        self._rec(ev, 0)
        bsg.group_offsets_i32_to_i64(self.sizes, sizes_i64=self.s64, offsets=self.off,
                                     capacity=self.R)
        if self.with_colwise:
            bsg.group_offsets_i32_to_i64(self.sizes, pad_to=128, offsets=self.poff)
        self._rec(ev, 1)
        if self.with_colwise:
            bsg.grouped_quantize_mxfp8(self.x, self.off, row_data=self.xr, row_scales=self.xrs,
                                       padded_offsets=self.poff, col_rows_cap=self.col_cap,
                                       col_data=self.xc, col_scales=self.xcs)
        else:
            bsg.grouped_quantize_mxfp8(self.x, self.off, row_data=self.xr, row_scales=self.xrs)
        self._rec(ev, 2)
        bsg.grouped_quantize_mxfp8(self.wt.view(self.G * self.N, self.K), self.woff, row_data=self.wq,
                                   row_scales=self.wqs)
        self._rec(ev, 3)
        bsg.grouped_gemm_mxfp8(bsg.BSG_FPROP_TN, self.xr, self.xrs, self.wq, self.wqs, self.off,
                               self.R, self.N, self.K, out=self.y, out_dtype=bsg.BSG_OUT_BF16,
                               workspace=self.ws)
        self._rec(ev, 4)


class MxWgrad(Case):
    """offsets -> columnwise quantize of dY and X -> grouped GEMM wgrad (e5m2:
    dY's copy in E5M2, the E5M2 x E4M3 product)."""

    def __init__(self, name, dev, e5m2=False):
        self.name = name
        self.e5m2 = e5m2
        self.w = w = workloads.get("wgrad" if e5m2 else name)
        t = workloads.tensors(w, device=dev)
        self.dy, self.x = t["dy"], t["x"]
        G, N, K, R = w.G, w.n, w.k, w.rows_cap
        self.G, self.N, self.K, self.R = G, N, K, R
        self.sizes = torch.from_numpy(w.sizes).to(dev)
        self.off = torch.empty(G + 1, dtype=torch.int64, device=dev)
        self.poff = torch.empty(G + 1, dtype=torch.int64, device=dev)
        self.cap = R + 128 * G
        self.dyc = torch.empty(self.cap * N, dtype=torch.uint8, device=dev)
        self.dycs = torch.empty(self.cap * N // 32, dtype=torch.uint8, device=dev)
        self.xc = torch.empty(self.cap * K, dtype=torch.uint8, device=dev)
        self.xcs = torch.empty(self.cap * K // 32, dtype=torch.uint8, device=dev)
        self.dw = torch.empty((G, N, K), dtype=torch.bfloat16, device=dev)
        self.kernels = ("offsets", "quantize_dy", "quantize_x", "gemm")
        live = w.live_rows
        per = 1.0 + 1.0 / 32
        self.flops = 2.0 * live * N * K
        self.bytes = {"offsets": 0.0, "quantize_dy": live * N * (2.0 + per),
                      "quantize_x": live * K * (2.0 + per),
                      "gemm": live * (N + K) * per + G * N * K * 2.0}

    def step(self, ev=None):
        self._rec(ev, 0)
        bsg.group_offsets_i32_to_i64(self.sizes, offsets=self.off, capacity=self.R)
        bsg.group_offsets_i32_to_i64(self.sizes, pad_to=128, offsets=self.poff)
        self._rec(ev, 1)
        if self.e5m2:
            bsg.grouped_quantize_mxfp8_colwise_e5m2(self.dy, self.off, self.poff,
                                                    col_rows_cap=self.cap, col_data=self.dyc,
                                                    col_scales=self.dycs)
        else:
            bsg.grouped_quantize_mxfp8(self.dy, self.off, rowwise=False, padded_offsets=self.poff,
                                       col_rows_cap=self.cap, col_data=self.dyc,
                                       col_scales=self.dycs)
        self._rec(ev, 2)
        bsg.grouped_quantize_mxfp8(self.x, self.off, rowwise=False, padded_offsets=self.poff,
                                   col_rows_cap=self.cap, col_data=self.xc, col_scales=self.xcs)
        self._rec(ev, 3)
        bsg.grouped_gemm_mxfp8(bsg.BSG_WGRAD_NT_E5M2 if self.e5m2 else bsg.BSG_WGRAD_NT, self.dyc,
                               self.dycs, self.xc, self.xcs, self.poff, self.cap, self.N, self.K,
                               out=self.dw, out_dtype=bsg.BSG_OUT_BF16)
        self._rec(ev, 4)


class MxDgrad(Case):
    """offsets -> E5M2 rowwise quantize of dY -> columnwise (transposed) E4M3
    quantize of W -> grouped GEMM dgrad (dX = dY W_g)."""

    def __init__(self, name, dev):
        self.name = name
        self.w = w = workloads.get(name)
        t = workloads.tensors(w, device=dev)
        self.dy, self.wt = t["dy"], t["w"]
        G, N, K, R = w.G, w.n, w.k, w.rows_cap      # K: contraction, N: dX columns
        self.G, self.N, self.K, self.R = G, N, K, R
        self.sizes = torch.from_numpy(w.sizes).to(dev)
        self.off = torch.empty(G + 1, dtype=torch.int64, device=dev)
        # the weights' expert offsets as rows of the [G * K, N] view (static)
        self.woff = torch.arange(G + 1, dtype=torch.int64, device=dev) * K
        self.dyd = torch.empty((R, K), dtype=torch.uint8, device=dev)
        self.dys = torch.empty(bsg.mx_scale_shape(R, K), dtype=torch.uint8, device=dev)
        self.wc = torch.empty(G * K * N, dtype=torch.uint8, device=dev)
        self.wcs = torch.empty(G * K * N // 32, dtype=torch.uint8, device=dev)
        self.dx = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
        self.ws = bsg.gemm_workspace(dev)  # lets the GEMM split a partly filled last round
        self.kernels = ("offsets", "quantize_dy", "quantize_w", "gemm")
        live = w.live_rows
        per = 1.0 + 1.0 / 32
        self.flops = 2.0 * live * K * N
        self.bytes = {"offsets": 0.0, "quantize_dy": live * K * (2.0 + per),
                      "quantize_w": G * K * N * (2.0 + per),
                      "gemm": (live * K + G * K * N) * per + live * N * 2.0}

    def step(self, ev=None):
        self._rec(ev, 0)
        bsg.group_offsets_i32_to_i64(self.sizes, offsets=self.off, capacity=self.R)
        self._rec(ev, 1)
        bsg.grouped_quantize_mxfp8_rowwise_e5m2(self.dy, self.off, row_data=self.dyd,
                                                row_scales=self.dys)
        self._rec(ev, 2)
        bsg.grouped_quantize_mxfp8(self.wt.view(self.G * self.K, self.N), self.woff, rowwise=False,
                                   padded_offsets=self.woff, col_rows_cap=self.G * self.K,
                                   col_data=self.wc, col_scales=self.wcs)
        self._rec(ev, 3)
        bsg.grouped_gemm_mxfp8(bsg.BSG_DGRAD_NN, self.dyd, self.dys, self.wc, self.wcs, self.off,
                               self.R, self.N, self.K, out=self.dx, out_dtype=bsg.BSG_OUT_BF16,
                               workspace=self.ws)
        self._rec(ev, 4)


class Nvfp4Wgrad(Case):
    """offsets -> row-scaled NVFP4 columnwise quantize of dY and X -> NVFP4
    grouped GEMM wgrad with the fused per-expert outer-scale epilogue."""

    def __init__(self, name, dev):
        self.name = name
        self.w = w = workloads.get(name)
        t = workloads.tensors(w, device=dev)
        self.dy, self.x = t["dy"], t["x"]
        G, N, K, R = w.G, w.n, w.k, w.rows_cap
        self.G, self.N, self.K, self.R = G, N, K, R
        self.sizes = torch.from_numpy(w.sizes).to(dev)
        self.off = torch.empty(G + 1, dtype=torch.int64, device=dev)
        self.poff = torch.empty(G + 1, dtype=torch.int64, device=dev)
        self.cap = R + 128 * G
        self.dyc = torch.empty(self.cap * N // 2, dtype=torch.uint8, device=dev)
        self.dys = torch.empty(self.cap * N // 16, dtype=torch.uint8, device=dev)
        self.dyo = torch.empty((G, N), dtype=torch.float32, device=dev)
        self.xc = torch.empty(self.cap * K // 2, dtype=torch.uint8, device=dev)
        self.xs = torch.empty(self.cap * K // 16, dtype=torch.uint8, device=dev)
        self.xo = torch.empty((G, K), dtype=torch.float32, device=dev)
        self.dw = torch.empty((G, N, K), dtype=torch.bfloat16, device=dev)
        self.kernels = ("offsets", "quantize_dy", "quantize_x", "gemm")
        live = w.live_rows
        per = 0.5 + 1.0 / 16
        self.flops = 2.0 * live * N * K
        self.bytes = {"offsets": 0.0, "quantize_dy": live * N * (2.0 + per) + 4.0 * G * N,
                      "quantize_x": live * K * (2.0 + per) + 4.0 * G * K,
                      "gemm": live * (N + K) * per + G * N * K * 2.0}

    def step(self, ev=None):
        self._rec(ev, 0)
        bsg.group_offsets_i32_to_i64(self.sizes, offsets=self.off, capacity=self.R)
        bsg.group_offsets_i32_to_i64(self.sizes, pad_to=128, offsets=self.poff)
        self._rec(ev, 1)
        bsg.grouped_quantize_nvfp4_rowscaled_colwise(self.dy, self.off, self.poff,
                                                     col_rows_cap=self.cap, data=self.dyc,
                                                     block_scales=self.dys, outer=self.dyo)
        self._rec(ev, 2)
        bsg.grouped_quantize_nvfp4_rowscaled_colwise(self.x, self.off, self.poff,
                                                     col_rows_cap=self.cap, data=self.xc,
                                                     block_scales=self.xs, outer=self.xo)
        self._rec(ev, 3)
        bsg.grouped_gemm_nvfp4_rowscaled_wgrad(self.dyc, self.dys, self.dyo, self.xc, self.xs,
                                               self.xo, self.poff, self.N, self.K,
                                               col_rows_cap=self.cap, out=self.dw)
        self._rec(ev, 4)


class Nvfp4Fprop(Case):
    """offsets -> row-scaled NVFP4 quantize of X and W -> grouped GEMM with the
    fused outer-scale epilogue, or (scratch) the pages' two-step flow: the GEMM
    stores FP32 S in a [rows_cap, ld] scratch and a second kernel applies the
    outer scales into the bf16 output ("gemm" then times both kernels)."""

    def __init__(self, name, dev, scratch=False):
        self.name = name
        self.w = w = workloads.get("nvfp4" if scratch else name)
        t = workloads.tensors(w, device=dev)
        self.x, self.wt = t["x"], t["w"]
        G, K, R = w.G, w.k, w.rows_cap
        self.npg = list(w.n_per_group)
        NB = sum(self.npg)
        self.G, self.K, self.R, self.ld = G, K, R, max(self.npg)
        self.sizes = torch.from_numpy(w.sizes).to(dev)
        self.off = torch.empty(G + 1, dtype=torch.int64, device=dev)
        self.xd = torch.empty((R, K // 2), dtype=torch.uint8, device=dev)
        self.xs = torch.empty((R, K // 16), dtype=torch.uint8, device=dev)
        self.xo = torch.empty(R, dtype=torch.float32, device=dev)
        self.woff = torch.tensor([0, NB], dtype=torch.int64, device=dev)
        self.wd = torch.empty((NB, K // 2), dtype=torch.uint8, device=dev)
        self.ws = torch.empty((NB, K // 16), dtype=torch.uint8, device=dev)
        self.wo = torch.empty(NB, dtype=torch.float32, device=dev)
        self.y = torch.empty((R, self.ld), dtype=torch.bfloat16, device=dev)
        self.scratch = (torch.empty((R, self.ld), dtype=torch.float32, device=dev) if scratch
                        else None)
        # the fused flow may split a partly filled last round of tiles
        self.gws = None if scratch else bsg.gemm_workspace(dev)
        self.kernels = ("offsets", "quantize_x", "quantize_w", "gemm")
        live = w.live_rows
        self.flops = 2.0 * K * float(sum(int(m) * n for m, n in zip(w.sizes, self.npg)))
        per = 0.5 + 1.0 / 16
        self.bytes = {"offsets": 0.0, "quantize_x": live * (K * (2.0 + per) + 4),
                      "quantize_w": NB * (K * (2.0 + per) + 4),
                      "gemm": live * K * per + NB * K * per
                      + 2.0 * float(sum(int(m) * n for m, n in zip(w.sizes, self.npg)))}

    def step(self, ev=None):
        self._rec(ev, 0)
        bsg.group_offsets_i32_to_i64(self.sizes, offsets=self.off, capacity=self.R)
        self._rec(ev, 1)
        bsg.grouped_quantize_nvfp4_rowscaled(self.x, self.off, data=self.xd, block_scales=self.xs,
                                             outer=self.xo)
        self._rec(ev, 2)
        bsg.grouped_quantize_nvfp4_rowscaled(self.wt, self.woff, data=self.wd, block_scales=self.ws,
                                             outer=self.wo)
        self._rec(ev, 3)
        bsg.grouped_gemm_nvfp4_rowscaled(self.xd, self.xs, self.xo, self.off, self.K, self.wd, self.ws,
                                         self.wo, self.npg, out=self.y, ld_out=self.ld,
                                         out_dtype=bsg.BSG_OUT_BF16, scratch=self.scratch,
                                         workspace=self.gws)
        self._rec(ev, 4)


class Nvfp4PerTensorFprop(Case):
    """offsets -> per-tensor NVFP4 quantize of X (one amax per expert's rows)
    and W (one amax per expert) -> grouped GEMM with alpha_g = tsi_A * tsi_B.
    variant "rht": X and W both through the randomized Hadamard transform with
    the same 16 signs (drawn from the workload's seed); "2d": W with 16 x 16
    block scales."""

    def __init__(self, name, dev, variant=None):
        self.name = name
        self.variant = variant
        self.w = w = workloads.get("nvfp4_pertensor" if variant else name)
        self.rht_mask = int(np.random.default_rng(w.seed).integers(0, 1 << 16))
        t = workloads.tensors(w, device=dev)
        self.x, self.wt = t["x"], t["w"]
        G, K, R = w.G, w.k, w.rows_cap
        self.npg = list(w.n_per_group)
        NB = sum(self.npg)
        self.G, self.K, self.R, self.ld = G, K, R, max(self.npg)
        self.sizes = torch.from_numpy(w.sizes).to(dev)
        self.off = torch.empty(G + 1, dtype=torch.int64, device=dev)
        self.xd = torch.empty((R, K // 2), dtype=torch.uint8, device=dev)
        self.xs = torch.empty((R, K // 16), dtype=torch.uint8, device=dev)
        self.xa = torch.empty(G, dtype=torch.float32, device=dev)
        self.woff = torch.from_numpy(np.concatenate([[0], np.cumsum(self.npg)])).to(dev)
        self.wd = torch.empty((NB, K // 2), dtype=torch.uint8, device=dev)
        self.ws = torch.empty((NB, K // 16), dtype=torch.uint8, device=dev)
        self.wa = torch.empty(G, dtype=torch.float32, device=dev)
        self.y = torch.empty((R, self.ld), dtype=torch.bfloat16, device=dev)
        self.gws = bsg.gemm_workspace(dev)  # lets the GEMM split a partly filled last round
        self.kernels = ("offsets", "quantize_x", "quantize_w", "gemm")
        live = w.live_rows
        self.flops = 2.0 * K * float(sum(int(m) * n for m, n in zip(w.sizes, self.npg)))
        per = 0.5 + 1.0 / 16
        # one read of the input counted (the group amax pass reads it a second time)
        self.bytes = {"offsets": 0.0, "quantize_x": live * K * (2.0 + per) + 4 * G,
                      "quantize_w": NB * K * (2.0 + per) + 4 * G,
                      "gemm": live * K * per + NB * K * per
                      + 2.0 * float(sum(int(m) * n for m, n in zip(w.sizes, self.npg)))}

    def step(self, ev=None):
        self._rec(ev, 0)
        bsg.group_offsets_i32_to_i64(self.sizes, offsets=self.off, capacity=self.R)
        self._rec(ev, 1)
        if self.variant == "rht":
            bsg.grouped_quantize_nvfp4_pertensor_rht(self.x, self.off, self.rht_mask, data=self.xd,
                                                     block_scales=self.xs, amax=self.xa)
        else:
            bsg.grouped_quantize_nvfp4_pertensor(self.x, self.off, data=self.xd,
                                                 block_scales=self.xs, amax=self.xa)
        self._rec(ev, 2)
        if self.variant == "rht":
            bsg.grouped_quantize_nvfp4_pertensor_rht(self.wt, self.woff, self.rht_mask,
                                                     data=self.wd, block_scales=self.ws,
                                                     amax=self.wa)
        elif self.variant == "2d":
            bsg.grouped_quantize_nvfp4_pertensor_2d(self.wt, self.woff, data=self.wd,
                                                    block_scales=self.ws, amax=self.wa)
        else:
            bsg.grouped_quantize_nvfp4_pertensor(self.wt, self.woff, data=self.wd,
                                                 block_scales=self.ws, amax=self.wa)
        self._rec(ev, 3)
        bsg.grouped_gemm_nvfp4_pertensor(self.xd, self.xs, self.xa, self.off, self.K, self.wd,
                                         self.ws, self.wa, self.npg, out=self.y, ld_out=self.ld,
                                         out_dtype=bsg.BSG_OUT_BF16, workspace=self.gws)
        self._rec(ev, 4)


def make_case(name, dev):
    if name in ("tiny", "zipf"):
        return MxFprop(name, dev, with_colwise=False)
    if name == "fprop":
        return MxFprop(name, dev, with_colwise=True)
    if name == "wgrad":
        return MxWgrad(name, dev)
    if name == "wgrad_e5m2":
        return MxWgrad(name, dev, e5m2=True)
    if name == "nvfp4":
        return Nvfp4Fprop(name, dev)
    if name == "nvfp4_scratch":
        return Nvfp4Fprop(name, dev, scratch=True)
    if name == "nvfp4_wgrad":
        return Nvfp4Wgrad(name, dev)
    if name == "dgrad":
        return MxDgrad(name, dev)
    if name == "nvfp4_pertensor":
        return Nvfp4PerTensorFprop(name, dev)
    if name == "nvfp4_rht":
        return Nvfp4PerTensorFprop(name, dev, variant="rht")
    if name == "nvfp4_2d":
        return Nvfp4PerTensorFprop(name, dev, variant="2d")
    raise KeyError(name)


# ---------------------------------------------------------------- timing

# GPU cycles of the spin kernel queued ahead of every timed step: while the GPU
# spins, the host enqueues the whole step, so the events around each kernel see
# the GPU go from one kernel to the next without waiting for the host
SPIN_CYCLES = 3_000_000

# Timing-only HIP events: created with hipEventDisableSystemFence, so that
# recording one does not write back and invalidate the caches (the HIP runtime
# documents the flag for events used only to measure time; their elapsed times
# are read after a full synchronize).  torch's events carry that fence, which
# adds ~1.5 us to each bracketed kernel and perturbs the next one.
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000
_hip = None


class TimingEvent:
    def __init__(self):
        import ctypes
        global _hip
        if _hip is None:
            _hip = ctypes.CDLL("libamdhip64.so")
            _hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            _hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            _hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
            _hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._ct = ctypes
        self.e = ctypes.c_void_p()
        rc = _hip.hipEventCreateWithFlags(ctypes.byref(self.e), _HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError("hipEventCreateWithFlags failed: %d" % rc)

    def record(self):
        stream = self._ct.c_void_p(torch.cuda.current_stream().cuda_stream)
        rc = _hip.hipEventRecord(self.e, stream)
        if rc != 0:
            raise RuntimeError("hipEventRecord failed: %d" % rc)

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        rc = _hip.hipEventElapsedTime(self._ct.byref(ms), self.e, end.e)
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return ms.value

    def __del__(self):
        if _hip is not None and self.e:
            _hip.hipEventDestroy(self.e)


def time_case(case, steps, warmup, flush_buf):
    for _ in range(warmup):
        case.step()
    torch.cuda.synchronize()
    nk = len(case.kernels)
    per_kernel = np.zeros((steps, nk))
    step_ms = np.zeros(steps)
    evs = [[TimingEvent() for _ in range(nk + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        if flush_buf is not None:
            flush_buf.sum()
        torch.cuda._sleep(SPIN_CYCLES)
        case.step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for s in range(steps):
        for i in range(nk):
            per_kernel[s, i] = evs[s][i].elapsed_time(evs[s][i + 1])
        step_ms[s] = evs[s][0].elapsed_time(evs[s][nk])
    return {
        "step_ms": float(np.median(step_ms)),
        "step_ms_mean": float(step_ms.mean()),
        "wall_ms_per_step": 1e3 * wall / steps,
        "kernel_ms": {k: float(np.median(per_kernel[:, i])) for i, k in enumerate(case.kernels)},
    }


def summarize(case, t, mfma_dtype):
    km = t["kernel_ms"]
    gemm_tf = case.flops / (km["gemm"] * 1e-3) / 1e12
    out = {"workload": case.name, "step_ms": round(t["step_ms"], 4),
           "step_ms_mean": round(t["step_ms_mean"], 4),
           "step_tflops": round(case.flops / (t["step_ms"] * 1e-3) / 1e12, 2),
           "gemm_us": round(km["gemm"] * 1e3, 2),
           "gemm_tflops": round(gemm_tf, 2),
           "gemm_frac_of_peak": round(gemm_tf / MFMA_PEAK_TFLOPS[mfma_dtype], 4),
           "mfma_peak_tflops": MFMA_PEAK_TFLOPS[mfma_dtype], "kernels_us": {}}
    if mfma_dtype == "bf16":
        # the NVFP4 GEMM runs on fp16 MFMA (the design bound); the FP4 peak alongside
        out["gemm_frac_of_fp4_peak"] = round(gemm_tf / MFMA_PEAK_TFLOPS["fp4"], 4)
    for k, ms in km.items():
        ent = {"us": round(ms * 1e3, 2)}
        b = case.bytes.get(k, 0.0)
        if b and k != "gemm":
            gbs = b / (ms * 1e-3) / 1e9
            ent.update({"algorithmic_bytes": int(b), "GB_s": round(gbs, 1),
                        "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4)})
        out["kernels_us"][k] = ent
    w = case.w
    out["group_sizes"] = [int(v) for v in w.sizes]
    if w.n_per_group is not None:
        out["n_per_group"] = [int(v) for v in w.n_per_group]
    return out


def input_digests(case):
    """SHA-256 of every bf16 input tensor of a case (the bytes on the device)."""
    import hashlib
    out = {}
    for key in ("x", "wt", "dy"):
        t = getattr(case, key, None)
        if t is None:
            continue
        h = hashlib.sha256()
        flat = t.reshape(-1).view(torch.int16)
        step = 1 << 26
        for i in range(0, flat.numel(), step):
            h.update(flat[i:i + step].cpu().numpy().tobytes())
        out["w" if key == "wt" else key] = h.hexdigest()
    return out


def device_copy_rate(dev, flush_buf, nbytes=256 << 20, iters=20):
    """Median rate of the runtime's device-to-device copy of nbytes, cold,
    counting bytes read + written: a practical ceiling for HBM-bound kernels."""
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ts = []
    for _ in range(iters):
        if flush_buf is not None:
            flush_buf.sum()
        torch.cuda._sleep(SPIN_CYCLES // 4)
        e0 = TimingEvent()
        e1 = TimingEvent()
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    ms = float(np.median(ts))
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


# ---------------------------------------------------------------- CPU baseline (the oracle)

def code_sha256(paths):
    """sha256 of source files' code: every line with its // comment and
    surrounding whitespace removed, blank lines dropped, files in the given
    order, so that editing a comment keeps the hash and editing code changes it."""
    import hashlib
    lines = []
    for path in paths:
        for line in open(path, encoding="utf-8"):
            code = line.split("//", 1)[0].strip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def gemm_traffic():
    """Counter-measured HBM bytes of one fprop GEMM launch and the record they
    come from, or (None, reason) when no record exists or the kernel's code (its
    source and the local headers it includes) has changed since it was taken."""
    rel = os.path.relpath(TRAFFIC_RECORD, ROOT)
    try:
        rec = json.load(open(TRAFFIC_RECORD))
        sha = code_sha256([os.path.join(ROOT, f) for f in rec["kernel_sources"]])
    except (OSError, ValueError, KeyError):
        return None, "no traffic record"
    if sha != rec.get("kernel_code_sha256"):
        return None, "%s was taken with other kernel code" % rel
    return int(rec["traffic_bytes"]), ("rocprofv3 FETCH_SIZE + WRITE_SIZE of the same kernel code, "
                                       "recorded in %s" % rel)


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_threads():
    try:
        import threadpoolctl
        n = [i.get("num_threads") for i in threadpoolctl.threadpool_info()
             if i.get("user_api") == "blas"]
        return max(n) if n else None
    except Exception:
        return None


def _host_bf16(shape, std, seed, outlier_p=0.0, outlier_mul=1.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(shape, generator=g) * std
    if outlier_p:
        x = torch.where(torch.rand(shape, generator=g) < outlier_p, x * outlier_mul, x)
    return workloads.bf16_bits(x.to(torch.bfloat16))


def cpu_baseline():
    """The oracle, untuned, on bounded samples of each workload (same value
    distributions, smaller shapes, drawn on the host), timed on this host's
    cores: quantize GB/s (numpy, single-threaded) and fp64 GEMM GFLOP/s (numpy
    matmul on BLAS threads).  The headline value is the fprop sample's
    quantize + GEMM work in the metric's unit (TFLOP/s)."""
    from oracle import gemm as GM
    from oracle import quantize as Q
    per = {}

    def tq(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, time.perf_counter() - t0

    # fprop: the first expert whole (its token rows and its 14336 x 4096 weight)
    w = workloads.get("fprop")
    rows, N, K = int(w.sizes[0]), w.n, w.k
    xb = _host_bf16((rows, K), 1.0, w.seed, 0.01, 20.0)
    wb = _host_bf16((N, K), 0.02, w.seed + 1)
    (ad, asc), tqx = tq(lambda: Q.mxfp8_rowwise(xb, np.array([0, rows])))
    (bd, bsc), tqw = tq(lambda: Q.mxfp8_rowwise(wb, np.array([0, N])))
    _, tg = tq(lambda: GM.mxfp8_fprop(ad, asc, bd.reshape(1, N, K), bsc, np.array([0, rows]), K))
    fl = 2.0 * rows * N * K
    qbytes = (rows + N) * K * (2 + 1 + 1 / 32)
    per["fprop"] = {"sample": "expert 0 whole: %d x %d activations, %d x %d weight" % (rows, K, N, K),
                    "quantize_GB_s": round(qbytes / (tqx + tqw) / 1e9, 3),
                    "gemm_GFLOP_s": round(fl / tg / 1e9, 2), "seconds": round(tqx + tqw + tg, 2)}
    head = {"value": round(fl / (tqx + tqw + tg) / 1e12, 6), "seconds": round(tqx + tqw + tg, 2)}

    # wgrad: 1024 tokens of one expert, columnwise copies of dY and X, the NT product
    M, N, K = 1024, 4096, 4096
    dy = _host_bf16((M, N), 1.0, 21)
    x = _host_bf16((M, K), 1.0, 22)
    off, poff = np.array([0, M]), np.array([0, M])
    (dyc, dys), t1 = tq(lambda: Q.mxfp8_colwise(dy, off, poff))
    (xc, xs), t2 = tq(lambda: Q.mxfp8_colwise(x, off, poff))
    _, tg = tq(lambda: GM.mxfp8_wgrad(dyc, dys, xc, xs, poff, N, K))
    per["wgrad"] = {"sample": "1024 tokens of one expert, N = K = 4096",
                    "quantize_GB_s": round(M * (N + K) * (2 + 1 + 1 / 32) / (t1 + t2) / 1e9, 3),
                    "gemm_GFLOP_s": round(2.0 * M * N * K / tg / 1e9, 2),
                    "seconds": round(t1 + t2 + tg, 2)}

    # zipf: 512 rows of one expert against its 2048 x 7168 weight
    M, N, K = 512, 2048, 7168
    xb = _host_bf16((M, K), 1.0, 31)
    wb = _host_bf16((N, K), 0.02, 32)
    (ad, asc), t1 = tq(lambda: Q.mxfp8_rowwise(xb, np.array([0, M])))
    (bd, bsc), t2 = tq(lambda: Q.mxfp8_rowwise(wb, np.array([0, N])))
    _, tg = tq(lambda: GM.mxfp8_fprop(ad, asc, bd.reshape(1, N, K), bsc, np.array([0, M]), K))
    per["zipf"] = {"sample": "512 rows of one expert, K = 7168, N = 2048",
                   "quantize_GB_s": round((M + N) * K * (2 + 1 + 1 / 32) / (t1 + t2) / 1e9, 3),
                   "gemm_GFLOP_s": round(2.0 * M * N * K / tg / 1e9, 2),
                   "seconds": round(t1 + t2 + tg, 2)}

    # dgrad: 512 rows of dY (E5M2) against 512 output columns of one expert's weight
    M, Kc, N = 512, 14336, 512
    dyb = _host_bf16((M, Kc), 1.0, 41)
    wb = _host_bf16((Kc, N), 0.02, 42)
    (dd, ds), t1 = tq(lambda: Q.mxfp8_rowwise(dyb, np.array([0, M]), elem="e5m2"))
    (wd, ws), t2 = tq(lambda: Q.mxfp8_colwise(wb, np.array([0, Kc]), np.array([0, Kc])))
    _, tg = tq(lambda: GM.mxfp8_dgrad(dd, ds, wd, ws, np.array([0, M]), Kc, N))
    per["dgrad"] = {"sample": "512 rows of dY [., 14336] against 512 output columns of one expert",
                    "quantize_GB_s": round((M + N) * Kc * (2 + 1 + 1 / 32) / (t1 + t2) / 1e9, 3),
                    "gemm_GFLOP_s": round(2.0 * M * Kc * N / tg / 1e9, 2),
                    "seconds": round(t1 + t2 + tg, 2)}

    # row-scaled and per-tensor NVFP4: 512 rows against a 2048 x 4096 expert weight
    M, N, K = 512, 2048, 4096
    xb = _host_bf16((M, K), 1.0, 51)
    wb = _host_bf16((N, K), 0.02, 52)
    for name, qf, gf in (("nvfp4", Q.nvfp4_rowscaled, GM.nvfp4_rowscaled_fprop),
                         ("nvfp4_pertensor", Q.nvfp4_pertensor, GM.nvfp4_pertensor_fprop)):
        (a0, a1, a2), t1 = tq(lambda: qf(xb, np.array([0, M])))
        (b0, b1, b2), t2 = tq(lambda: qf(wb, np.array([0, N])))
        _, tg = tq(lambda: gf(a0, a1, a2, np.array([0, M]), b0, b1, b2, [N], K))
        per[name] = {"sample": "512 rows against one 2048 x 4096 expert weight",
                     "quantize_GB_s": round((M + N) * K * (2 + 0.5 + 1 / 16) / (t1 + t2) / 1e9, 3),
                     "gemm_GFLOP_s": round(2.0 * M * N * K / tg / 1e9, 2),
                     "seconds": round(t1 + t2 + tg, 2)}

    # row-scaled NVFP4 wgrad: 512 tokens of one expert, columnwise copies, N = K = 4096
    M, N, K = 512, 4096, 4096
    dy = _host_bf16((M, N), 1.0, 61)
    x = _host_bf16((M, K), 1.0, 62)
    off, poff = np.array([0, M]), np.array([0, M])
    a, t1 = tq(lambda: Q.nvfp4_rowscaled_colwise(dy, off, poff))
    b, t2 = tq(lambda: Q.nvfp4_rowscaled_colwise(x, off, poff))
    _, tg = tq(lambda: GM.nvfp4_rowscaled_wgrad(*a, *b, poff, N, K))
    per["nvfp4_wgrad"] = {"sample": "512 tokens of one expert, N = K = 4096",
                          "quantize_GB_s": round(M * (N + K) * (2 + 0.5 + 1 / 16) / (t1 + t2) / 1e9, 3),
                          "gemm_GFLOP_s": round(2.0 * M * N * K / tg / 1e9, 2),
                          "seconds": round(t1 + t2 + tg, 2)}

    threads = _blas_threads()
    try:
        affinity = len(os.sched_getaffinity(0))
    except Exception:
        affinity = os.cpu_count()
    return {"value": head["value"], "unit": "TFLOP/s", "cores": threads or affinity,
            "kind": "oracle", "seconds": round(sum(v["seconds"] for v in per.values()), 2),
            "sample": "fprop expert 0 whole (%s): oracle MXFP8 rowwise quantize of both operands "
                      "+ fp64 GEMM; per-config samples under per_config" % per["fprop"]["sample"],
            "cpu_model": _cpu_model(), "blas_threads": threads, "host_cpus": affinity,
            "quantize_threads": 1, "per_config": per}


def vendor_reference(dev, iters):
    """Dense GEMMs of the vendor library (hipBLASLt, called through
    torch._scaled_mm) at the fprop shapes, cold cache like the bench: MXFP8
    (E4M3 with one E8M0 scale per 32 along K, unit scales) and per-tensor FP8.
    Context for the grouped kernel's figures, not part of the hot path."""
    flush = torch.ones((512 << 20) // 4, dtype=torch.int32, device=dev)
    gen = torch.Generator(device=dev).manual_seed(7)
    out = {"kind": "vendor reference (hipBLASLt via torch._scaled_mm), dense, bf16 out"}
    for M, N, K in ((16384, 14336, 4096), (3456, 14336, 4096), (8192, 8192, 8192)):
        a = torch.randn((M, K), generator=gen, device=dev).to(torch.float8_e4m3fn)
        b = torch.randn((N, K), generator=gen, device=dev).mul_(1.28).to(torch.float8_e4m3fn)
        unit = lambda r: torch.full((r, K // 32), 127, dtype=torch.uint8,
                                    device=dev).view(torch.float8_e8m0fnu)
        one = torch.ones((), device=dev)
        for name, sa, sb in (("mxfp8", unit(M), unit(N)), ("fp8_per_tensor", one, one)):
            def call():
                return torch._scaled_mm(a, b.t(), scale_a=sa, scale_b=sb, out_dtype=torch.bfloat16)
            key = "%s_%dx%dx%d" % (name, M, N, K)
            try:
                call()
            except Exception as e:  # the vendor library may not offer this path
                out[key] = {"error": repr(e)[:200]}
                continue
            times = []
            for _ in range(max(iters, 10)):
                flush.sum()
                e0 = TimingEvent()
                e1 = TimingEvent()
                e0.record()
                call()
                e1.record()
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            ms = float(np.median(times))
            tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
            out[key] = {"us": round(ms * 1e3, 1), "tflops": round(tf, 1),
                        "frac_of_fp8_peak": round(tf / MFMA_PEAK_TFLOPS["fp8"], 4)}
    return out


# ---------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="time only the headline workload")
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-digests", action="store_true", help="skip the input SHA-256 digests")
    ap.add_argument("--only", default=None, help="comma list of workloads to time")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy (3x), the reference for "
                         "scaling FETCH_SIZE / WRITE_SIZE counter readings")
    ap.add_argument("--vendor-reference", action="store_true",
                    help="only time the vendor library's dense GEMMs (hipBLASLt through "
                         "torch._scaled_mm: MXFP8 with E8M0 scales per 32, and per-tensor FP8) "
                         "at the fprop shapes, as context; prints one JSON line")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.vendor_reference:
        print(json.dumps(vendor_reference(dev, args.steps)))
        return
    bsg.load_library()
    flush = None
    if not args.no_flush:
        flush = torch.ones((512 << 20) // 4, dtype=torch.int32, device=dev)
    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copy calibration: 3 x 268435456 bytes read + written")
        del src, dst

    names = ["fprop"] if args.no_extra else ["fprop", "tiny", "wgrad", "wgrad_e5m2", "zipf", "dgrad",
                                             "nvfp4",
                                             "nvfp4_scratch", "nvfp4_wgrad", "nvfp4_pertensor",
                                             "nvfp4_rht", "nvfp4_2d"]
    if args.only:
        names = args.only.split(",")
    results = {}
    for name in names:
        log("[bench] %s: setup" % name)
        case = make_case(name, dev)
        torch.cuda.synchronize()
        t = time_case(case, args.steps, args.warmup, flush)
        results[name] = summarize(case, t, "bf16" if name.startswith("nvfp4") else "fp8")
        results[name]["steps"] = args.steps
        if not args.no_digests:
            results[name]["input_sha256"] = input_digests(case)
        log("[bench] %s: %s" % (name, json.dumps(results[name])))
        del case
        torch.cuda.empty_cache()
    copy_gbs = device_copy_rate(dev, flush)
    log("[bench] device copy: %.1f GB/s (read + write)" % copy_gbs)

    head = results.get("fprop") or results[names[0]]
    achieved = head["gemm_tflops"]
    qx = head["kernels_us"].get("quantize_x", {})
    # all quantize launches of the step together (X row + col and W rowwise)
    qk = [v for k, v in head["kernels_us"].items() if k.startswith("quantize")]
    q_bytes = sum(v.get("algorithmic_bytes", 0) for v in qk)
    q_us = sum(v["us"] for v in qk)
    q_rate = q_bytes / (q_us * 1e-6) / 1e9 if q_us > 0 else None
    traffic, traffic_src = gemm_traffic() if head is results.get("fprop") else (None, None)
    line = {
        "metric": METRIC,
        "value": head["step_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp8_e4m3 (e8m0/32), fp32 accumulate, bf16 out",
        "data": "synthetic (seeded; no dataset)",
        "config": {"workload": "MoE fprop MXFP8: 8 experts, 16384 routed rows (uneven multiples "
                               "of 128), K=4096, N=14336; step = offsets + quantize X (row+col) + "
                               "quantize W + grouped GEMM",
                   "cache": "cold (a 512 MiB buffer read before each step)" if flush is not None
                   else "warm",
                   "timing": "median over %d steps after %d warm-up steps; HIP events (timing "
                             "only: no system-scope fence) around each kernel on its stream, a "
                             "spin kernel queued ahead of each step"
                             % (args.steps, args.warmup)},
        "targets": {
            "gemm_frac_of_mxfp8_peak": {"value": head["gemm_frac_of_peak"], "target": 0.60},
            "quantize_x_frac_of_hbm": {"value": qx.get("frac_of_hbm"), "target": 0.70,
                                       "what": "grouped activation quantize, rowwise + columnwise "
                                               "in one pass (16384 x 4096 bf16)"},
        },
        "quantize_x_GB_s": qx.get("GB_s"),
        "quantize_x_frac_of_hbm": qx.get("frac_of_hbm"),
        "quantize_xw_GB_s": round(q_rate, 1) if q_rate else None,
        "quantize_xw_frac_of_hbm": round(q_rate / HBM_PEAK_GBS, 4) if q_rate else None,
        "device_copy_GB_s": copy_gbs,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_PEAK_TFLOPS["fp8"], "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_PEAK_TFLOPS["fp8"], 4),
                     "traffic": traffic, "traffic_source": traffic_src,
                     "kernel": "grouped_gemm_mxfp8 (fprop)"},
        "configs": results,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
