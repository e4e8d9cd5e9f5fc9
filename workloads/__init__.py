"""Seeded synthetic MoE workloads (inputs only; none of the method's arithmetic).

Both the HIP path's tests / benchmark and the CPU oracle draw their inputs here.
Group sizes come from numpy ``Generator(PCG64(seed))``; tensors from a seeded
``torch.Generator`` on the requested device (float32 draws rounded to bf16 by
torch's round-to-nearest-even cast), generated in slabs to bound temporary
memory.  The same (config, device) always gives the same bytes.

Configurations (MoE expert-product shapes):

=====  ===========================================================================
tiny   4 experts, sizes [32, 0, 64, 32] (M=128), K=128, N=128; X, W ~ N(0, 1)
fprop  8 experts, K=4096, N=14336, 16384 rows, sizes 128 * Multinomial(128,
       Dirichlet(2)) (uneven multiples of 128); X ~ N(0, 1) with 1% of elements
       x20; W ~ N(0, 0.02)
wgrad  8 experts, dY [16384, 4096], X [16384, 4096]; two experts empty, the rest
       Multinomial(16384, Dirichlet(2)) redrawn until no size is a multiple of 32
zipf   64 experts, K=7168, N=2048, 32768 rows; p_i ~ rank_i^-1.2 over a seeded
       permutation of ranks, the 4 least likely experts empty; X ~ N(0, 1),
       W ~ N(0, 0.02)
nvfp4  8 experts, K=4096, N_e = 2048 (even e) / 4096 (odd e), 16384 live rows of
       a capacity of 18432 (dead rows hold bf16 NaN); Multinomial(16384,
       Dirichlet(2)); X ~ N(0, 1), W_e ~ N(0, 0.02)
nvfp4_wgrad
       the wgrad shapes and size recipe (its own seed) for the row-scaled NVFP4
       weight gradient: dY [16384, 4096], X [16384, 4096] ~ N(0, 1)
dgrad  the fprop experts' data gradient: sizes as fprop (its own seed), dY
       [16384, 14336] ~ N(0, 1), W [8, 14336, 4096] ~ N(0, 0.02); dX [16384, 4096]
nvfp4_pertensor
       the nvfp4 shapes and size recipe (its own seed) for per-tensor NVFP4
       (one outer scale per expert's activations and per expert's weight)
=====  ===========================================================================
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

CONFIG_NAMES = ("tiny", "fprop", "wgrad", "zipf", "nvfp4", "nvfp4_wgrad", "dgrad",
                "nvfp4_pertensor")
SEED_BASE = 1000
BF16_NAN_BITS = 0x7FC0


@dataclass
class Workload:
    name: str
    mode: str                   # "fprop", "wgrad" or "nvfp4"
    sizes: np.ndarray           # int32 [G] live rows (tokens) per expert
    rows_cap: int               # activation rows allocated (>= sum(sizes))
    k: int                      # contraction dim for fprop / nvfp4; X columns for wgrad
    n: int                      # output columns (fprop); dY columns (wgrad); max N_e (nvfp4)
    n_per_group: Optional[List[int]] = None
    seed: int = 0
    x_std: float = 1.0
    x_outlier_p: float = 0.0
    x_outlier_mul: float = 1.0
    w_std: float = 1.0
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def G(self):
        return len(self.sizes)

    @property
    def live_rows(self):
        return int(np.sum(self.sizes))


def _dirichlet_multinomial(rng, total, groups, alpha=2.0):
    p = rng.dirichlet(np.full(groups, alpha))
    return rng.multinomial(total, p)


def group_sizes(name, seed=None):
    """int32 group sizes of a named configuration (numpy PCG64, seeded)."""
    idx = CONFIG_NAMES.index(name)
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + idx if seed is None else seed))
    if name == "tiny":
        s = np.array([32, 0, 64, 32])
    elif name in ("fprop", "dgrad"):
        s = 128 * _dirichlet_multinomial(rng, 128, 8)
    elif name in ("wgrad", "nvfp4_wgrad"):
        empty = rng.choice(8, size=2, replace=False)
        while True:
            live = _dirichlet_multinomial(rng, 16384, 6)
            if np.all(live % 32 != 0):
                break
        s = np.zeros(8, dtype=np.int64)
        s[np.setdiff1d(np.arange(8), empty)] = live
    elif name == "zipf":
        ranks = rng.permutation(64) + 1
        p = ranks.astype(np.float64) ** -1.2
        p[np.argsort(p)[:4]] = 0.0
        s = rng.multinomial(32768, p / p.sum())
    elif name in ("nvfp4", "nvfp4_pertensor"):
        s = _dirichlet_multinomial(rng, 16384, 8)
    else:
        raise KeyError(name)
    return np.asarray(s, dtype=np.int32)


def get(name, seed=None):
    """Workload description (shapes, sizes, distributions) of a named config."""
    idx = CONFIG_NAMES.index(name)
    sd = SEED_BASE + idx if seed is None else seed
    s = group_sizes(name, sd)
    if name == "tiny":
        return Workload(name, "fprop", s, 128, 128, 128, seed=sd)
    if name == "fprop":
        return Workload(name, "fprop", s, 16384, 4096, 14336, seed=sd, x_outlier_p=0.01,
                        x_outlier_mul=20.0, w_std=0.02)
    if name in ("wgrad", "nvfp4_wgrad"):
        return Workload(name, "wgrad", s, 16384, 4096, 4096, seed=sd)
    if name == "zipf":
        return Workload(name, "fprop", s, 32768, 7168, 2048, seed=sd, w_std=0.02)
    if name == "dgrad":
        # k: the contraction (fprop's N), n: dX columns (fprop's K)
        return Workload(name, "dgrad", s, 16384, 14336, 4096, seed=sd, w_std=0.02)
    if name in ("nvfp4", "nvfp4_pertensor"):
        npg = [2048 if e % 2 == 0 else 4096 for e in range(8)]
        return Workload(name, "nvfp4", s, 18432, 4096, 4096, n_per_group=npg, seed=sd, w_std=0.02)
    raise KeyError(name)


def scaled(w: Workload, rows_cap=None, k=None, n=None, sizes=None, n_per_group=None):
    """A smaller copy of a workload with the same distributions (for tests)."""
    import copy
    v = copy.deepcopy(w)
    if sizes is not None:
        v.sizes = np.asarray(sizes, dtype=np.int32)
    v.rows_cap = int(rows_cap) if rows_cap is not None else max(int(np.sum(v.sizes)), 1)
    if k is not None:
        v.k = int(k)
    if n is not None:
        v.n = int(n)
    if n_per_group is not None:
        v.n_per_group = list(n_per_group)
    return v


def _randn_bf16(torch, gen, shape, std, device, outlier_p=0.0, outlier_mul=1.0, slab_rows=4096):
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1, shape[-1]) if len(shape) > 1 else out.view(1, -1)
    for r0 in range(0, flat.shape[0], slab_rows):
        r1 = min(flat.shape[0], r0 + slab_rows)
        t = torch.randn((r1 - r0, flat.shape[1]), generator=gen, device=device,
                        dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        if outlier_p > 0.0:
            mask = torch.rand((r1 - r0, flat.shape[1]), generator=gen, device=device) < outlier_p
            t = torch.where(mask, t * outlier_mul, t)
        flat[r0:r1].copy_(t.to(torch.bfloat16))
    return out


def tensors(w: Workload, device="cpu"):
    """Seeded bf16 tensors of a workload on ``device``.

    fprop: {"x": [rows_cap, k], "w": [G, n, k]}
    wgrad: {"dy": [rows_cap, n], "x": [rows_cap, k]}
    dgrad: {"dy": [rows_cap, k], "w": [G, k, n]}
    nvfp4: {"x": [rows_cap, k], "w": [sum(N_e), k]}
    Rows past sum(sizes) are capacity rows filled with bf16 NaN."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed))
    live = w.live_rows
    out = {}
    if w.mode == "fprop":
        out["x"] = _randn_bf16(torch, gen, (w.rows_cap, w.k), w.x_std, device, w.x_outlier_p,
                               w.x_outlier_mul)
        out["w"] = _randn_bf16(torch, gen, (w.G, w.n, w.k), w.w_std, device)
    elif w.mode == "wgrad":
        out["dy"] = _randn_bf16(torch, gen, (w.rows_cap, w.n), w.x_std, device)
        out["x"] = _randn_bf16(torch, gen, (w.rows_cap, w.k), w.x_std, device)
    elif w.mode == "dgrad":
        out["dy"] = _randn_bf16(torch, gen, (w.rows_cap, w.k), w.x_std, device)
        out["w"] = _randn_bf16(torch, gen, (w.G, w.k, w.n), w.w_std, device)
    elif w.mode == "nvfp4":
        out["x"] = _randn_bf16(torch, gen, (w.rows_cap, w.k), w.x_std, device)
        out["w"] = _randn_bf16(torch, gen, (int(sum(w.n_per_group)), w.k), w.w_std, device)
    for key in ("x", "dy"):
        if key in out and live < w.rows_cap:
            out[key][live:].view(torch.int16).fill_(BF16_NAN_BITS)
    return out


def bf16_bits(t):
    """bf16 torch tensor (any device) -> numpy uint16 bit patterns on the host."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
