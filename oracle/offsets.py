"""Group sizes -> int64 sizes and offsets (oracle; test infrastructure only).

"[JAX] MXFP8 Grouped Quant+GEMM", Changes list and the review thread on
``cublaslt_grouped_gemm.cu``: group sizes arrive as int32 and are widened to
int64 with a multiplier; offsets are the exclusive prefix sums
``offsets[0] = 0, offsets[i] = sum_{j<i} first_dims[j] * last_dim`` (G + 1
values).  "gemm.py", ``grouped_gemm``: padding, if any, is part of the group
sizes.  ``pad_to`` is added here (each size rounded up to a multiple of it
before the sum), used for the 128-padded columnwise copies; pad_to = 1 is the
pages' formula.
"""

import numpy as np

STATUS_NEGATIVE_SIZE = 1
STATUS_OVER_CAPACITY = 2


def group_offsets(sizes_i32, multiplier=1, pad_to=1):
    """Returns (sizes_i64, offsets_i64) for int32 group sizes.

    sizes_i64[g] = sizes[g] * multiplier
    offsets[0] = 0, offsets[g + 1] = offsets[g] + roundup(sizes[g], pad_to) * multiplier
    """
    s = np.asarray(sizes_i32, dtype=np.int32).astype(np.int64)
    if np.any(s < 0):
        raise ValueError("negative group size")
    if pad_to < 1 or multiplier < 1:
        raise ValueError("pad_to and multiplier must be >= 1")
    padded = ((s + pad_to - 1) // pad_to) * pad_to
    offsets = np.zeros(len(s) + 1, dtype=np.int64)
    total = 0
    for g in range(len(s)):          # the scan, written out
        total += int(padded[g]) * multiplier
        offsets[g + 1] = total
    return s * multiplier, offsets


def check_capacity(offsets, capacity):
    """The invariant the pages leave commented out: sum(group sizes) <= rows."""
    return int(offsets[-1]) <= int(capacity)
