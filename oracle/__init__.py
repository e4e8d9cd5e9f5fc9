"""CPU oracle for the grouped block-scaled quantize and the grouped block-scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything in this package: it is used by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, and nowhere else.  It shares no
code, table or constant generator with the HIP library under
``block_scaled_grouped_amd/``; neither side imports the other.

What it computes, written plainly and slowly (numpy, float64 unless a step is
defined in float32):

* ``formats``   -- the E8M0, E4M3 and E2M1 element/scale codecs.
* ``offsets``   -- int32 group sizes -> int64 sizes and exclusive prefix-sum offsets.
* ``layout``    -- the byte layout the quantizers write and the GEMMs read
                   (the GEMM-ready scale order, written by the quantize itself).
* ``quantize``  -- grouped MXFP8 rowwise / columnwise quantize (E4M3, and E5M2 for
                   gradients), the row-scaled NVFP4 quantize (rows and columnwise
                   copies) and the per-tensor (per-expert) NVFP4 quantize, also
                   with a randomized Hadamard transform along the contraction
                   and with 2-D (16 x 16) block scales.
* ``rht``       -- the randomized Hadamard transform of 16-element blocks.
* ``gemm``      -- per-expert dense products of the dequantized operands in fp64:
                   fprop (TN, ragged rows), wgrad (NT, ragged contraction), dgrad,
                   the row-scaled NVFP4 fprop / wgrad with their outer-scale
                   epilogue, the per-tensor NVFP4 fprop (alpha per group) and the
                   per-group epilogue terms (alpha, beta, bias).

Sources (the pages): "gemm.py" of TransformerEngine's JAX cpp_extensions
(``grouped_gemm``, ``_quantize_gemm_operands``, ``_jax_scaled_matmul``,
``_get_nvfp4_tensor_scale_inv``); "[JAX] MXFP8 Grouped Quant+GEMM" (PR #2763:
description and review threads); "[Common][PyTorch] Add row-scaled NVFP4 support
to grouped-tensor GEMM" (PR #3661: description, Greptile findings, commit
messages).  Where the pages leave a step open, the reading taken is stated at
the function that takes it.

Parity unpinned by the pages (pinned instead by the OCP MX / NVFP4 format
definitions, closed forms and brute force in ``tests/test_oracle_*.py``):
the E8M0 exponent rule, the NVFP4 float32 operation order, the GEMM-ready
scale byte order, the RHT's size and float32 butterfly order, and the 2-D
block shape.
"""

from . import formats, offsets, layout, quantize, gemm, rht  # noqa: F401
