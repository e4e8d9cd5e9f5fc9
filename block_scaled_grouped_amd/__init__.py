"""Python binding of libbsg (include/bsg.h): block-scaled grouped quantize and
grouped GEMM for MoE expert products on MI355X.

Argument marshalling only.  Every function has the name of its C entry point,
takes torch tensors (device memory) and enqueues on the current torch stream;
outputs the caller does not pass are allocated with torch.  Every step of the
computation runs in the HIP library: if ``libbsg.so`` is missing or fails to
load, every call raises.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsg.so")

BSG_FPROP_TN = 0
BSG_WGRAD_NT = 1
BSG_OUT_BF16 = 0
BSG_OUT_F32 = 1
BSG_DGRAD_NN = 2
BSG_WGRAD_NT_E5M2 = 3
BSG_MAX_GROUPS = 256
BSG_COLWISE_PAD = 128
DEV_NEGATIVE_SIZE = 1
DEV_OVER_CAPACITY = 2
DEV_BAD_PADDING = 4

EXPORTS = ("bsg_last_error", "bsg_version", "group_offsets_i32_to_i64", "grouped_quantize_mxfp8",
           "grouped_quantize_mxfp8_rowwise_e5m2",
           "grouped_quantize_nvfp4_rowscaled", "grouped_quantize_nvfp4_rowscaled_colwise",
           "grouped_quantize_nvfp4_pertensor",
           "grouped_gemm_mxfp8", "grouped_gemm_mxfp8_ex", "grouped_gemm_nvfp4_rowscaled",
           "grouped_gemm_nvfp4_rowscaled_wgrad", "grouped_gemm_nvfp4_pertensor",
           "grouped_gemm_nvfp4_rowscaled_noalloc", "grouped_quantize_nvfp4_pertensor_rht",
           "grouped_quantize_nvfp4_pertensor_2d", "grouped_quantize_mxfp8_colwise_e5m2",
           "grouped_gemm_nvfp4_rowscaled_ex", "grouped_gemm_nvfp4_rowscaled_wgrad_ex",
           "grouped_gemm_mxfp8_workspace_size", "grouped_gemm_mxfp8_ws",
           "grouped_gemm_nvfp4_workspace_size", "grouped_gemm_nvfp4_rowscaled_ws",
           "grouped_gemm_nvfp4_pertensor_ws")
BSG_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


class BsgError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("bsg status %d: %s" % (code, msg))
        self.code = code


def load_library(path=LIB_PATH):
    """Loads libbsg.so once; raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("libbsg.so not built at %s (run python -m block_scaled_grouped_amd.build)"
                           % path)
    lib = ctypes.CDLL(path)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.bsg_last_error.restype = ctypes.c_char_p
    lib.bsg_last_error.argtypes = []
    lib.bsg_version.restype = I32
    lib.bsg_version.argtypes = []
    lib.group_offsets_i32_to_i64.restype = I32
    lib.group_offsets_i32_to_i64.argtypes = [P, I64, I64, I64, P, P, I64, P, P]
    lib.grouped_quantize_mxfp8.restype = I32
    lib.grouped_quantize_mxfp8.argtypes = [P, I64, I64, I64, P, P, P, P, I64, P, P, P, P]
    lib.grouped_quantize_mxfp8_rowwise_e5m2.restype = I32
    lib.grouped_quantize_mxfp8_rowwise_e5m2.argtypes = [P, I64, I64, I64, P, P, P, P, P]
    lib.grouped_quantize_mxfp8_colwise_e5m2.restype = I32
    lib.grouped_quantize_mxfp8_colwise_e5m2.argtypes = [P, I64, I64, I64, P, P, I64, P, P, P, P]
    lib.grouped_quantize_nvfp4_rowscaled.restype = I32
    lib.grouped_quantize_nvfp4_rowscaled.argtypes = [P, I64, I64, I64, P, P, P, P, P, P]
    lib.grouped_quantize_nvfp4_rowscaled_colwise.restype = I32
    lib.grouped_quantize_nvfp4_rowscaled_colwise.argtypes = [P, I64, I64, I64, P, P, I64, P, P, P,
                                                             P, P]
    lib.grouped_gemm_mxfp8.restype = I32
    lib.grouped_gemm_mxfp8.argtypes = [I32, I64, P, P, P, P, P, I64, I64, I64, P, I32, P, P]
    lib.grouped_gemm_mxfp8_workspace_size.restype = ctypes.c_size_t
    lib.grouped_gemm_mxfp8_workspace_size.argtypes = []
    lib.grouped_gemm_mxfp8_ws.restype = I32
    lib.grouped_gemm_mxfp8_ws.argtypes = [I32, I64, P, P, P, P, P, I64, I64, I64, P, I32, P,
                                          ctypes.c_size_t, P, P]
    lib.grouped_gemm_mxfp8_ex.restype = I32
    lib.grouped_gemm_mxfp8_ex.argtypes = [I32, I64, P, P, P, P, P, I64, I64, I64, P, I32, P, P, P,
                                          P, P]
    lib.grouped_gemm_nvfp4_rowscaled.restype = I32
    lib.grouped_gemm_nvfp4_rowscaled.argtypes = [I64, P, P, P, P, I64, I64, P, P, P, P, P, I64, I32,
                                                 P, P, P]
    lib.grouped_quantize_nvfp4_pertensor.restype = I32
    lib.grouped_quantize_nvfp4_pertensor.argtypes = [P, I64, I64, I64, P, P, P, P, P, P]
    lib.grouped_quantize_nvfp4_pertensor_rht.restype = I32
    lib.grouped_quantize_nvfp4_pertensor_rht.argtypes = [P, I64, I64, I64, P, ctypes.c_uint32, P, P,
                                                         P, P, P]
    lib.grouped_quantize_nvfp4_pertensor_2d.restype = I32
    lib.grouped_quantize_nvfp4_pertensor_2d.argtypes = [P, I64, I64, I64, P, P, P, P, P, P]
    lib.grouped_gemm_nvfp4_pertensor.restype = I32
    lib.grouped_gemm_nvfp4_pertensor.argtypes = [I64, P, P, P, P, I64, I64, P, P, P, P, P, I64, I32,
                                                 P, P]
    lib.grouped_gemm_nvfp4_rowscaled_ex.restype = I32
    lib.grouped_gemm_nvfp4_rowscaled_ex.argtypes = [I64, P, P, P, P, I64, I64, P, P, P, P, P, I64,
                                                    I32, P, I32, P, P]
    lib.grouped_gemm_nvfp4_rowscaled_wgrad_ex.restype = I32
    lib.grouped_gemm_nvfp4_rowscaled_wgrad_ex.argtypes = [I64, P, P, P, P, P, P, P, I64, I64, I64,
                                                          P, I32, I32, P, P]
    lib.grouped_gemm_nvfp4_rowscaled_noalloc.restype = I32
    lib.grouped_gemm_nvfp4_rowscaled_noalloc.argtypes = [I64, P, P, P, P, I64, I64, P, P, P, P, P,
                                                         I64, I32, P, P]
    lib.grouped_gemm_nvfp4_workspace_size.restype = ctypes.c_size_t
    lib.grouped_gemm_nvfp4_workspace_size.argtypes = []
    lib.grouped_gemm_nvfp4_rowscaled_ws.restype = I32
    lib.grouped_gemm_nvfp4_rowscaled_ws.argtypes = [I64, P, P, P, P, I64, I64, P, P, P, P, P, I64,
                                                    I32, I32, P, ctypes.c_size_t, P, P]
    lib.grouped_gemm_nvfp4_pertensor_ws.restype = I32
    lib.grouped_gemm_nvfp4_pertensor_ws.argtypes = [I64, P, P, P, P, I64, I64, P, P, P, P, P, I64,
                                                    I32, P, ctypes.c_size_t, P, P]
    lib.grouped_gemm_nvfp4_rowscaled_wgrad.restype = I32
    lib.grouped_gemm_nvfp4_rowscaled_wgrad.argtypes = [I64, P, P, P, P, P, P, P, I64, I64, I64, P,
                                                       I32, P, P]
    _lib = lib
    return lib


def _check(rc):
    if rc != 0:
        raise BsgError(rc, _lib.bsg_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("bsg operates on device tensors")


def _dtype_name(dt):
    return str(dt).replace("torch.", "")


def _req(t, name, nbytes, dtype=None, optional=False):
    """Checks, before anything is launched, that tensor t can hold what the C
    call will touch: a contiguous device tensor of at least nbytes bytes (and of
    the given torch dtype).  A buffer that is too small would otherwise be read
    or written out of bounds on the device."""
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if dtype is not None:
        allowed = dtype if isinstance(dtype, tuple) else (dtype,)
        if t.dtype not in allowed:
            raise ValueError("%s must be %s, not %s" % (
                name, " or ".join(_dtype_name(d) for d in allowed), _dtype_name(t.dtype)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s holds %d bytes; the call touches %d" % (name, have, int(nbytes)))


def _i64():
    import torch
    return torch.int64


def _f32():
    import torch
    return torch.float32


def _bf16_2d(x, name="x"):
    import torch
    if x.dim() != 2:
        raise ValueError("%s must be 2-D [rows, cols]" % name)
    _req(x, name, 0, torch.bfloat16)
    return x.shape


def _out_dtype(out_dtype):
    import torch
    if out_dtype == BSG_OUT_F32:
        return torch.float32, 4
    if out_dtype == BSG_OUT_BF16:
        return torch.bfloat16, 2
    raise ValueError("unknown out_dtype %r" % (out_dtype,))


def mx_scale_row_bytes(cols):
    """Stored E8M0 bytes per row of a rowwise MXFP8 tensor (cols / 32 rounded up to 4)."""
    return ((cols // 32 + 3) // 4) * 4


def mx_scale_shape(rows, cols):
    """Shape of rowwise MXFP8 scales: [NQ][rows] words of 4 bytes, NQ = ceil(cols / 128)."""
    return (mx_scale_row_bytes(cols) // 4, rows, 4)


def group_offsets_i32_to_i64(sizes, multiplier=1, pad_to=1, capacity=0, sizes_i64=None,
                             offsets=None, status=None):
    """int32 [G] sizes -> (int64 [G] sizes * multiplier, int64 [G+1] offsets)."""
    import torch
    lib = load_library()
    _req(sizes, "sizes", 0, torch.int32)
    G = sizes.numel()
    if sizes_i64 is None:
        sizes_i64 = torch.empty(G, dtype=torch.int64, device=sizes.device)
    if offsets is None:
        offsets = torch.empty(G + 1, dtype=torch.int64, device=sizes.device)
    _req(sizes_i64, "sizes_i64", 8 * G, torch.int64)
    _req(offsets, "offsets", 8 * (G + 1), torch.int64)
    _req(status, "status", 4, optional=True)
    _check(lib.group_offsets_i32_to_i64(_ptr(sizes), G, multiplier, pad_to, _ptr(sizes_i64),
                                        _ptr(offsets), capacity, _ptr(status), _stream(sizes)))
    return sizes_i64, offsets


def grouped_quantize_mxfp8(x, offsets, G=None, rowwise=True, padded_offsets=None,
                           col_rows_cap=None, row_data=None, row_scales=None, col_data=None,
                           col_scales=None, status=None):
    """bf16 [rows_cap, cols] -> dict with "row_data"/"row_scales" (rowwise) and
    "col_data"/"col_scales" (when padded_offsets is given), uint8 tensors."""
    import torch
    lib = load_library()
    rows_cap, cols = _bf16_2d(x)
    G = offsets.numel() - 1 if G is None else G
    _req(offsets, "offsets", 8 * (G + 1), _i64())
    out = {}
    if rowwise:
        if row_data is None:
            row_data = torch.empty((rows_cap, cols), dtype=torch.uint8, device=x.device)
        if row_scales is None:
            row_scales = torch.empty(mx_scale_shape(rows_cap, cols), dtype=torch.uint8,
                                     device=x.device)
        out["row_data"], out["row_scales"] = row_data, row_scales
    else:
        row_data = row_scales = None
    if padded_offsets is not None:
        if col_rows_cap is None:
            col_rows_cap = rows_cap + BSG_COLWISE_PAD * G
        if col_data is None:
            col_data = torch.empty(col_rows_cap * cols, dtype=torch.uint8, device=x.device)
        if col_scales is None:
            col_scales = torch.empty(col_rows_cap * cols // 32, dtype=torch.uint8, device=x.device)
        out["col_data"], out["col_scales"] = col_data, col_scales
        out["col_rows_cap"] = col_rows_cap
        _req(padded_offsets, "padded_offsets", 8 * (G + 1), _i64())
        _req(col_data, "col_data", col_rows_cap * cols)
        _req(col_scales, "col_scales", col_rows_cap * cols // 32)
    if rowwise:
        _req(row_data, "row_data", rows_cap * cols)
        _req(row_scales, "row_scales", rows_cap * mx_scale_row_bytes(cols))
    _req(status, "status", 4, optional=True)
    _check(lib.grouped_quantize_mxfp8(_ptr(x), rows_cap, cols, G, _ptr(offsets), _ptr(row_data),
                                      _ptr(row_scales), _ptr(padded_offsets),
                                      col_rows_cap or 0, _ptr(col_data), _ptr(col_scales),
                                      _ptr(status), _stream(x)))
    return out


def grouped_quantize_mxfp8_rowwise_e5m2(x, offsets, G=None, row_data=None, row_scales=None,
                                        status=None):
    """bf16 [rows_cap, cols] gradient -> (E5M2 [rows_cap, cols], E8M0 scale words as
    grouped_quantize_mxfp8's rowwise output)."""
    import torch
    lib = load_library()
    rows_cap, cols = _bf16_2d(x)
    G = offsets.numel() - 1 if G is None else G
    _req(offsets, "offsets", 8 * (G + 1), torch.int64)
    if row_data is None:
        row_data = torch.empty((rows_cap, cols), dtype=torch.uint8, device=x.device)
    if row_scales is None:
        row_scales = torch.empty(mx_scale_shape(rows_cap, cols), dtype=torch.uint8, device=x.device)
    _req(row_data, "row_data", rows_cap * cols)
    _req(row_scales, "row_scales", rows_cap * mx_scale_row_bytes(cols))
    _req(status, "status", 4, optional=True)
    _check(lib.grouped_quantize_mxfp8_rowwise_e5m2(_ptr(x), rows_cap, cols, G, _ptr(offsets),
                                                   _ptr(row_data), _ptr(row_scales), _ptr(status),
                                                   _stream(x)))
    return row_data, row_scales


def grouped_quantize_mxfp8_colwise_e5m2(x, offsets, padded_offsets, G=None, col_rows_cap=None,
                                        col_data=None, col_scales=None, status=None):
    """bf16 [rows_cap, cols] gradient -> its E5M2 columnwise copy (col_data,
    col_scales) in grouped_quantize_mxfp8's columnwise layout."""
    import torch
    lib = load_library()
    rows_cap, cols = _bf16_2d(x)
    G = offsets.numel() - 1 if G is None else G
    _req(offsets, "offsets", 8 * (G + 1), torch.int64)
    _req(padded_offsets, "padded_offsets", 8 * (G + 1), torch.int64)
    if col_rows_cap is None:
        col_rows_cap = rows_cap + BSG_COLWISE_PAD * G
    if col_data is None:
        col_data = torch.empty(col_rows_cap * cols, dtype=torch.uint8, device=x.device)
    if col_scales is None:
        col_scales = torch.empty(col_rows_cap * cols // 32, dtype=torch.uint8, device=x.device)
    _req(col_data, "col_data", col_rows_cap * cols)
    _req(col_scales, "col_scales", col_rows_cap * cols // 32)
    _req(status, "status", 4, optional=True)
    _check(lib.grouped_quantize_mxfp8_colwise_e5m2(_ptr(x), rows_cap, cols, G, _ptr(offsets),
                                                   _ptr(padded_offsets), col_rows_cap,
                                                   _ptr(col_data), _ptr(col_scales), _ptr(status),
                                                   _stream(x)))
    return col_data, col_scales


def grouped_quantize_nvfp4_rowscaled(x, offsets, G=None, data=None, block_scales=None, outer=None,
                                     status=None):
    """bf16 [rows_cap, cols] -> (E2M1 [rows_cap, cols/2], E4M3 [rows_cap, cols/16], f32 [rows_cap])."""
    import torch
    lib = load_library()
    rows_cap, cols = _bf16_2d(x)
    G = offsets.numel() - 1 if G is None else G
    _req(offsets, "offsets", 8 * (G + 1), torch.int64)
    if data is None:
        data = torch.empty((rows_cap, cols // 2), dtype=torch.uint8, device=x.device)
    if block_scales is None:
        block_scales = torch.empty((rows_cap, cols // 16), dtype=torch.uint8, device=x.device)
    if outer is None:
        outer = torch.empty(rows_cap, dtype=torch.float32, device=x.device)
    _req(data, "data", rows_cap * cols // 2)
    _req(block_scales, "block_scales", rows_cap * cols // 16)
    _req(outer, "outer", 4 * rows_cap, torch.float32)
    _req(status, "status", 4, optional=True)
    _check(lib.grouped_quantize_nvfp4_rowscaled(_ptr(x), rows_cap, cols, G, _ptr(offsets),
                                                _ptr(data), _ptr(block_scales), _ptr(outer),
                                                _ptr(status), _stream(x)))
    return data, block_scales, outer


def grouped_quantize_nvfp4_pertensor(x, offsets, G=None, data=None, block_scales=None, amax=None,
                                     status=None):
    """bf16 [rows_cap, cols] -> (E2M1 [rows_cap, cols/2], E4M3 [rows_cap, cols/16], f32 amax [G])."""
    import torch
    lib = load_library()
    rows_cap, cols = _bf16_2d(x)
    G = offsets.numel() - 1 if G is None else G
    _req(offsets, "offsets", 8 * (G + 1), torch.int64)
    if data is None:
        data = torch.empty((rows_cap, cols // 2), dtype=torch.uint8, device=x.device)
    if block_scales is None:
        block_scales = torch.empty((rows_cap, cols // 16), dtype=torch.uint8, device=x.device)
    if amax is None:
        amax = torch.empty(G, dtype=torch.float32, device=x.device)
    _req(data, "data", rows_cap * cols // 2)
    _req(block_scales, "block_scales", rows_cap * cols // 16)
    _req(amax, "amax", 4 * G, torch.float32)
    _req(status, "status", 4, optional=True)
    _check(lib.grouped_quantize_nvfp4_pertensor(_ptr(x), rows_cap, cols, G, _ptr(offsets),
                                                _ptr(data), _ptr(block_scales), _ptr(amax),
                                                _ptr(status), _stream(x)))
    return data, block_scales, amax


def _pertensor_variant(cfn, x, offsets, G, data, block_scales, amax, status, *extra):
    import torch
    rows_cap, cols = _bf16_2d(x)
    G = offsets.numel() - 1 if G is None else G
    _req(offsets, "offsets", 8 * (G + 1), torch.int64)
    if data is None:
        data = torch.empty((rows_cap, cols // 2), dtype=torch.uint8, device=x.device)
    if block_scales is None:
        block_scales = torch.empty((rows_cap, cols // 16), dtype=torch.uint8, device=x.device)
    if amax is None:
        amax = torch.empty(G, dtype=torch.float32, device=x.device)
    _req(data, "data", rows_cap * cols // 2)
    _req(block_scales, "block_scales", rows_cap * cols // 16)
    _req(amax, "amax", 4 * G, torch.float32)
    _req(status, "status", 4, optional=True)
    args = [_ptr(x), rows_cap, cols, G, _ptr(offsets)] + list(extra) + [
        _ptr(data), _ptr(block_scales), _ptr(amax), _ptr(status), _stream(x)]
    _check(cfn(*args))
    return data, block_scales, amax


def grouped_quantize_nvfp4_pertensor_rht(x, offsets, rht_sign_mask, G=None, data=None,
                                         block_scales=None, amax=None, status=None):
    """Per-tensor NVFP4 of the rows' randomized Hadamard transform (16-element
    blocks, signs from the 16-bit mask): outputs as
    grouped_quantize_nvfp4_pertensor.  See include/bsg.h."""
    lib = load_library()
    return _pertensor_variant(lib.grouped_quantize_nvfp4_pertensor_rht, x, offsets, G, data,
                              block_scales, amax, status, ctypes.c_uint32(int(rht_sign_mask)))


def grouped_quantize_nvfp4_pertensor_2d(x, offsets, G=None, data=None, block_scales=None, amax=None,
                                        status=None):
    """Per-tensor NVFP4 with one E4M3 scale per 16 x 16 block (written into each
    row of the block): outputs as grouped_quantize_nvfp4_pertensor.  See
    include/bsg.h."""
    lib = load_library()
    return _pertensor_variant(lib.grouped_quantize_nvfp4_pertensor_2d, x, offsets, G, data,
                              block_scales, amax, status)


def grouped_quantize_nvfp4_rowscaled_colwise(x, offsets, padded_offsets, G=None, col_rows_cap=None,
                                             data=None, block_scales=None, outer=None, status=None):
    """bf16 [rows_cap, cols] -> per-expert transposed copies: (E2M1 bytes
    [col_rows_cap * cols / 2], E4M3 [col_rows_cap * cols / 16], f32 outer [G, cols]).
    See include/bsg.h for the block layout."""
    import torch
    lib = load_library()
    rows_cap, cols = _bf16_2d(x)
    G = offsets.numel() - 1 if G is None else G
    _req(offsets, "offsets", 8 * (G + 1), torch.int64)
    _req(padded_offsets, "padded_offsets", 8 * (G + 1), torch.int64)
    if col_rows_cap is None:
        col_rows_cap = rows_cap + BSG_COLWISE_PAD * G
    if data is None:
        data = torch.empty(col_rows_cap * cols // 2, dtype=torch.uint8, device=x.device)
    if block_scales is None:
        block_scales = torch.empty(col_rows_cap * cols // 16, dtype=torch.uint8, device=x.device)
    if outer is None:
        outer = torch.empty((G, cols), dtype=torch.float32, device=x.device)
    _req(data, "data", col_rows_cap * cols // 2)
    _req(block_scales, "block_scales", col_rows_cap * cols // 16)
    _req(outer, "outer", 4 * G * cols, torch.float32)
    _req(status, "status", 4, optional=True)
    _check(lib.grouped_quantize_nvfp4_rowscaled_colwise(
        _ptr(x), rows_cap, cols, G, _ptr(offsets), _ptr(padded_offsets), col_rows_cap, _ptr(data),
        _ptr(block_scales), _ptr(outer), _ptr(status), _stream(x)))
    return data, block_scales, outer


def _mx_gemm_bytes(mode, G, rows_cap, n, k):
    """Bytes grouped_gemm_mxfp8 reads from a, a_scales, b, b_scales, and the
    output's element count (include/bsg.h gives the layouts)."""
    nq = (k + 127) // 128
    if mode == BSG_FPROP_TN:
        return (rows_cap * k, 4 * nq * rows_cap, G * n * k, 4 * nq * G * n, rows_cap * n)
    if mode == BSG_DGRAD_NN:
        kpad = 128 * nq   # the weights' columnwise copy pads each expert to 128 tokens
        return (rows_cap * k, 4 * nq * rows_cap, G * n * kpad, G * n * kpad // 32, rows_cap * n)
    if mode in (BSG_WGRAD_NT, BSG_WGRAD_NT_E5M2):
        return (rows_cap * n, rows_cap * n // 32, rows_cap * k, rows_cap * k // 32, G * n * k)
    raise ValueError("unknown mode %r" % (mode,))


def _mx_gemm_check(mode, G, a, a_scales, b, b_scales, offsets, rows_cap, n, k, out, out_dtype,
                   status):
    na, nas, nb, nbs, nout = _mx_gemm_bytes(mode, G, rows_cap, n, k)
    _req(a, "a", na)
    _req(a_scales, "a_scales", nas)
    _req(b, "b", nb)
    _req(b_scales, "b_scales", nbs)
    _req(offsets, "offsets", 8 * (G + 1), _i64())
    dt, esz = _out_dtype(out_dtype)
    _req(out, "out", esz * nout, dt)
    _req(status, "status", 4, optional=True)


def gemm_workspace(device=None):
    """A uint8 device tensor of max(grouped_gemm_mxfp8_workspace_size(),
    grouped_gemm_nvfp4_workspace_size()) bytes (256-byte aligned: torch's caching
    allocator aligns blocks to 512), for the `workspace` argument of
    grouped_gemm_mxfp8, grouped_gemm_nvfp4_rowscaled and grouped_gemm_nvfp4_pertensor."""
    import torch
    lib = load_library()
    n = max(int(lib.grouped_gemm_mxfp8_workspace_size()),
            int(lib.grouped_gemm_nvfp4_workspace_size()))
    return torch.empty(n, dtype=torch.uint8, device=device or "cuda")


def grouped_gemm_mxfp8(mode, a, a_scales, b, b_scales, offsets, rows_cap, n, k, out=None,
                       out_dtype=BSG_OUT_BF16, G=None, status=None, workspace=None):
    """FPROP_TN, DGRAD_NN: out [rows_cap, n]; WGRAD_NT: out [G, n, k].  With a
    `workspace` (gemm_workspace()), grouped_gemm_mxfp8_ws: the last round of
    tiles is split along the contraction.  See include/bsg.h."""
    import torch
    lib = load_library()
    _need_cuda(a, a_scales, b, b_scales, offsets)
    G = offsets.numel() - 1 if G is None else G
    if out is None:
        dt = _out_dtype(out_dtype)[0]
        shape = (G, n, k) if mode in (BSG_WGRAD_NT, BSG_WGRAD_NT_E5M2) else (rows_cap, n)
        out = torch.empty(shape, dtype=dt, device=a.device)
    _mx_gemm_check(mode, G, a, a_scales, b, b_scales, offsets, rows_cap, n, k, out, out_dtype,
                   status)
    if workspace is not None:
        _need_cuda(workspace)
        _check(lib.grouped_gemm_mxfp8_ws(mode, G, _ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales),
                                         _ptr(offsets), rows_cap, n, k, _ptr(out), out_dtype,
                                         _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         _ptr(status), _stream(a)))
        return out
    _check(lib.grouped_gemm_mxfp8(mode, G, _ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales),
                                  _ptr(offsets), rows_cap, n, k, _ptr(out), out_dtype, _ptr(status),
                                  _stream(a)))
    return out


def grouped_gemm_mxfp8_ex(mode, a, a_scales, b, b_scales, offsets, rows_cap, n, k, out,
                          out_dtype=BSG_OUT_BF16, alpha=None, beta=None, bias=None, G=None,
                          status=None):
    """grouped_gemm_mxfp8 with out = alpha[g] * S + beta[g] * out + bias[g]
    (float32 [G] alpha / beta, [G, output columns] bias; None = 1 / 0 / none).
    `out` is required (it is read where beta != 0).  See include/bsg.h."""
    lib = load_library()
    _need_cuda(a, a_scales, b, b_scales, offsets, out)
    G = offsets.numel() - 1 if G is None else G
    _mx_gemm_check(mode, G, a, a_scales, b, b_scales, offsets, rows_cap, n, k, out, out_dtype,
                   status)
    _req(alpha, "alpha", 4 * G, _f32(), optional=True)
    _req(beta, "beta", 4 * G, _f32(), optional=True)
    _req(bias, "bias", 4 * G * (k if mode in (BSG_WGRAD_NT, BSG_WGRAD_NT_E5M2) else n), _f32(),
         optional=True)
    _check(lib.grouped_gemm_mxfp8_ex(mode, G, _ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales),
                                     _ptr(offsets), rows_cap, n, k, _ptr(out), out_dtype,
                                     _ptr(alpha), _ptr(beta), _ptr(bias), _ptr(status),
                                     _stream(a)))
    return out


def _nv_gemm_check(G, a, a_scales, a_outer, offsets, rows_cap, k, b, b_scales, b_outer, npg, out,
                   ld_out, out_dtype, status, per_tensor):
    nb = sum(npg)
    _req(a, "a", rows_cap * k // 2)
    _req(a_scales, "a_scales", rows_cap * k // 16)
    _req(a_outer, "a_amax" if per_tensor else "a_outer", 4 * (G if per_tensor else rows_cap),
         _f32())
    _req(offsets, "offsets", 8 * (G + 1), _i64())
    _req(b, "b", nb * k // 2)
    _req(b_scales, "b_scales", nb * k // 16)
    _req(b_outer, "b_amax" if per_tensor else "b_outer", 4 * (G if per_tensor else nb), _f32())
    dt, esz = _out_dtype(out_dtype)
    _req(out, "out", esz * rows_cap * ld_out, dt)
    _req(status, "status", 4, optional=True)


def grouped_gemm_nvfp4_rowscaled(a, a_scales, a_outer, offsets, k, b, b_scales, b_outer,
                                 n_per_group, out=None, ld_out=None, out_dtype=BSG_OUT_BF16,
                                 scratch=None, G=None, status=None, accumulate=False,
                                 workspace=None):
    """Row-scaled NVFP4 fprop: out [rows_cap, ld_out]; n_per_group is a host list.
    accumulate=True adds Y to out's previous contents (grouped_gemm_nvfp4_rowscaled_ex).
    With a `workspace` (gemm_workspace(), fused epilogue only),
    grouped_gemm_nvfp4_rowscaled_ws: the last round of tiles is split along the
    contraction."""
    import torch
    lib = load_library()
    _need_cuda(a, a_scales, a_outer, offsets, b, b_scales, b_outer)
    rows_cap = a.shape[0]
    G = offsets.numel() - 1 if G is None else G
    npg = [int(v) for v in n_per_group]
    if len(npg) != G:
        raise ValueError("n_per_group needs G entries")
    if ld_out is None:
        ld_out = max(npg) if out is None else out.shape[1]
    if out is None:
        dt = _out_dtype(out_dtype)[0]
        out = torch.empty((rows_cap, ld_out), dtype=dt, device=a.device)
    _nv_gemm_check(G, a, a_scales, a_outer, offsets, rows_cap, k, b, b_scales, b_outer, npg, out,
                   ld_out, out_dtype, status, per_tensor=False)
    _req(scratch, "scratch", 4 * rows_cap * ld_out, torch.float32, optional=True)
    host_n = (ctypes.c_int64 * G)(*npg)
    if workspace is not None:
        if scratch is not None:
            raise ValueError("a workspace serves the fused epilogue only (no scratch)")
        _need_cuda(workspace)
        _check(lib.grouped_gemm_nvfp4_rowscaled_ws(
            G, _ptr(a), _ptr(a_scales), _ptr(a_outer), _ptr(offsets), rows_cap, k, _ptr(b),
            _ptr(b_scales), _ptr(b_outer), ctypes.cast(host_n, ctypes.c_void_p), _ptr(out), ld_out,
            out_dtype, 1 if accumulate else 0, _ptr(workspace),
            workspace.numel() * workspace.element_size(), _ptr(status), _stream(a)))
        return out
    if accumulate:
        _check(lib.grouped_gemm_nvfp4_rowscaled_ex(
            G, _ptr(a), _ptr(a_scales), _ptr(a_outer), _ptr(offsets), rows_cap, k, _ptr(b),
            _ptr(b_scales), _ptr(b_outer), ctypes.cast(host_n, ctypes.c_void_p), _ptr(out), ld_out,
            out_dtype, _ptr(scratch), 1, _ptr(status), _stream(a)))
        return out
    _check(lib.grouped_gemm_nvfp4_rowscaled(G, _ptr(a), _ptr(a_scales), _ptr(a_outer),
                                            _ptr(offsets), rows_cap, k, _ptr(b), _ptr(b_scales),
                                            _ptr(b_outer), ctypes.cast(host_n, ctypes.c_void_p),
                                            _ptr(out), ld_out, out_dtype, _ptr(scratch),
                                            _ptr(status), _stream(a)))
    return out


def grouped_gemm_nvfp4_rowscaled_noalloc(a, a_scales, a_outer, offsets, k, b, b_scales, b_outer,
                                         n_per_group, out, ld_out=None, out_dtype=BSG_OUT_BF16,
                                         G=None, status=None):
    """grouped_gemm_nvfp4_rowscaled's two-step (FP32 S) flow with S in the
    library's static device scratch: allocates nothing, so `out` is required.
    rows_cap * ld_out * 4 must fit BSG_NOALLOC_SCRATCH_BYTES; calls that overlap
    on one GPU race.  See include/bsg.h."""
    lib = load_library()
    _need_cuda(a, a_scales, a_outer, offsets, b, b_scales, b_outer, out)
    rows_cap = a.shape[0]
    G = offsets.numel() - 1 if G is None else G
    npg = [int(v) for v in n_per_group]
    if len(npg) != G:
        raise ValueError("n_per_group needs G entries")
    if ld_out is None:
        ld_out = out.shape[1]
    _nv_gemm_check(G, a, a_scales, a_outer, offsets, rows_cap, k, b, b_scales, b_outer, npg, out,
                   ld_out, out_dtype, status, per_tensor=False)
    host_n = (ctypes.c_int64 * G)(*npg)
    _check(lib.grouped_gemm_nvfp4_rowscaled_noalloc(
        G, _ptr(a), _ptr(a_scales), _ptr(a_outer), _ptr(offsets), rows_cap, k, _ptr(b),
        _ptr(b_scales), _ptr(b_outer), ctypes.cast(host_n, ctypes.c_void_p), _ptr(out), ld_out,
        out_dtype, _ptr(status), _stream(a)))
    return out


def grouped_gemm_nvfp4_pertensor(a, a_scales, a_amax, offsets, k, b, b_scales, b_amax, n_per_group,
                                 out=None, ld_out=None, out_dtype=BSG_OUT_BF16, G=None,
                                 status=None, workspace=None):
    """Per-tensor NVFP4 fprop (alpha per group from the two amax arrays): out
    [rows_cap, ld_out]; n_per_group is a host list.  With a `workspace`
    (gemm_workspace()), grouped_gemm_nvfp4_pertensor_ws: the last round of tiles
    is split along the contraction."""
    import torch
    lib = load_library()
    _need_cuda(a, a_scales, a_amax, offsets, b, b_scales, b_amax)
    rows_cap = a.shape[0]
    G = offsets.numel() - 1 if G is None else G
    npg = [int(v) for v in n_per_group]
    if len(npg) != G:
        raise ValueError("n_per_group needs G entries")
    if ld_out is None:
        ld_out = max(npg) if out is None else out.shape[1]
    if out is None:
        dt = _out_dtype(out_dtype)[0]
        out = torch.empty((rows_cap, ld_out), dtype=dt, device=a.device)
    _nv_gemm_check(G, a, a_scales, a_amax, offsets, rows_cap, k, b, b_scales, b_amax, npg, out,
                   ld_out, out_dtype, status, per_tensor=True)
    host_n = (ctypes.c_int64 * G)(*npg)
    if workspace is not None:
        _need_cuda(workspace)
        _check(lib.grouped_gemm_nvfp4_pertensor_ws(
            G, _ptr(a), _ptr(a_scales), _ptr(a_amax), _ptr(offsets), rows_cap, k, _ptr(b),
            _ptr(b_scales), _ptr(b_amax), ctypes.cast(host_n, ctypes.c_void_p), _ptr(out), ld_out,
            out_dtype, _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(status),
            _stream(a)))
        return out
    _check(lib.grouped_gemm_nvfp4_pertensor(G, _ptr(a), _ptr(a_scales), _ptr(a_amax),
                                            _ptr(offsets), rows_cap, k, _ptr(b), _ptr(b_scales),
                                            _ptr(b_amax), ctypes.cast(host_n, ctypes.c_void_p),
                                            _ptr(out), ld_out, out_dtype, _ptr(status),
                                            _stream(a)))
    return out


def grouped_gemm_nvfp4_rowscaled_wgrad(a, a_scales, a_outer, b, b_scales, b_outer, padded_offsets,
                                       n, k, col_rows_cap=None, out=None, out_dtype=BSG_OUT_BF16,
                                       G=None, status=None, accumulate=False):
    """Row-scaled NVFP4 wgrad from the columnwise copies: out [G, n, k];
    accumulate=True adds to out's previous contents
    (grouped_gemm_nvfp4_rowscaled_wgrad_ex).  See include/bsg.h."""
    import torch
    lib = load_library()
    _need_cuda(a, a_scales, a_outer, b, b_scales, b_outer, padded_offsets)
    G = padded_offsets.numel() - 1 if G is None else G
    if col_rows_cap is None:
        col_rows_cap = a.numel() * 2 // n
    if out is None:
        dt = _out_dtype(out_dtype)[0]
        out = torch.empty((G, n, k), dtype=dt, device=a.device)
    _req(a, "a", col_rows_cap * n // 2)
    _req(a_scales, "a_scales", col_rows_cap * n // 16)
    _req(a_outer, "a_outer", 4 * G * n, torch.float32)
    _req(b, "b", col_rows_cap * k // 2)
    _req(b_scales, "b_scales", col_rows_cap * k // 16)
    _req(b_outer, "b_outer", 4 * G * k, torch.float32)
    _req(padded_offsets, "padded_offsets", 8 * (G + 1), torch.int64)
    dt, esz = _out_dtype(out_dtype)
    _req(out, "out", esz * G * n * k, dt)
    _req(status, "status", 4, optional=True)
    if accumulate:
        _check(lib.grouped_gemm_nvfp4_rowscaled_wgrad_ex(
            G, _ptr(a), _ptr(a_scales), _ptr(a_outer), _ptr(b), _ptr(b_scales), _ptr(b_outer),
            _ptr(padded_offsets), col_rows_cap, n, k, _ptr(out), out_dtype, 1, _ptr(status),
            _stream(a)))
        return out
    _check(lib.grouped_gemm_nvfp4_rowscaled_wgrad(
        G, _ptr(a), _ptr(a_scales), _ptr(a_outer), _ptr(b), _ptr(b_scales), _ptr(b_outer),
        _ptr(padded_offsets), col_rows_cap, n, k, _ptr(out), out_dtype, _ptr(status), _stream(a)))
    return out
