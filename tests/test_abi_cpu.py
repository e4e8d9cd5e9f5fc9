"""The C-ABI library loads without a GPU, exports every entry point include/bsg.h
declares, and rejects bad arguments on the host before any HIP call (no
compute calls here)."""

import ctypes
import os
import re

import pytest

import block_scaled_grouped_amd as bsg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsg.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|size_t|const char\*)\s+(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bsg.LIB_PATH):
        pytest.fail("libbsg.so is not built; run python -m block_scaled_grouped_amd.build")
    return bsg.load_library()


def test_exports_match_header(lib):
    declared = _declared_functions()
    assert set(declared) == set(bsg.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.bsg_version() >= 1


def _buf(n=4096):
    # host buffers aligned to 16 bytes stand in for device pointers: the calls
    # below must fail validation before dereferencing or launching anything
    raw = ctypes.create_string_buffer(n + 16)
    addr = (ctypes.addressof(raw) + 15) & ~15
    return raw, ctypes.c_void_p(addr)


def test_offsets_validation(lib):
    _, p = _buf()
    assert lib.group_offsets_i32_to_i64(None, 4, 1, 1, None, p, 0, None, None) == 1
    assert lib.group_offsets_i32_to_i64(p, 0, 1, 1, None, p, 0, None, None) == 2
    assert lib.group_offsets_i32_to_i64(p, 257, 1, 1, None, p, 0, None, None) == 2
    assert lib.group_offsets_i32_to_i64(p, 4, 0, 1, None, p, 0, None, None) == 2
    assert lib.group_offsets_i32_to_i64(p, 4, 1, 0, None, p, 0, None, None) == 2
    lib.group_offsets_i32_to_i64(p, 0, 1, 1, None, p, 0, None, None)
    assert b"G=0" in lib.bsg_last_error()


def test_quantize_validation(lib):
    _, p = _buf()
    q = lib.grouped_quantize_mxfp8
    assert q(None, 128, 128, 4, p, p, p, None, 0, None, None, None, None) == 1
    assert q(p, 128, 128, 4, p, None, None, None, 0, None, None, None, None) == 1   # nothing requested
    assert q(p, 128, 128, 4, p, p, None, None, 0, None, None, None, None) == 1      # half a pair
    assert q(p, 128, 100, 4, p, p, p, None, 0, None, None, None, None) == 2         # cols % 32
    assert q(p, 128, 128, 0, p, p, p, None, 0, None, None, None, None) == 2         # G
    mis = ctypes.c_void_p(p.value + 2)
    assert q(mis, 128, 128, 4, p, p, p, None, 0, None, None, None, None) == 3       # alignment
    n = lib.grouped_quantize_nvfp4_rowscaled
    assert n(p, 128, 128, 4, p, p, p, None, None, None) == 1
    assert n(p, 128, 48, 4, p, p, p, p, None, None) == 2
    assert n(p, 128, 0, 4, p, p, p, p, None, None) == 2
    assert n(p, -1, 128, 4, p, p, p, p, None, None) == 2
    t = lib.grouped_quantize_nvfp4_pertensor
    assert t(p, 128, 128, 4, p, p, p, None, None, None) == 1                        # amax
    assert t(p, 128, 48, 4, p, p, p, p, None, None) == 2
    assert t(p, 128, 128, 0, p, p, p, p, None, None) == 2
    assert t(p, 128, 16400, 4, p, p, p, p, None, None) == 2                      # cols % 32
    assert t(p, 128, 128, 4, p, mis, p, p, None, None) == 3


def test_gemm_validation(lib):
    _, p = _buf()
    g = lib.grouped_gemm_mxfp8
    assert g(0, 4, None, p, p, p, p, 128, 128, 128, p, 0, None, None) == 1
    assert g(7, 4, p, p, p, p, p, 128, 128, 128, p, 0, None, None) == 4
    assert g(0, 4, p, p, p, p, p, 128, 128, 128, p, 9, None, None) == 4
    assert g(0, 4, p, p, p, p, p, 128, 128, 100, p, 0, None, None) == 2            # fprop k % 32
    assert g(2, 4, p, p, p, p, p, 128, 128, 48, p, 0, None, None) == 2             # dgrad k % 32
    assert g(0, 4, p, p, p, p, p, 128, 128, 0, p, 0, None, None) == 2
    assert g(1, 4, p, p, p, p, p, 128, 100, 128, p, 0, None, None) == 2            # wgrad n % 32
    assert g(0, 300, p, p, p, p, p, 128, 128, 128, p, 0, None, None) == 2
    need = lib.grouped_gemm_mxfp8_workspace_size()
    assert need >= 16384 + 256 * 1024                # header and at least one 256 KiB part
    wsg = lib.grouped_gemm_mxfp8_ws
    big, wsp = _buf(4096 + 256)
    wsa = ctypes.c_void_p((wsp.value + 255) & ~255)
    assert wsg(0, 4, p, p, p, p, p, 128, 128, 128, p, 0, None, need, None, None) == 1     # NULL
    assert wsg(0, 4, p, p, p, p, p, 128, 128, 128, p, 0, wsa, need - 1, None, None) == 5  # small
    assert wsg(0, 4, p, p, p, p, p, 128, 128, 128, p, 0, ctypes.c_void_p(wsa.value + 16), need,
               None, None) == 3                                                        # aligned
    assert wsg(0, 4, p, p, p, p, p, 128, 128, 100, p, 0, wsa, need, None, None) == 2      # k % 32
    nv = lib.grouped_gemm_nvfp4_rowscaled
    npg = (ctypes.c_int64 * 2)(64, 128)
    hp = ctypes.cast(npg, ctypes.c_void_p)
    assert nv(2, p, p, p, p, 64, 128, p, p, p, None, p, 128, 0, None, None, None) == 1
    assert nv(2, p, p, p, p, 64, 48, p, p, p, hp, p, 128, 0, None, None, None) == 2   # k % 32
    assert nv(2, p, p, p, p, 64, 0, p, p, p, hp, p, 128, 0, None, None, None) == 2
    assert nv(2, p, p, p, p, 64, 128, p, p, p, hp, p, 100, 0, None, None, None) == 2  # ld_out
    pt = lib.grouped_gemm_nvfp4_pertensor
    assert pt(2, p, p, None, p, 64, 128, p, p, p, hp, p, 128, 0, None, None) == 1
    assert pt(2, p, p, p, p, 64, 80, p, p, p, hp, p, 128, 0, None, None) == 2       # k % 32
    assert pt(2, p, p, p, p, 64, 128, p, p, p, hp, p, 100, 0, None, None) == 2      # ld_out
    assert pt(2, p, p, p, p, 64, 128, p, p, p, hp, p, 128, 5, None, None) == 4      # out_dtype
    ex = lib.grouped_gemm_nvfp4_rowscaled_ex
    assert ex(2, p, p, p, p, 64, 128, p, p, p, hp, p, 128, 0, None, 2, None, None) == 4  # flag
    nneed = lib.grouped_gemm_nvfp4_workspace_size()
    assert nneed >= 16384 + 256 * 1024
    nws = lib.grouped_gemm_nvfp4_rowscaled_ws
    assert nws(2, p, p, p, p, 64, 128, p, p, p, hp, p, 128, 0, 0, None, nneed, None, None) == 1
    assert nws(2, p, p, p, p, 64, 128, p, p, p, hp, p, 128, 0, 0, wsa, nneed - 1, None, None) == 5
    assert nws(2, p, p, p, p, 64, 128, p, p, p, hp, p, 128, 0, 0,
               ctypes.c_void_p(wsa.value + 64), nneed, None, None) == 3
    assert nws(2, p, p, p, p, 64, 128, p, p, p, hp, p, 128, 0, 2, wsa, nneed, None, None) == 4
    assert nws(2, p, p, p, p, 64, 48, p, p, p, hp, p, 128, 0, 0, wsa, nneed, None, None) == 2
    pws = lib.grouped_gemm_nvfp4_pertensor_ws
    assert pws(2, p, p, p, p, 64, 128, p, p, p, hp, p, 128, 0, None, nneed, None, None) == 1
    assert pws(2, p, p, p, p, 64, 128, p, p, p, hp, p, 128, 0, wsa, nneed - 1, None, None) == 5
    assert pws(2, p, p, p, p, 64, 80, p, p, p, hp, p, 128, 0, wsa, nneed, None, None) == 2
    assert ex(2, p, p, p, p, 64, 48, p, p, p, hp, p, 128, 0, None, 1, None, None) == 2   # k % 32
    wx = lib.grouped_gemm_nvfp4_rowscaled_wgrad_ex
    assert wx(2, p, p, p, p, p, p, p, 256, 128, 128, p, 0, -1, None, None) == 4          # flag
    neg = (ctypes.c_int64 * 2)(64, -1)
    assert nv(2, p, p, p, p, 64, 128, p, p, p, ctypes.cast(neg, ctypes.c_void_p), p, 128, 0,
              None, None, None) == 2


def test_binding_requires_library(monkeypatch, tmp_path):
    monkeypatch.setattr(bsg, "_lib", None)
    with pytest.raises(RuntimeError):
        bsg.load_library(str(tmp_path / "missing.so"))


def test_product_path_never_touches_the_oracle():
    """Nothing under block_scaled_grouped_amd/ (binding, build, HIP sources) may
    import, load or name the CPU oracle package."""
    pkg = os.path.join(ROOT, "block_scaled_grouped_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"\boracle\b", text), os.path.join(dirpath, f)


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _prototypes():
    """(name, [(type, arg name)]) of every function include/bsg.h declares."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = []
    for m in re.finditer(r"\b(?:int|size_t|const char\*)\s+(\w+)\s*\(([^)]*)\)\s*;", text):
        params = [p.strip() for p in m.group(2).replace("\n", " ").split(",") if p.strip()]
        if params == ["void"]:
            params = []
        args = []
        for p in params:
            t, name = re.match(r"(.*?)(\w+)$", p).groups()
            args.append((t.strip(), name))
        out.append((m.group(1), args))
    return out


_SIZES = {"G": 2, "rows_cap": 256, "cols": 128, "n": 128, "k": 128, "ld_out": 256,
          "col_rows_cap": 512, "multiplier": 1, "pad_to": 1, "capacity": 0}


def _call(lib, name, args, G, ptr):
    vals = []
    for t, a in args:
        if "*" in t:
            vals.append(ptr)
        elif a == "G":
            vals.append(G)
        else:
            vals.append(_SIZES.get(a, 0))
    return getattr(lib, name)(*vals)


def test_every_entry_point_validates_before_any_hip_call(lib):
    """Every compute entry point returns a host validation error -- not success,
    and not BSG_ERR_HIP (this container has no GPU, so a HIP call would fail
    with it) -- when given NULL buffers, and when given G outside [1, 256] with
    buffers present (host memory stands in for them: nothing may be read but
    the [host] arrays, which hold zeros)."""
    raw, p = _buf(1 << 16)
    seen = 0
    for name, args in _prototypes():
        if not any("*" in t for t, _ in args):
            continue                               # version, last error, workspace queries
        rc = _call(lib, name, args, 2, None)
        assert rc in (1, 2, 3, 4, 5), (name, rc, lib.bsg_last_error())
        if any(a == "G" for _, a in args):
            for G in (0, 257):
                rc = _call(lib, name, args, G, p)
                assert rc in (1, 2, 3, 4, 5), (name, G, rc, lib.bsg_last_error())
        seen += 1
    assert seen >= 20, seen
