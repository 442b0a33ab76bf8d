"""The C-ABI library (CPU only: no compute calls).

The built library must load and export every function the public header declares, with no
torch types in the signatures; the Python binding must declare a matching signature for each.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8_quant_grouped.h")
LIB = os.path.join(ROOT, "fp8_quantization_grouped_amd", "libfp8qg.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_hot_path():
    names = declared_functions()
    for must in ("fp8_quant_rowwise", "fp8_quant_rowwise_gather", "fp8_quant_colwise_grouped",
                 "fp8_grouped_gemm",
                 "fp8_mx_quant_rowwise", "fp8_mx_quant_colwise", "fp8_mx_grouped_gemm",
                 "fp8_mx_grouped_gemm_wgrad",
                 "fp8_quant_colwise_grouped_workspace_size", "fp8_grouped_gemm_workspace_size",
                 "fp8q_status_string", "fp8q_abi_version", "fp8_status_string",
                 "fp8_abi_version"):
        assert must in names
    text = open(HEADER).read()
    assert "torch" not in re.sub(r"/\*.*?\*/", "", text, flags=re.S)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_symbol():
    import fp8_quantization_grouped_amd as fq
    assert sorted(fq.SIGNATURES) == declared_functions()


def test_host_only_calls(lib):
    for ver, txt in (("fp8q_abi_version", "fp8q_status_string"),
                     ("fp8_abi_version", "fp8_status_string")):
        getattr(lib, ver).restype = ctypes.c_int
        assert getattr(lib, ver)() == 2
        f = getattr(lib, txt)
        f.restype = ctypes.c_char_p
        f.argtypes = [ctypes.c_int]
        assert f(0) == b"ok"
        assert f(3) == b"workspace too small"
        assert f(99) == b"unknown status"
    ws = lib.fp8_grouped_gemm_workspace_size
    ws.restype = ctypes.c_size_t
    ws.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    assert ws(0, 16384, 2048, 7168, 32) >= 8 and ws(1, 16384, 2048, 7168, 32) >= 8
    f = lib.fp8_quant_colwise_grouped_workspace_size
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]
    assert f(16384, 7168, 32) == 32 * 7168 * 4
    assert f(10, 3, 1) == 256
    assert f(10, -1, 1) == 0


def test_argument_errors_are_caught_on_the_host(lib):
    """Invalid arguments return a status before any device work (no GPU needed)."""
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    f = lib.fp8_quant_rowwise
    f.restype = I
    f.argtypes = [P, I64, I64, I64, I, P, I64, P, P]
    dummy = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation
    assert f(dummy, -1, 8, 8, 1, dummy, 8, dummy, None) == 1
    assert f(dummy, 4, 8, 4, 1, dummy, 8, dummy, None) == 1
    assert f(dummy, 4, 8, 8, 2, dummy, 8, dummy, None) == 1
    assert f(dummy, 0, 8, 8, 1, dummy, 8, dummy, None) == 0  # empty: no-op
    gq = lib.fp8_quant_rowwise_gather
    gq.restype = I
    gq.argtypes = [P, I64, I64, I64, P, I64, I, P, I64, P, P]
    assert gq(dummy, 0, 8, 8, dummy, 4, 1, dummy, 8, dummy, None) == 1   # no source rows
    assert gq(dummy, 4, 8, 8, None, 4, 1, dummy, 8, dummy, None) == 1    # no index
    assert gq(dummy, 4, 8, 8, dummy, -1, 1, dummy, 8, dummy, None) == 1
    assert gq(dummy, 0, 8, 8, None, 0, 1, dummy, 8, dummy, None) == 0    # empty: no-op
    g = lib.fp8_grouped_gemm
    g.restype = I
    SZ = ctypes.c_size_t
    g.argtypes = [I, I, P, I64, P, P, I64, I64, P, P, ctypes.c_int32, I64, I64, I64, P, I64, I, P,
                  SZ, P]
    ws = ctypes.c_void_p(256)  # 4-byte aligned, never dereferenced either
    assert g(5, 1, dummy, 16, dummy, dummy, 16, 0, dummy, dummy, 1, 4, 4, 16, dummy, 4, 0, ws, 256,
             None) == 1  # unknown mode
    assert g(0, 1, dummy, 16, dummy, dummy, 16, 0, dummy, dummy, 0, 4, 4, 16, dummy, 4, 0, ws, 256,
             None) == 1  # no groups
    assert g(1, 1, dummy, 16, dummy, dummy, 16, 16, dummy, dummy, 1, 4, 4, 16, dummy, 4, 0, ws,
             256, None) == 1  # wgrad needs b_group_stride == 0
    assert g(0, 1, dummy, 16, dummy, dummy, 16, 0, dummy, dummy, 1, 4, 4, 16, dummy, 4, 2, ws, 256,
             None) == 1  # unknown output type
    assert g(0, 1, dummy, 16, dummy, dummy, 16, 0, dummy, dummy, 1, 4, 4, 16, dummy, 4, 0, None,
             256, None) == 3  # no workspace
    assert g(0, 1, dummy, 16, dummy, dummy, 16, 0, dummy, dummy, 1, 4, 4, 16, dummy, 4, 0, ws, 8,
             None) == 3  # workspace too small
    assert g(0, 1, dummy, 16, dummy, dummy, 16, 0, dummy, dummy, 1, 0, 4, 16, dummy, 4, 1, ws, 256,
             None) == 0  # M == 0: no-op
    assert g(0, 1, dummy, 16, dummy, dummy, 16, 0, dummy, dummy, 1, 4, 4, 8, dummy, 4, 0, ws, 256,
             None) == 2  # K not a multiple of 16
    mw = lib.fp8_mx_grouped_gemm_wgrad
    mw.restype = I
    mw.argtypes = [P, I64, P, I64, P, I64, P, I64, P, ctypes.c_int32, I64, I64, I64, P, I64, I, P,
                   SZ, P]
    assert mw(dummy, 48, dummy, 2, dummy, 48, dummy, 2, dummy, 1, 48, 16, 16, dummy, 16, 0, ws,
              256, None) == 1  # M not a multiple of 32
    assert mw(dummy, 64, dummy, 1, dummy, 64, dummy, 2, dummy, 1, 64, 16, 16, dummy, 16, 0, ws,
              256, None) == 1  # scale rows shorter than M/32
    assert mw(dummy, 64, dummy, 2, dummy, 64, dummy, 2, dummy, 1, 64, 0, 16, dummy, 16, 0, ws,
              256, None) == 0  # N == 0: no-op
    assert mw(dummy, 64, dummy, 2, dummy, 64, dummy, 2, dummy, 1, 64, 16, 16, dummy, 16, 0, ws,
              100, None) == 3  # workspace too small


def test_device_code_has_no_generic_memory_instructions():
    """Every device access is written against LDS or global memory explicitly (no flat
    instructions, whose LDS/global routing follows the aperture of the base register)."""
    from fp8_quantization_grouped_amd import _build
    srcs = sorted(os.listdir(os.path.join(ROOT, "fp8_quantization_grouped_amd", "csrc")))
    names = [s[:-4] for s in srcs if s.endswith(".hip")]
    missing = [n for n in names if not os.path.exists(_build.device_asm(n))]
    if missing:
        pytest.skip(f"device assembly not kept for {missing} (run __graft_entry__.build())")
    for n in names:
        text = open(_build.device_asm(n)).read()
        assert "amdgcn" in text
        hits = _build.FLAT_INSN.findall(text)
        assert not hits, (n, hits[:4])


def test_binding_fails_loudly_without_the_library(monkeypatch):
    """No fallback: with the HIP library absent every entry point raises, and host tensors are
    rejected instead of being computed on the CPU."""
    import torch
    import fp8_quantization_grouped_amd as fq
    x = torch.zeros((4, 8), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        fq.fp8_quant_rowwise(x, fq.E4M3FN)
    monkeypatch.setattr(fq, "_lib", None)
    monkeypatch.setattr(fq, "LIB_PATH", os.path.join(os.path.dirname(fq.LIB_PATH), "absent.so"))
    with pytest.raises(RuntimeError, match="missing"):
        fq.lib()
