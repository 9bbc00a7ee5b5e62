"""C-ABI checks that need no GPU: the library loads, exports every function
include/fp8w8a8.h declares, and rejects invalid arguments on the host before
anything reaches the device (these calls make no HIP call at all)."""
import ctypes
import os
import re

import pytest

import fp8_w8a8_quantized_amd as fp8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8w8a8.h")

OK, INVALID, UNSUPPORTED = 0, 1, 2
NULL = ctypes.c_void_p(0)
P = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fp8.LIB_PATH):
        pytest.skip("library not built")
    return fp8.lib()


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "fp8_quant_workspace_bytes", "fp8_quant_dynamic", "fp8_quant_static",
        "fp8_quant_dynamic_per_row", "fp8_scaled_mm", "fp8_last_error",
        "fp8_norm_quant_workspace_bytes", "fp8_add_rmsnorm_quant_dynamic", "fp8_silu_mul_quant_dynamic",
        "fp8_quant_dynamic_fmt", "fp8_quant_static_fmt", "fp8_quant_dynamic_per_row_fmt", "fp8_scaled_mm_fmt",
        "fp8_linear_workspace_bytes", "fp8_linear_dynamic", "fp8_linear_dynamic_noalloc"])


def test_library_exports_every_declared_function(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(fp8.SIGNATURES) == set(declared_functions())


def test_workspace_size_is_small(lib):
    n = lib.fp8_quant_workspace_bytes()
    assert 0 < n <= 64 * 1024


def _err(lib):
    return lib.fp8_last_error().decode()


def test_quant_dynamic_rejects_bad_arguments(lib):
    f = lib.fp8_quant_dynamic
    assert f(P, -1, 4, 4, P, 4, P, P, NULL) == INVALID
    assert "negative" in _err(lib)
    assert f(P, 2, 4, 3, P, 4, P, P, NULL) == INVALID        # ld_x < cols
    assert f(P, 2, 4, 4, P, 3, P, P, NULL) == INVALID        # ld_q < cols
    assert f(NULL, 2, 4, 4, P, 4, P, P, NULL) == INVALID     # null x
    assert f(P, 2, 4, 4, NULL, 4, P, P, NULL) == INVALID     # null q
    assert f(P, 2, 4, 4, P, 4, NULL, P, NULL) == INVALID     # null scale
    assert f(P, 2, 4, 4, P, 4, P, NULL, NULL) == INVALID     # null workspace
    assert f(P, 2 ** 33, 2 ** 10, 2 ** 10, P, 2 ** 10, P, P, NULL) == UNSUPPORTED


def test_quant_static_and_per_row_reject_bad_arguments(lib):
    assert lib.fp8_quant_static(P, 2, 4, 4, NULL, P, 4, NULL) == INVALID
    assert lib.fp8_quant_static(P, 2, -4, 4, P, P, 4, NULL) == INVALID
    assert lib.fp8_quant_dynamic_per_row(P, 2, 4, 4, P, 4, NULL, NULL) == INVALID
    assert lib.fp8_quant_dynamic_per_row(P, 2, 8, 4, P, 8, P, NULL) == INVALID


def test_scaled_mm_rejects_bad_arguments(lib):
    # the boundary's argument list: a_q, lda, w_q, ldw, s_a, s_w, mode, bias, out, ldo, M, N, K, stream
    f = lib.fp8_scaled_mm
    good = dict(a=P, lda=64, w=P, ldw=64, sa=P, sw=P, mode=0, bias=NULL, out=P, ldo=32, M=4, N=32, K=64)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["a"], a["lda"], a["w"], a["ldw"], a["sa"], a["sw"], a["mode"], a["bias"], a["out"],
                 a["ldo"], a["M"], a["N"], a["K"], NULL)
    assert call(M=-1) == INVALID
    assert call(N=-2) == INVALID
    assert call(K=0) == INVALID
    assert call(lda=63) == INVALID
    assert call(ldw=10) == INVALID
    assert call(ldo=31) == INVALID
    assert call(mode=2) == INVALID and "mode" in _err(lib)
    for p in ("a", "w", "sa", "sw", "out"):
        assert call(**{p: NULL}) == INVALID, p
    assert call(M=2 ** 31) == UNSUPPORTED
    assert call(K=2 ** 30, lda=2 ** 30, ldw=2 ** 30) == UNSUPPORTED
    # empty problems are valid no-ops that launch nothing
    assert call(M=0) == OK
    assert call(N=0, ldo=0) == OK


def test_scaled_mm_signature_is_the_boundarys():
    """fp8_scaled_mm takes (a_q, lda, w_q, ldw, s_a, s_w, mode, bias, out, ldo,
    M, N, K, stream): no accumulation argument between mode and bias."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decl = re.search(r"fp8_status\s+fp8_scaled_mm\s*\((.*?)\);", text, flags=re.S).group(1)
    names = [re.sub(r"[^A-Za-z0-9_]", " ", a).split()[-1] for a in decl.split(",")]
    assert names == ["a_q", "lda", "w_q", "ldw", "s_a", "s_w", "mode", "bias_bf16", "out_bf16", "ldo",
                     "M", "N", "K", "stream"]
    assert len(fp8.SIGNATURES["fp8_scaled_mm"][1]) == 14


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fp8, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fp8, "_lib", None)
    with pytest.raises(fp8.Fp8Error, match="no fallback"):
        fp8.lib()


def test_fused_producers_reject_bad_arguments(lib):
    F = ctypes.c_float
    f = lib.fp8_add_rmsnorm_quant_dynamic
    # h, ld_h, delta, ld_delta, h_out, ld_h_out, rows, cols, eps, y, ld_y, q, ld_q, scale, ws, stream
    assert f(P, 8, P, 8, NULL, 0, 2, 8, F(1e-5), NULL, 0, P, 8, P, P, NULL) == INVALID        # delta without h_out
    assert "h_out" in _err(lib)
    assert f(P, 8, P, 4, P, 8, 2, 8, F(1e-5), NULL, 0, P, 8, P, P, NULL) == INVALID           # ld_delta < cols
    assert f(P, 8, NULL, 0, NULL, 0, 2, 8, F(-1.0), NULL, 0, P, 8, P, P, NULL) == INVALID     # eps < 0
    assert f(P, 8, NULL, 0, NULL, 0, 2, 8, F(float("nan")), NULL, 0, P, 8, P, P, NULL) == INVALID
    assert f(P, 8, NULL, 0, NULL, 0, 2, 8, F(1e-5), P, 4, P, 8, P, P, NULL) == INVALID        # ld_y < cols
    assert f(P, 8, NULL, 0, NULL, 0, 2, 8, F(1e-5), NULL, 0, P, 8, NULL, P, NULL) == INVALID  # null scale
    assert f(P, 8, NULL, 0, NULL, 0, 2, 8, F(1e-5), NULL, 0, P, 8, P, NULL, NULL) == INVALID  # null workspace
    g = lib.fp8_silu_mul_quant_dynamic
    # gu, ld_gu, rows, cols, y, ld_y, q, ld_q, scale, ws, stream
    assert g(P, 12, 2, 8, NULL, 0, P, 8, P, P, NULL) == INVALID     # ld_gu < 2 cols
    assert "2 * cols" in _err(lib)
    assert g(P, 16, 2, 8, NULL, 0, P, 8, NULL, P, NULL) == INVALID  # null scale
    assert g(P, 16, 2, 8, NULL, 0, P, 8, P, NULL, NULL) == INVALID  # null workspace
    assert g(P, 16, -2, 8, NULL, 0, P, 8, P, P, NULL) == INVALID
    assert lib.fp8_norm_quant_workspace_bytes(16384) >= lib.fp8_quant_workspace_bytes() + 8 * 16384


def test_format_arguments_are_validated(lib):
    assert lib.fp8_quant_dynamic_fmt(P, 2, 4, 4, 2, P, 4, P, P, NULL) == INVALID
    assert "format" in _err(lib)
    assert lib.fp8_quant_static_fmt(P, 2, 4, 4, -1, P, P, 4, NULL) == INVALID
    assert lib.fp8_quant_dynamic_per_row_fmt(P, 2, 4, 4, 7, P, 4, P, NULL) == INVALID
    f = lib.fp8_scaled_mm_fmt
    assert f(P, 64, 0, P, 64, 0, P, P, 0, 5, NULL, P, 32, 4, 32, 64, NULL) == INVALID   # accumulation mode
    assert "accumulation" in _err(lib)
    assert f(P, 64, 0, P, 64, 3, P, P, 0, 0, NULL, P, 32, 4, 32, 64, NULL) == INVALID
    assert f(P, 64, 5, P, 64, 1, P, P, 0, 0, NULL, P, 32, 4, 32, 64, NULL) == INVALID
    assert f(P, 63, 1, P, 64, 1, P, P, 0, 0, NULL, P, 32, 4, 32, 64, NULL) == INVALID   # lda < K


def test_linear_dynamic_rejects_bad_arguments(lib):
    f = lib.fp8_linear_dynamic
    good = dict(x=P, ldx=64, w=P, ldw=64, sw=P, mode=1, accum=0, bias=NULL, aq=P, ldaq=64, sa=P, out=P, ldo=32,
                M=4, N=32, K=64, ws=P)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["x"], a["ldx"], a["w"], a["ldw"], a["sw"], a["mode"], a["accum"], a["bias"], a["aq"], a["ldaq"],
                 a["sa"], a["out"], a["ldo"], a["M"], a["N"], a["K"], a["ws"], NULL)
    assert call(M=-1) == INVALID and "negative" in _err(lib)
    assert call(N=-1) == INVALID
    assert call(K=0) == INVALID
    for ld in ("ldx", "ldaq", "ldw"):
        assert call(**{ld: 63}) == INVALID, ld
    assert call(ldo=31) == INVALID
    assert call(mode=3) == INVALID and "mode" in _err(lib)
    assert call(accum=2) == INVALID
    for p in ("x", "w", "sw", "aq", "sa", "out", "ws"):
        assert call(**{p: NULL}) == INVALID, p
    assert call(N=0, ldo=0, sa=NULL) == INVALID    # the scale is an output even with N == 0
    assert call(M=2 ** 31) == UNSUPPORTED
    assert lib.fp8_linear_workspace_bytes() == lib.fp8_quant_workspace_bytes()


def test_linear_noalloc_rejects_bad_arguments(lib):
    """Validation runs before the scratch lookup or any launch (no GPU here)."""
    f = lib.fp8_linear_dynamic_noalloc
    good = dict(x=P, ldx=64, w=P, ldw=64, sw=P, mode=1, accum=0, bias=NULL, aq=P, ldaq=64, sa=P, out=P, ldo=32,
                M=4, N=32, K=64)

    def call(**kw):
        a = dict(good, **kw)
        return f(a["x"], a["ldx"], a["w"], a["ldw"], a["sw"], a["mode"], a["accum"], a["bias"], a["aq"], a["ldaq"],
                 a["sa"], a["out"], a["ldo"], a["M"], a["N"], a["K"], NULL)
    assert call(M=-1) == INVALID and "fp8_linear_dynamic_noalloc" in _err(lib)
    assert call(K=0) == INVALID
    assert call(ldaq=63) == INVALID
    assert call(accum=2) == INVALID
    for p in ("x", "w", "sw", "aq", "sa", "out"):
        assert call(**{p: NULL}) == INVALID, p
    assert call(M=2 ** 31) == UNSUPPORTED
