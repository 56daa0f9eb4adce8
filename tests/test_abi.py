"""The C ABI library loads without a GPU, exports every symbol include/bsq.h declares, and
rejects bad arguments on the host before any HIP call.

No call here reaches a kernel launch: every call is either invalid (caught by host
validation) or has a zero size (a documented no-op that makes no HIP call), so fake
pointers are safe.
"""
import ctypes
import os
import re

import pytest

import block_scaled_precision_mxfp8_amd as bsq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsq.h")

A = 0x10000          # a 16-byte aligned fake device address
B = 0x20000000
C = 0x40000000
D = 0x60000000
E_ = 0x70000000


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsq.LIB_PATH):
        from block_scaled_precision_mxfp8_amd import build
        build.build()
    return bsq.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\*?\s*([A-Za-z_][A-Za-z_0-9]*)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_expected_entry_points():
    names = _declared_functions()
    for n in ("mx_quantize_mxfp8", "mx_quantize_mxfp8_grouped", "nv_quantize_nvfp4_per_group",
              "nv_dequantize_per_group", "nv_quantize_nvfp4_per_token_scatter",
              "nv_quantize_nvfp4_2d", "nv_dequantize_2d", "nv_quantize_nvfp4_per_token",
              "nv_quantize_nvfp4_per_token_grouped", "mx_dequantize", "nv_dequantize",
              "bsq_status_string", "bsq_abi_version"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in _declared_functions():
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert bsq.abi_version() == 1
    for s in range(0, 8):
        assert bsq.status_string(s) and bsq.status_string(s) != "unknown status"
    assert bsq.status_string(99) == "unknown status"


# ---------------------------------------------------------------------------------------
# mx_quantize_mxfp8

def mxq(L, x=A, M=64, K=64, mode=3, qr=B, sr=C, qc=D, sc=E_):
    return L.mx_quantize_mxfp8(x, M, K, mode, qr, sr, qc, sc, None)


def test_mx_quant_validation(L):
    assert mxq(L, mode=0) == bsq.BSQ_ERR_MODE
    assert mxq(L, mode=4) == bsq.BSQ_ERR_MODE
    assert mxq(L, M=-1) == bsq.BSQ_ERR_SHAPE
    assert mxq(L, K=-32) == bsq.BSQ_ERR_SHAPE
    assert mxq(L, K=48) == bsq.BSQ_ERR_SHAPE                  # K % 32
    assert mxq(L, M=48, mode=3) == bsq.BSQ_ERR_SHAPE          # M % 32 for the columnwise copy
    assert mxq(L, M=48, mode=2) == bsq.BSQ_ERR_SHAPE
    assert mxq(L, M=2 ** 40, K=2 ** 40) == bsq.BSQ_ERR_SHAPE  # size overflow
    assert mxq(L, x=None) == bsq.BSQ_ERR_NULL
    assert mxq(L, mode=1, sr=None) == bsq.BSQ_ERR_NULL
    assert mxq(L, mode=2, qc=None) == bsq.BSQ_ERR_NULL
    assert mxq(L, mode=3, sc=None) == bsq.BSQ_ERR_NULL
    assert mxq(L, x=A + 8) == bsq.BSQ_ERR_ALIGN
    assert mxq(L, qr=B + 4) == bsq.BSQ_ERR_ALIGN
    assert mxq(L, sc=E_ + 1) == bsq.BSQ_ERR_ALIGN
    assert mxq(L, qr=A + 16) == bsq.BSQ_ERR_ALIAS              # output inside the input
    assert mxq(L, qc=B + 64 * 64 - 16) == bsq.BSQ_ERR_ALIAS    # two outputs overlap


def test_mx_quant_zero_sizes_are_noops(L):
    assert mxq(L, M=0) == bsq.BSQ_OK
    assert mxq(L, K=0, x=None, qr=None) == bsq.BSQ_OK
    assert mxq(L, M=0, mode=1, x=None, qr=None, sr=None) == bsq.BSQ_OK


def test_mx_quant_unused_copy_pointers_are_ignored(L):
    # rowwise only: the columnwise pointers may be anything, even misaligned
    assert mxq(L, mode=1, qc=3, sc=5, M=0) == bsq.BSQ_OK
    assert mxq(L, mode=1, qc=3, sc=5, K=48) == bsq.BSQ_ERR_SHAPE


# ---------------------------------------------------------------------------------------
# mx_quantize_mxfp8_grouped

F_ = 0x7F000000


def mxg(L, x=A, M=70, K=64, mode=2, off=E_, E=3, qr=B, sr=C, qc=D, sc=F_, s_ld=5, status=None):
    return L.mx_quantize_mxfp8_grouped(x, M, K, mode, off, E, qr, sr, qc, sc, s_ld, status, None)


def test_mx_grouped_validation(L):
    assert mxg(L, mode=1) == bsq.BSQ_ERR_MODE                 # rowwise: the flat call
    assert mxg(L, mode=0) == bsq.BSQ_ERR_MODE
    assert mxg(L, K=48) == bsq.BSQ_ERR_SHAPE                  # K % 32
    assert mxg(L, M=-1) == bsq.BSQ_ERR_SHAPE
    assert mxg(L, E=0) == bsq.BSQ_ERR_SHAPE
    assert mxg(L, s_ld=2) == bsq.BSQ_ERR_SHAPE                # fewer than ceil(70/32) = 3
    assert mxg(L, M=2 ** 40, s_ld=2 ** 35) == bsq.BSQ_ERR_SHAPE   # 32-bit block indices
    assert mxg(L, off=None) == bsq.BSQ_ERR_NULL
    assert mxg(L, qc=None) == bsq.BSQ_ERR_NULL
    assert mxg(L, mode=3, sr=None) == bsq.BSQ_ERR_NULL
    assert mxg(L, off=E_ + 4) == bsq.BSQ_ERR_ALIGN
    assert mxg(L, status=E_ + 0x1002) == bsq.BSQ_ERR_ALIGN
    assert mxg(L, sc=F_ + 8) == bsq.BSQ_ERR_ALIGN
    assert mxg(L, qc=A + 16) == bsq.BSQ_ERR_ALIAS              # output inside the input
    assert mxg(L, off=F_ + 64) == bsq.BSQ_ERR_ALIAS            # offsets inside s_col
    assert mxg(L, status=D + 8) == bsq.BSQ_ERR_ALIAS           # status inside q_col
    assert mxg(L, M=0, s_ld=0) == bsq.BSQ_OK                   # no status asked: nothing to do
    assert mxg(L, mode=2, qr=3, sr=5, M=0, s_ld=0) == bsq.BSQ_OK   # unused rowwise pointers


# ---------------------------------------------------------------------------------------
# nv quantize (flat and grouped)

def nvq(L, x=A, R=4, K=64, q=B, sb=C, st=D):
    return L.nv_quantize_nvfp4_per_token(x, R, K, q, sb, st, None)


def nvg(L, x=A, R=4, K=64, off=E_, E=2, q=B, sb=C, st=D, status=None):
    return L.nv_quantize_nvfp4_per_token_grouped(x, R, K, off, E, q, sb, st, status, None)


def test_nv_quant_validation(L):
    assert nvq(L, K=24) == bsq.BSQ_ERR_SHAPE
    assert nvq(L, R=-1) == bsq.BSQ_ERR_SHAPE
    assert nvq(L, x=None) == bsq.BSQ_ERR_NULL
    assert nvq(L, st=None) == bsq.BSQ_ERR_NULL
    assert nvq(L, q=B + 2) == bsq.BSQ_ERR_ALIGN
    assert nvq(L, st=D + 4) == bsq.BSQ_ERR_ALIGN
    assert nvq(L, sb=B + 16) == bsq.BSQ_ERR_ALIAS
    assert nvq(L, R=0) == bsq.BSQ_OK
    assert nvq(L, K=0, x=None, q=None) == bsq.BSQ_OK


def test_nv_grouped_validation(L):
    assert nvg(L, E=0) == bsq.BSQ_ERR_SHAPE
    assert nvg(L, E=-3) == bsq.BSQ_ERR_SHAPE
    assert nvg(L, off=None) == bsq.BSQ_ERR_NULL
    assert nvg(L, off=E_ + 4) == bsq.BSQ_ERR_ALIGN
    assert nvg(L, status=E_ + 0x1002) == bsq.BSQ_ERR_ALIGN
    assert nvg(L, off=A + 8) == bsq.BSQ_ERR_ALIAS             # offsets inside the input
    assert nvg(L, status=B) == bsq.BSQ_ERR_ALIAS               # status inside q
    assert nvg(L, K=40) == bsq.BSQ_ERR_SHAPE
    assert nvg(L, R=0) == bsq.BSQ_OK                           # no status asked: nothing to do


def nvpg(L, x=A, R=4, K=64, off=E_, G=2, q=B, sb=C, s=D, status=None):
    return L.nv_quantize_nvfp4_per_group(x, R, K, off, G, q, sb, s, status, None)


def test_nv_per_group_validation(L):
    assert nvpg(L, K=40) == bsq.BSQ_ERR_SHAPE
    assert nvpg(L, R=-2) == bsq.BSQ_ERR_SHAPE
    assert nvpg(L, G=0) == bsq.BSQ_ERR_SHAPE
    assert nvpg(L, off=None) == bsq.BSQ_ERR_NULL
    assert nvpg(L, s=None) == bsq.BSQ_ERR_NULL
    assert nvpg(L, q=None) == bsq.BSQ_ERR_NULL
    assert nvpg(L, off=E_ + 4) == bsq.BSQ_ERR_ALIGN
    assert nvpg(L, s=D + 4) == bsq.BSQ_ERR_ALIGN
    assert nvpg(L, status=E_ + 0x1002) == bsq.BSQ_ERR_ALIGN
    assert nvpg(L, s=A + 16) == bsq.BSQ_ERR_ALIAS              # scales inside the input
    assert nvpg(L, off=C) == bsq.BSQ_ERR_ALIAS                 # offsets inside sb
    f = L.nv_dequantize_per_group
    assert f(A, B, C, D, 2, 4, 40, E_, None) == bsq.BSQ_ERR_SHAPE
    assert f(A, B, C, D, 0, 4, 64, E_, None) == bsq.BSQ_ERR_SHAPE
    assert f(A, B, None, D, 2, 4, 64, E_, None) == bsq.BSQ_ERR_NULL
    assert f(A, B, C, D + 4, 2, 4, 64, E_, None) == bsq.BSQ_ERR_ALIGN
    assert f(A, B, C, D, 2, 4, 64, A + 16, None) == bsq.BSQ_ERR_ALIAS
    assert f(A, B, C, D, 2, 0, 64, E_, None) == bsq.BSQ_OK


def test_nv_2d_validation(L):
    def f(x=A, R=32, K=64, off=E_, G=2, q=B, sb=C, s=D, status=None):
        return L.nv_quantize_nvfp4_2d(x, R, K, off, G, q, sb, s, status, None)
    assert f(R=24) == bsq.BSQ_ERR_SHAPE                        # R % 16
    assert f(K=40) == bsq.BSQ_ERR_SHAPE
    assert f(G=0) == bsq.BSQ_ERR_SHAPE
    assert f(s=None) == bsq.BSQ_ERR_NULL
    assert f(sb=None) == bsq.BSQ_ERR_NULL
    assert f(sb=C + 8) == bsq.BSQ_ERR_ALIGN
    assert f(sb=B + 16) == bsq.BSQ_ERR_ALIAS                   # tile scales inside q
    d = L.nv_dequantize_2d
    assert d(A, B, C, D, 2, 24, 64, E_, None) == bsq.BSQ_ERR_SHAPE
    assert d(A, B, None, D, 2, 32, 64, E_, None) == bsq.BSQ_ERR_NULL
    assert d(A, B, C, D, 2, 32, 64, A + 16, None) == bsq.BSQ_ERR_ALIAS
    assert d(A, B, C, D, 2, 0, 64, E_, None) == bsq.BSQ_OK


def test_nv_scatter_validation(L):
    def f(h=A, T=4, K=64, dst=E_, top_k=2, N=8, q=B, sb=C, st=D, status=None):
        return L.nv_quantize_nvfp4_per_token_scatter(h, T, K, dst, top_k, N, q, sb, st, status, None)
    assert f(K=40) == bsq.BSQ_ERR_SHAPE
    assert f(T=-1) == bsq.BSQ_ERR_SHAPE
    assert f(N=-1) == bsq.BSQ_ERR_SHAPE
    assert f(top_k=0) == bsq.BSQ_ERR_SHAPE
    assert f(h=None) == bsq.BSQ_ERR_NULL
    assert f(dst=None) == bsq.BSQ_ERR_NULL
    assert f(st=None) == bsq.BSQ_ERR_NULL
    assert f(dst=E_ + 4) == bsq.BSQ_ERR_ALIGN
    assert f(q=B + 8) == bsq.BSQ_ERR_ALIGN
    assert f(q=A + 16) == bsq.BSQ_ERR_ALIAS                    # output inside the input
    assert f(dst=C) == bsq.BSQ_ERR_ALIAS                       # map inside sb
    assert f(T=0) == bsq.BSQ_OK                                # nothing to do, no status asked
    assert f(N=0, q=None, sb=None, st=None, T=0) == bsq.BSQ_OK


# ---------------------------------------------------------------------------------------
# dequant

def test_mx_dequant_validation(L):
    f = L.mx_dequantize
    assert f(A, B, 4, 48, C, None) == bsq.BSQ_ERR_SHAPE
    assert f(A, B, -4, 64, C, None) == bsq.BSQ_ERR_SHAPE
    assert f(None, B, 4, 64, C, None) == bsq.BSQ_ERR_NULL
    assert f(A, B, 4, 64, None, None) == bsq.BSQ_ERR_NULL
    assert f(A + 1, B, 4, 64, C, None) == bsq.BSQ_ERR_ALIGN
    assert f(A, A + 16, 4, 64, C, None) == bsq.BSQ_ERR_ALIAS
    assert f(A, B, 4, 64, B - 16, None) == bsq.BSQ_ERR_ALIAS   # y runs into the scales
    assert f(A, B, 0, 64, C, None) == bsq.BSQ_OK


def test_nv_dequant_validation(L):
    f = L.nv_dequantize
    assert f(A, B, C, 4, 40, D, None) == bsq.BSQ_ERR_SHAPE
    assert f(A, B, None, 4, 64, D, None) == bsq.BSQ_ERR_NULL
    assert f(A, B, C + 4, 4, 64, D, None) == bsq.BSQ_ERR_ALIGN
    assert f(A, B, C, 4, 64, A + 16, None) == bsq.BSQ_ERR_ALIAS
    assert f(A, B, C, 0, 64, D, None) == bsq.BSQ_OK


def test_binding_refuses_cpu_tensors_without_calling_the_library():
    import torch
    x = torch.zeros(32, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        bsq.mx_quantize_mxfp8(x, "both")
    with pytest.raises(ValueError):
        bsq.nv_quantize_nvfp4_per_token(x)
    with pytest.raises(ValueError):
        bsq.mx_quantize_mxfp8(x, "bogus")


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: without the built library the binding raises instead of computing
    anything another way."""
    monkeypatch.setattr(bsq, "_lib", None)
    monkeypatch.setattr(bsq, "LIB_PATH", str(tmp_path / "libbsq.so"))
    with pytest.raises(ImportError, match="not built"):
        bsq.lib()


# Random argument sets with exactly one defect each (a property test of the host validation):
# the call must return that defect's status before any launch.
from hypothesis import given, settings, strategies as st  # noqa: E402

_MX_REQUIRED = {1: ("qr", "sr"), 2: ("qc", "sc"), 3: ("qr", "sr", "qc", "sc")}


@st.composite
def _mx_defective_call(draw):
    mode = draw(st.sampled_from([1, 2, 3]))
    M = 32 * draw(st.integers(1, 64))
    K = 32 * draw(st.integers(1, 64))
    args = dict(x=A, M=M, K=K, mode=mode, qr=B, sr=C, qc=D, sc=E_)
    defect = draw(st.sampled_from(["mode", "k_mod", "m_mod", "neg", "null", "align", "alias"]))
    if defect == "mode":
        args["mode"] = draw(st.sampled_from([0, 4, 5, -1, 7]))
        want = bsq.BSQ_ERR_MODE
    elif defect == "k_mod":                             # rowwise/dual: K % 32; columnwise: K % 8
        d = draw(st.integers(1, 31))
        args["K"] = K + (d if mode != 2 or d % 8 else d + 1)
        want = bsq.BSQ_ERR_SHAPE
    elif defect == "m_mod":
        args["mode"] = draw(st.sampled_from([2, 3]))
        args["M"] = M + draw(st.integers(1, 31))
        want = bsq.BSQ_ERR_SHAPE
    elif defect == "neg":
        key = draw(st.sampled_from(["M", "K"]))
        args[key] = -draw(st.integers(1, 1 << 20))
        want = bsq.BSQ_ERR_SHAPE
    elif defect == "null":
        key = draw(st.sampled_from(("x",) + _MX_REQUIRED[mode]))
        args[key] = None
        want = bsq.BSQ_ERR_NULL
    elif defect == "align":
        key = draw(st.sampled_from(("x",) + _MX_REQUIRED[mode]))
        args[key] += draw(st.integers(1, 15))
        want = bsq.BSQ_ERR_ALIGN
    else:                                              # an output inside the input or another output
        key = draw(st.sampled_from(_MX_REQUIRED[mode]))
        other = draw(st.sampled_from([k for k in ("x",) + _MX_REQUIRED[mode] if k != key]))
        args[key] = args[other] + 16 * draw(st.integers(0, 1))   # every buffer here is >= 32 bytes
        want = bsq.BSQ_ERR_ALIAS
    return args, want


@settings(max_examples=400, deadline=None)
@given(_mx_defective_call())
def test_mx_quant_rejects_every_single_defect(L, call):
    args, want = call
    assert mxq(L, **args) == want, args


def test_mx_colwise_needs_only_m_multiple_of_32_and_16_byte_rows(L):
    """The columnwise copy's blocks run along M, so K only has to give 16-byte rows
    (K % 8 == 0); the rowwise and dual modes keep K % 32 == 0.  Zero M: nothing launches."""
    for K in (8, 40, 72, 6184):
        assert mxq(L, M=0, K=K, mode=2) == bsq.BSQ_OK, K
        assert mxq(L, M=0, K=K, mode=1) == bsq.BSQ_ERR_SHAPE, K
        assert mxq(L, M=0, K=K, mode=3) == bsq.BSQ_ERR_SHAPE, K
    for K in (4, 36, 6180):
        assert mxq(L, M=0, K=K, mode=2) == bsq.BSQ_ERR_SHAPE, K
    assert mxq(L, M=48, K=40, mode=2) == bsq.BSQ_ERR_SHAPE      # M % 32 still applies


def test_calls_too_large_for_one_launch_are_shape_errors(L):
    """A launch holds fewer than 2^32 threads and the dequantizers split a tensor into row
    ranges of at most 2^31 half blocks; sizes beyond either are rejected before any launch
    (the host sizes only, no memory behind the fake pointers)."""
    big = 2 ** 26
    # per-token NVFP4: 64 threads a row above K = 768, 32 at or below
    assert L.nv_quantize_nvfp4_per_token(A, big, 1024, B, C, D, None) == bsq.BSQ_ERR_SHAPE
    assert L.nv_quantize_nvfp4_per_token(A, 2 * big, 768, B, C, D, None) == bsq.BSQ_ERR_SHAPE
    assert L.nv_quantize_nvfp4_per_token_grouped(A, big, 1024, E_, 1, B, C, D, None, None) == bsq.BSQ_ERR_SHAPE
    assert L.nv_quantize_nvfp4_per_token_scatter(A, big, 1024, E_, 1, 16, B, C, D, None, None) == bsq.BSQ_ERR_SHAPE
    assert L.nv_quantize_nvfp4_per_group(A, big, 1024, E_, 1, B, C, D, None, None) == bsq.BSQ_ERR_SHAPE
    assert L.nv_quantize_nvfp4_2d(A, 2 ** 22, 2 ** 16, E_, 1, B, C, D, None, None) == bsq.BSQ_ERR_SHAPE
    # MXFP8: rowwise one thread per 64 elements, dual one per 128, dequant one per 16
    assert mxq(L, M=2 ** 22, K=2 ** 16, mode=1) == bsq.BSQ_ERR_SHAPE
    assert mxq(L, M=2 ** 23, K=2 ** 16, mode=3) == bsq.BSQ_ERR_SHAPE
    assert L.mx_dequantize(A, B, 2 ** 20, 2 ** 16, C, None) == bsq.BSQ_ERR_SHAPE
    assert L.mx_quantize_mxfp8_grouped(A, 2 ** 23, 2 ** 16, 2, E_, 1, B, C, D, F_, 2 ** 18, None,
                                       None) == bsq.BSQ_ERR_SHAPE
    # dequantizers: K / 8 half blocks of a row within one range (whole 16-row tiles for 2-D)
    assert L.nv_dequantize(A, B, C, 0, 2 ** 34, D, None) == bsq.BSQ_OK
    assert L.nv_dequantize(A, B, C, 0, 2 ** 35, D, None) == bsq.BSQ_ERR_SHAPE
    assert L.nv_dequantize_per_group(A, B, C, E_, 1, 0, 2 ** 35, D, None) == bsq.BSQ_ERR_SHAPE
    assert L.nv_dequantize_2d(A, B, C, E_, 1, 0, 2 ** 30, D, None) == bsq.BSQ_OK
    assert L.nv_dequantize_2d(A, B, C, E_, 1, 0, 2 ** 31, D, None) == bsq.BSQ_ERR_SHAPE
    assert L.nv_dequantize_2d(A, B, C, E_, 1, 16, 2 ** 31, D, None) == bsq.BSQ_ERR_SHAPE
