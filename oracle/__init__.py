"""CPU oracle for the block-scaled quantizer contract (MXFP8, per-token NVFP4, BF16 dequant).

TEST INFRASTRUCTURE ONLY.  The product path (the HIP library and its Python binding)
never imports, links or calls anything in this package; only ``tests/``, the smoke
check in ``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` do.  The oracle
shares no code with the HIP path.

Two implementations live here:

* ``bsq_oracle.c`` -- plain C, OpenMP over rows, binary64 for exact steps and one C
  float operation for each step the contract rounds to binary32.  Wrapped below for
  numpy arrays.  This is the oracle the parity tests compare against.
* ``exact.py`` -- exact-rational (``fractions.Fraction``) brute-force verifier for tiny
  inputs.  It pins the C oracle; it is never timed.
* ``numpy_ref.py`` -- a vectorized numpy re-implementation (binary32 steps as numpy
  float32 operations) that pins the C oracle on the workloads' own tensors, where the
  exact verifier is too slow.

Every function cites the passage of the pages it follows in ``bsq_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "bsq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    """Compile the C oracle into ``oracle/liboracle.so`` with gcc and return its path."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    """Load the compiled oracle, building it first if it has never been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_dec_e4m3.restype = ctypes.c_double
        L.oracle_dec_e4m3.argtypes = [ctypes.c_uint8]
        L.oracle_enc_e4m3.restype = ctypes.c_uint8
        L.oracle_enc_e4m3.argtypes = [ctypes.c_double]
        L.oracle_dec_e2m1.restype = ctypes.c_double
        L.oracle_dec_e2m1.argtypes = [ctypes.c_uint8]
        L.oracle_enc_e2m1.restype = ctypes.c_uint8
        L.oracle_enc_e2m1.argtypes = [ctypes.c_double]
        L.oracle_dec_e8m0.restype = ctypes.c_double
        L.oracle_dec_e8m0.argtypes = [ctypes.c_uint8]
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_rne_bf16.restype = ctypes.c_uint16
        L.oracle_rne_bf16.argtypes = [ctypes.c_double]
        L.oracle_e8m0_code.restype = ctypes.c_uint8
        L.oracle_e8m0_code.argtypes = [ctypes.c_double]
        L.oracle_nv_token_scale.restype = ctypes.c_float
        L.oracle_nv_token_scale.argtypes = [ctypes.c_float]
        L.oracle_nv_block_scale.restype = ctypes.c_uint8
        L.oracle_nv_block_scale.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_nv_block_multiplier.restype = ctypes.c_float
        L.oracle_nv_block_multiplier.argtypes = [ctypes.c_uint8, ctypes.c_float]
        for name in ("oracle_mx_quantize_rowwise", "oracle_mx_quantize_colwise"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [P, I64, I64, P, P]
        L.oracle_mx_quantize_colwise_grouped.restype = None
        L.oracle_mx_quantize_colwise_grouped.argtypes = [P, I64, I64, P, I64, P, P, I64]
        L.oracle_mx_dequantize.restype = None
        L.oracle_mx_dequantize.argtypes = [P, P, I64, I64, P]
        L.oracle_nv_quantize_per_token.restype = None
        L.oracle_nv_quantize_per_token.argtypes = [P, I64, I64, P, P, P]
        L.oracle_nv_quantize_per_group.restype = None
        L.oracle_nv_quantize_per_group.argtypes = [P, I64, I64, P, I64, P, P, P]
        L.oracle_nv_quantize_2d.restype = None
        L.oracle_nv_quantize_2d.argtypes = [P, I64, I64, P, I64, P, P, P]
        L.oracle_nv_dequantize_2d.restype = None
        L.oracle_nv_dequantize_2d.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.oracle_nv_dequantize.restype = None
        L.oracle_nv_dequantize.argtypes = [P, P, P, I64, I64, P]
        for name in ("oracle_enc_e4m3_array", "oracle_enc_e2m1_array", "oracle_rne_bf16_array"):
            getattr(L, name).restype = None
            getattr(L, name).argtypes = [P, I64, P]
        L.oracle_enc_e2m1_f32_range.restype = None
        L.oracle_enc_e2m1_f32_range.argtypes = [ctypes.c_uint32, I64, P]
        L.oracle_rne_bf16_f32_range.restype = None
        L.oracle_rne_bf16_f32_range.argtypes = [ctypes.c_uint32, I64, P]
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_max_threads.argtypes = []
        L.oracle_set_threads.restype = None
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def _as_bf16_bits(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    if x.dtype != np.uint16:
        raise TypeError("BF16 inputs are passed as uint16 bit patterns, got %s" % x.dtype)
    return x


# ---------------------------------------------------------------------------------------
# Scalar codecs
# ---------------------------------------------------------------------------------------

def dec_e4m3(code: int) -> float:
    return lib().oracle_dec_e4m3(code)


def enc_e4m3(v: float) -> int:
    return lib().oracle_enc_e4m3(v)


def dec_e2m1(code: int) -> float:
    return lib().oracle_dec_e2m1(code)


def enc_e2m1(v: float) -> int:
    return lib().oracle_enc_e2m1(v)


def dec_e8m0(code: int) -> float:
    return lib().oracle_dec_e8m0(code)


def bf16_to_float(bits: int) -> float:
    return lib().oracle_bf16_to_double(bits)


def rne_bf16(v: float) -> int:
    return lib().oracle_rne_bf16(v)


def e8m0_code(amax: float) -> int:
    return lib().oracle_e8m0_code(amax)


def nv_token_scale(amax: float) -> float:
    return lib().oracle_nv_token_scale(amax)


def nv_block_scale(amax_b: float, s_t: float) -> int:
    return lib().oracle_nv_block_scale(amax_b, s_t)


def nv_block_multiplier(sb: int, s_t: float) -> float:
    return lib().oracle_nv_block_multiplier(sb, s_t)


def enc_e4m3_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_enc_e4m3_array(_ptr(v), v.size, _ptr(out))
    return out


def enc_e2m1_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_enc_e2m1_array(_ptr(v), v.size, _ptr(out))
    return out


def rne_bf16_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_rne_bf16_array(_ptr(v), v.size, _ptr(out))
    return out


# ---------------------------------------------------------------------------------------
# Tensor-level contract
# ---------------------------------------------------------------------------------------

def mx_quantize_rowwise(x: np.ndarray):
    """MXFP8 1x32 blocks along the last dim of x[M][K] (BF16 bits) -> (q[M][K], s[M][K/32])."""
    x = _as_bf16_bits(x)
    M, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 32), np.uint8)
    lib().oracle_mx_quantize_rowwise(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def mx_quantize_colwise(x: np.ndarray):
    """MXFP8 32x1 blocks down the columns of x[M][K], stored transposed:
    (q_col[K][M], s_col[K][M/32])."""
    x = _as_bf16_bits(x)
    M, K = x.shape
    if M % 32:
        raise ValueError("M must be a multiple of 32")
    q = np.empty((K, M), np.uint8)
    s = np.empty((K, M // 32), np.uint8)
    lib().oracle_mx_quantize_colwise(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def mx_group_blocks(offsets) -> np.ndarray:
    """Per-expert block counts ceil(m_e / 32) of a grouped columnwise copy."""
    m = np.diff(np.asarray(offsets, dtype=np.int64))
    return (m + 31) // 32


def mx_quantize_colwise_grouped(x: np.ndarray, offsets, s_ld=None):
    """Grouped columnwise MXFP8 of x[M][K] over expert segments offsets int64[E+1]: 32x1
    blocks confined to each segment, a partial last block per segment.  Returns
    (q_col[K][M], s_col[K][s_ld], ok); s_ld defaults to the total block count.  ok is
    False (and the arrays None) when the offsets are invalid or s_ld is too small."""
    x = _as_bf16_bits(x)
    M, K = x.shape
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    ok = bool(off.ndim == 1 and off.size >= 2 and off[0] == 0 and off[-1] == M
              and np.all(np.diff(off) >= 0))
    if not ok:
        return None, None, False
    nb = int(mx_group_blocks(off).sum())
    s_ld = nb if s_ld is None else int(s_ld)
    if s_ld < nb:
        return None, None, False
    q = np.empty((K, M), np.uint8)
    s = np.empty((K, s_ld), np.uint8)
    lib().oracle_mx_quantize_colwise_grouped(_ptr(x), M, K, _ptr(off), off.size - 1,
                                             _ptr(q), _ptr(s), s_ld)
    return q, s, True


def mx_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """BF16 bits of DEC(q) * 2^(s-127), blocks of 32 along the stored last dim."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    rows, cols = q.shape
    assert s.shape == (rows, cols // 32)
    y = np.empty((rows, cols), np.uint16)
    lib().oracle_mx_dequantize(_ptr(q), _ptr(s), rows, cols, _ptr(y))
    return y


def nv_quantize_per_token(x: np.ndarray):
    """Per-token NVFP4 of x[R][K] (BF16 bits) -> (q[R][K/2], sb[R][K/16], st[R] float32)."""
    x = _as_bf16_bits(x)
    R, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    q = np.empty((R, K // 2), np.uint8)
    sb = np.empty((R, K // 16), np.uint8)
    st = np.empty((R,), np.float32)
    lib().oracle_nv_quantize_per_token(_ptr(x), R, K, _ptr(q), _ptr(sb), _ptr(st))
    return q, sb, st


def nv_quantize_per_token_grouped(x: np.ndarray, offsets: np.ndarray):
    """Grouped-by-expert per-token NVFP4.  Per-token math is row-local, so the bytes are
    those of the flat call on the concatenated rows; the offsets int64[E+1] must satisfy
    offsets[0] == 0, offsets[E] == R and be non-decreasing (empty experts allowed).
    Returns (q, sb, st, ok)."""
    R = x.shape[0]
    off = np.asarray(offsets, dtype=np.int64)
    ok = bool(off.ndim == 1 and off.size >= 2 and off[0] == 0 and off[-1] == R
              and np.all(np.diff(off) >= 0))
    q, sb, st = nv_quantize_per_token(x)
    return q, sb, st, ok


def nv_quantize_per_token_routed(h: np.ndarray, dst: np.ndarray, n_rows: int):
    """Per-token NVFP4 of the routed rows X[dst[t, j]] = h[t] (negative dst = dropped),
    computed the plain way: gather X, then quantize every row.  Returns (q, sb, st,
    written) where written marks the rows some entry names."""
    h = _as_bf16_bits(h)
    T, K = h.shape
    dst = np.asarray(dst, dtype=np.int64).reshape(T, -1)
    x = np.zeros((n_rows, K), np.uint16)
    written = np.zeros(n_rows, bool)
    for j in range(dst.shape[1]):
        keep = dst[:, j] >= 0
        x[dst[keep, j]] = h[keep]
        written[dst[keep, j]] = True
    q, sb, st = nv_quantize_per_token(x)
    return q, sb, st, written


def nv_quantize_per_group(x: np.ndarray, offsets):
    """Standard NVFP4 with one FP32 scale per row group (a tensor, or an expert's tensor with
    gate and up together): groups are row ranges offsets int64[G+1].  Returns (q[R][K/2],
    sb[R][K/16], s_group[G] float32, ok); ok False (arrays None) for invalid offsets."""
    x = _as_bf16_bits(x)
    R, K = x.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    ok = bool(off.ndim == 1 and off.size >= 2 and off[0] == 0 and off[-1] == R
              and np.all(np.diff(off) >= 0))
    if not ok:
        return None, None, None, False
    G = off.size - 1
    q = np.empty((R, K // 2), np.uint8)
    sb = np.empty((R, K // 16), np.uint8)
    s = np.empty(G, np.float32)
    lib().oracle_nv_quantize_per_group(_ptr(x), R, K, _ptr(off), G, _ptr(q), _ptr(sb), _ptr(s))
    return q, sb, s, True


def nv_quantize_2d(x: np.ndarray, offsets):
    """NVFP4 with 16x16 weight tiles (one E4M3 scale per tile) under one FP32 scale per row
    group.  x[R][K] with R % 16 == K % 16 == 0, every group whole tiles.  Returns
    (q[R][K/2], sb[R/16][K/16], s_group[G] float32, ok); ok False (arrays None) for
    invalid offsets or shapes."""
    x = _as_bf16_bits(x)
    R, K = x.shape
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    ok = bool(R % 16 == 0 and K % 16 == 0 and off.ndim == 1 and off.size >= 2 and off[0] == 0
              and off[-1] == R and np.all(np.diff(off) >= 0) and np.all(off % 16 == 0))
    if not ok:
        return None, None, None, False
    G = off.size - 1
    q = np.empty((R, K // 2), np.uint8)
    sb = np.empty((R // 16, K // 16), np.uint8)
    s = np.empty(G, np.float32)
    lib().oracle_nv_quantize_2d(_ptr(x), R, K, _ptr(off), G, _ptr(q), _ptr(sb), _ptr(s))
    return q, sb, s, True


def nv_dequantize_2d(q: np.ndarray, sb: np.ndarray, s_group: np.ndarray, offsets) -> np.ndarray:
    """BF16 bits of the 16x16-tile NVFP4 layout (see nv_quantize_2d)."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    s = np.ascontiguousarray(s_group, dtype=np.float32)
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    R, half = q.shape
    K = 2 * half
    assert sb.shape == (R // 16, K // 16) and s.shape == (off.size - 1,)
    y = np.empty((R, K), np.uint16)
    lib().oracle_nv_dequantize_2d(_ptr(q), _ptr(sb), _ptr(s), _ptr(off), off.size - 1, R, K, _ptr(y))
    return y


def nv_dequantize(q: np.ndarray, sb: np.ndarray, st: np.ndarray) -> np.ndarray:
    """BF16 bits of RNE_BF16(fl(DEC(q) * DEC(sb) * s_t)) for the per-token NVFP4 layout."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    sb = np.ascontiguousarray(sb, dtype=np.uint8)
    st = np.ascontiguousarray(st, dtype=np.float32)
    R, half = q.shape
    K = 2 * half
    assert sb.shape == (R, K // 16) and st.shape == (R,)
    y = np.empty((R, K), np.uint16)
    lib().oracle_nv_dequantize(_ptr(q), _ptr(sb), _ptr(st), R, K, _ptr(y))
    return y


def enc_e2m1_f32_range(start: int, n: int) -> np.ndarray:
    """E2M1 codes of the binary32 patterns start .. start+n-1 (NaN patterns give 0)."""
    out = np.empty(n, np.uint8)
    lib().oracle_enc_e2m1_f32_range(start, n, _ptr(out))
    return out


def rne_bf16_f32_range(start: int, n: int) -> np.ndarray:
    """BF16 patterns of the binary32 patterns start .. start+n-1 (NaN gives 0x7FC0)."""
    out = np.empty(n, np.uint16)
    lib().oracle_rne_bf16_f32_range(start, n, _ptr(out))
    return out


def max_threads() -> int:
    return lib().oracle_max_threads()


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops (for timing; results do not depend on it)."""
    lib().oracle_set_threads(int(n))
