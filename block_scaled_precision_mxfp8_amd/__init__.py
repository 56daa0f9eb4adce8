"""Bit-exact block-scaled quantization (MXFP8, per-token NVFP4) for AMD MI355X (gfx950).

Thin Python binding of ``libbsq.so`` (C ABI in ``include/bsq.h``).  Each function has the
name of the C entry point it calls and only marshals arguments: it checks tensor
metadata, allocates outputs with PyTorch when the caller does not pass them, and passes
device pointers plus the current HIP stream.  Every step of the computation runs in the
library's HIP kernels; there is no fallback of any kind, and a missing library is an
error.

Layouts (all row-major, all on the GPU):
  MXFP8 rowwise     q_row u8 [M, K]      s_row u8 [M, K/32]   (E4M3 / E8M0)
  MXFP8 columnwise  q_col u8 [K, M]      s_col u8 [K, M/32]   (stored transposed)
  MXFP8 grouped     q_col u8 [K, M]      s_col u8 [K, s_ld]   (32x1 blocks per expert)
  NVFP4 per token   q u8 [R, K/2]        sb u8 [R, K/16]      st f32 [R]
  NVFP4 per group   q u8 [R, K/2]        sb u8 [R, K/16]      s_group f32 [G]
  NVFP4 16x16 tiles q u8 [R, K/2]        sb u8 [R/16, K/16]   s_group f32 [G]
BF16 tensors are ``torch.bfloat16``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsq.so")

BSQ_OK = 0
BSQ_ERR_NULL = 1
BSQ_ERR_SHAPE = 2
BSQ_ERR_ALIGN = 3
BSQ_ERR_MODE = 4
BSQ_ERR_ALIAS = 5
BSQ_ERR_OFFSETS = 6
BSQ_ERR_HIP = 7

MX_ROWWISE = 1
MX_COLWISE = 2
MX_BOTH = 3

_MODES = {"rowwise": MX_ROWWISE, "colwise": MX_COLWISE, "both": MX_BOTH,
          MX_ROWWISE: MX_ROWWISE, MX_COLWISE: MX_COLWISE, MX_BOTH: MX_BOTH}


class BsqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: status %d (%s)" % (fn, status, status_string(status)))


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded libbsq.so.  Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libbsq.so is not built (expected at %s); run "
                "`python -m block_scaled_precision_mxfp8_amd.build` or __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.mx_quantize_mxfp8.restype = I32
        L.mx_quantize_mxfp8.argtypes = [P, I64, I64, I32, P, P, P, P, P]
        L.nv_quantize_nvfp4_per_token.restype = I32
        L.nv_quantize_nvfp4_per_token.argtypes = [P, I64, I64, P, P, P, P]
        L.nv_quantize_nvfp4_per_token_grouped.restype = I32
        L.nv_quantize_nvfp4_per_token_grouped.argtypes = [P, I64, I64, P, I64, P, P, P, P, P]
        L.mx_quantize_mxfp8_grouped.restype = I32
        L.mx_quantize_mxfp8_grouped.argtypes = [P, I64, I64, I32, P, I64, P, P, P, P, I64, P, P]
        L.nv_quantize_nvfp4_per_token_scatter.restype = I32
        L.nv_quantize_nvfp4_per_token_scatter.argtypes = [P, I64, I64, P, I64, I64, P, P, P, P, P]
        L.nv_quantize_nvfp4_2d.restype = I32
        L.nv_quantize_nvfp4_2d.argtypes = [P, I64, I64, P, I64, P, P, P, P, P]
        L.nv_dequantize_2d.restype = I32
        L.nv_dequantize_2d.argtypes = [P, P, P, P, I64, I64, I64, P, P]
        L.nv_quantize_nvfp4_per_group.restype = I32
        L.nv_quantize_nvfp4_per_group.argtypes = [P, I64, I64, P, I64, P, P, P, P, P]
        L.nv_dequantize_per_group.restype = I32
        L.nv_dequantize_per_group.argtypes = [P, P, P, P, I64, I64, I64, P, P]
        L.mx_dequantize.restype = I32
        L.mx_dequantize.argtypes = [P, P, I64, I64, P, P]
        L.nv_dequantize.restype = I32
        L.nv_dequantize.argtypes = [P, P, P, I64, I64, P, P]
        L.bsq_status_string.restype = ctypes.c_char_p
        L.bsq_status_string.argtypes = [I32]
        L.bsq_abi_version.restype = I32
        L.bsq_abi_version.argtypes = []
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().bsq_status_string(status).decode()


def abi_version() -> int:
    return lib().bsq_abi_version()


# ---------------------------------------------------------------------------------------

def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(fn: str, status: int) -> None:
    if status != BSQ_OK:
        raise BsqError(fn, status)


def _dev_tensor(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _out(t, name, dtype, shape, like):
    if t is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _dev_tensor(t, name, dtype, shape)
    return t


# ---------------------------------------------------------------------------------------

def mx_quantize_mxfp8(x: torch.Tensor, mode="both", q_row=None, s_row=None, q_col=None,
                      s_col=None, stream=None):
    """MXFP8 of x [M, K] bf16.  mode: "rowwise" | "colwise" | "both" (or MX_* ints).
    Returns (q_row, s_row, q_col, s_col); the copies the mode does not make are None."""
    m = _MODES.get(mode)
    if m is None:
        raise ValueError("unknown mode %r" % (mode,))
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    _dev_tensor(x, "x", torch.bfloat16, (M, K))
    row, col = bool(m & MX_ROWWISE), bool(m & MX_COLWISE)
    if (row and K % 32) or K % 8 or (col and M % 32):
        raise ValueError("MXFP8 needs K % 32 == 0 for the rowwise copy, M % 32 == 0 and "
                         "K % 8 == 0 for the columnwise copy")
    q_row = _out(q_row, "q_row", torch.uint8, (M, K), x) if row else None
    s_row = _out(s_row, "s_row", torch.uint8, (M, K // 32), x) if row else None
    q_col = _out(q_col, "q_col", torch.uint8, (K, M), x) if col else None
    s_col = _out(s_col, "s_col", torch.uint8, (K, M // 32), x) if col else None
    _check("mx_quantize_mxfp8",
           lib().mx_quantize_mxfp8(_ptr(x), M, K, m, _ptr(q_row), _ptr(s_row), _ptr(q_col),
                                   _ptr(s_col), _stream(stream)))
    return q_row, s_row, q_col, s_col


def mx_group_scale_entries(M: int, E: int) -> int:
    """Scale entries per column that any expert offsets of M rows and E experts fit in."""
    return (M + 31 * E) // 32


def mx_quantize_mxfp8_grouped(x: torch.Tensor, expert_offsets: torch.Tensor, mode="colwise",
                              s_ld=None, q_row=None, s_row=None, q_col=None, s_col=None,
                              status=None, stream=None):
    """MXFP8 of x [M, K] bf16 with 32x1 blocks confined to expert segments (expert_offsets
    int64 [E+1] on the GPU).  mode "colwise" | "both".  s_ld defaults to a length that any
    offsets fit in.  Returns (q_row, s_row, q_col, s_col, status); status is a device
    int32 [1] the kernel sets to BSQ_OK or BSQ_ERR_OFFSETS (read it after synchronising)."""
    m = _MODES.get(mode)
    if m not in (MX_COLWISE, MX_BOTH):
        raise ValueError("mode must be 'colwise' or 'both', got %r" % (mode,))
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    M, K = x.shape
    _dev_tensor(x, "x", torch.bfloat16, (M, K))
    if expert_offsets.dim() != 1 or expert_offsets.numel() < 2:
        raise ValueError("expert_offsets must be int64 [E+1] with E >= 1")
    E = expert_offsets.numel() - 1
    _dev_tensor(expert_offsets, "expert_offsets", torch.int64, (E + 1,))
    if K % 32:
        raise ValueError("MXFP8 needs K % 32 == 0")
    if s_ld is None:
        s_ld = mx_group_scale_entries(M, E)
    row = m == MX_BOTH
    q_row = _out(q_row, "q_row", torch.uint8, (M, K), x) if row else None
    s_row = _out(s_row, "s_row", torch.uint8, (M, K // 32), x) if row else None
    q_col = _out(q_col, "q_col", torch.uint8, (K, M), x)
    s_col = _out(s_col, "s_col", torch.uint8, (K, s_ld), x)
    status = _out(status, "status", torch.int32, (1,), x)
    _check("mx_quantize_mxfp8_grouped",
           lib().mx_quantize_mxfp8_grouped(_ptr(x), M, K, m, _ptr(expert_offsets), E,
                                           _ptr(q_row), _ptr(s_row), _ptr(q_col), _ptr(s_col),
                                           s_ld, _ptr(status), _stream(stream)))
    return q_row, s_row, q_col, s_col, status


def nv_quantize_nvfp4_per_token(x: torch.Tensor, q=None, sb=None, st=None, stream=None):
    """Per-token NVFP4 of x [R, K] bf16 -> (q [R, K/2] u8, sb [R, K/16] u8, st [R] f32)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, K = x.shape
    _dev_tensor(x, "x", torch.bfloat16, (R, K))
    if K % 16:
        raise ValueError("NVFP4 needs K % 16 == 0")
    q = _out(q, "q", torch.uint8, (R, K // 2), x)
    sb = _out(sb, "sb", torch.uint8, (R, K // 16), x)
    st = _out(st, "st", torch.float32, (R,), x)
    _check("nv_quantize_nvfp4_per_token",
           lib().nv_quantize_nvfp4_per_token(_ptr(x), R, K, _ptr(q), _ptr(sb), _ptr(st),
                                             _stream(stream)))
    return q, sb, st


def nv_quantize_nvfp4_per_token_grouped(x: torch.Tensor, expert_offsets: torch.Tensor, q=None,
                                        sb=None, st=None, status=None, stream=None):
    """Per-token NVFP4 of rows grouped by expert (expert_offsets int64 [E+1] on the GPU).
    Returns (q, sb, st, status) where status is a device int32 [1] the kernel sets to
    BSQ_OK or BSQ_ERR_OFFSETS (read it only after synchronising)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, K = x.shape
    _dev_tensor(x, "x", torch.bfloat16, (R, K))
    if expert_offsets.dim() != 1 or expert_offsets.numel() < 2:
        raise ValueError("expert_offsets must be int64 [E+1] with E >= 1")
    E = expert_offsets.numel() - 1
    _dev_tensor(expert_offsets, "expert_offsets", torch.int64, (E + 1,))
    if K % 16:
        raise ValueError("NVFP4 needs K % 16 == 0")
    q = _out(q, "q", torch.uint8, (R, K // 2), x)
    sb = _out(sb, "sb", torch.uint8, (R, K // 16), x)
    st = _out(st, "st", torch.float32, (R,), x)
    status = _out(status, "status", torch.int32, (1,), x)
    _check("nv_quantize_nvfp4_per_token_grouped",
           lib().nv_quantize_nvfp4_per_token_grouped(_ptr(x), R, K, _ptr(expert_offsets), E,
                                                     _ptr(q), _ptr(sb), _ptr(st), _ptr(status),
                                                     _stream(stream)))
    return q, sb, st, status


def mx_dequantize(q: torch.Tensor, s: torch.Tensor, y=None, stream=None) -> torch.Tensor:
    """BF16 [rows, cols] from an MXFP8 copy in its stored layout (q [rows, cols],
    s [rows, cols/32]); pass the columnwise copy as (q_col, s_col) to get [K, M]."""
    if q.dim() != 2:
        raise ValueError("q must be 2-D")
    rows, cols = q.shape
    _dev_tensor(q, "q", torch.uint8, (rows, cols))
    if cols % 32:
        raise ValueError("MXFP8 needs the stored last dimension % 32 == 0")
    _dev_tensor(s, "s", torch.uint8, (rows, cols // 32))
    y = _out(y, "y", torch.bfloat16, (rows, cols), q)
    _check("mx_dequantize", lib().mx_dequantize(_ptr(q), _ptr(s), rows, cols, _ptr(y),
                                                _stream(stream)))
    return y


def nv_dequantize(q: torch.Tensor, sb: torch.Tensor, st: torch.Tensor, y=None,
                  stream=None) -> torch.Tensor:
    """BF16 [R, K] from per-token NVFP4 (q [R, K/2], sb [R, K/16], st [R])."""
    if q.dim() != 2:
        raise ValueError("q must be 2-D")
    R, half = q.shape
    K = 2 * half
    _dev_tensor(q, "q", torch.uint8, (R, half))
    if K % 16:
        raise ValueError("NVFP4 needs K % 16 == 0")
    _dev_tensor(sb, "sb", torch.uint8, (R, K // 16))
    _dev_tensor(st, "st", torch.float32, (R,))
    y = _out(y, "y", torch.bfloat16, (R, K), q)
    _check("nv_dequantize", lib().nv_dequantize(_ptr(q), _ptr(sb), _ptr(st), R, K, _ptr(y),
                                                _stream(stream)))
    return y


__all__ = [
    "mx_quantize_mxfp8", "nv_quantize_nvfp4_per_token", "nv_quantize_nvfp4_per_token_grouped",
    "mx_dequantize", "nv_dequantize", "status_string", "abi_version", "lib", "BsqError",
    "MX_ROWWISE", "MX_COLWISE", "MX_BOTH",
]


def nv_quantize_nvfp4_per_group(x: torch.Tensor, group_offsets: torch.Tensor, q=None, sb=None,
                                s_group=None, status=None, stream=None):
    """Standard NVFP4 of x [R, K] bf16 with one FP32 scale per row group (group_offsets
    int64 [G+1] on the GPU; put an expert's gate and up rows in one group).  Returns
    (q [R, K/2], sb [R, K/16], s_group [G] f32, status); status is a device int32 [1] the
    kernel sets to BSQ_OK or BSQ_ERR_OFFSETS (read it after synchronising)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, K = x.shape
    _dev_tensor(x, "x", torch.bfloat16, (R, K))
    if group_offsets.dim() != 1 or group_offsets.numel() < 2:
        raise ValueError("group_offsets must be int64 [G+1] with G >= 1")
    G = group_offsets.numel() - 1
    _dev_tensor(group_offsets, "group_offsets", torch.int64, (G + 1,))
    if K % 16:
        raise ValueError("NVFP4 needs K % 16 == 0")
    q = _out(q, "q", torch.uint8, (R, K // 2), x)
    sb = _out(sb, "sb", torch.uint8, (R, K // 16), x)
    s_group = _out(s_group, "s_group", torch.float32, (G,), x)
    status = _out(status, "status", torch.int32, (1,), x)
    _check("nv_quantize_nvfp4_per_group",
           lib().nv_quantize_nvfp4_per_group(_ptr(x), R, K, _ptr(group_offsets), G, _ptr(q), _ptr(sb),
                                             _ptr(s_group), _ptr(status), _stream(stream)))
    return q, sb, s_group, status


def nv_dequantize_per_group(q: torch.Tensor, sb: torch.Tensor, s_group: torch.Tensor,
                            group_offsets: torch.Tensor, y=None, stream=None) -> torch.Tensor:
    """BF16 [R, K] from NVFP4 with one FP32 scale per row group."""
    if q.dim() != 2:
        raise ValueError("q must be 2-D")
    R, half = q.shape
    K = 2 * half
    _dev_tensor(q, "q", torch.uint8, (R, half))
    if K % 16:
        raise ValueError("NVFP4 needs K % 16 == 0")
    G = group_offsets.numel() - 1
    _dev_tensor(group_offsets, "group_offsets", torch.int64, (G + 1,))
    _dev_tensor(sb, "sb", torch.uint8, (R, K // 16))
    _dev_tensor(s_group, "s_group", torch.float32, (G,))
    y = _out(y, "y", torch.bfloat16, (R, K), q)
    _check("nv_dequantize_per_group",
           lib().nv_dequantize_per_group(_ptr(q), _ptr(sb), _ptr(s_group), _ptr(group_offsets), G, R, K,
                                         _ptr(y), _stream(stream)))
    return y


def nv_quantize_nvfp4_per_token_scatter(h: torch.Tensor, dst_rows: torch.Tensor, n_rows: int, q=None,
                                        sb=None, st=None, status=None, stream=None):
    """Per-token NVFP4 of the routed rows X[dst_rows[t, j]] = h[t] without gathering X:
    each token of h [T, K] bf16 is quantized once and written to its routed rows
    (dst_rows int64 [T, top_k] on the GPU; negative = dropped).  Returns (q [N, K/2],
    sb [N, K/16], st [N], status) for N = n_rows routed rows."""
    if h.dim() != 2 or dst_rows.dim() != 2:
        raise ValueError("h and dst_rows must be 2-D")
    T, K = h.shape
    _dev_tensor(h, "h", torch.bfloat16, (T, K))
    top_k = dst_rows.shape[1]
    _dev_tensor(dst_rows, "dst_rows", torch.int64, (T, top_k))
    if K % 16:
        raise ValueError("NVFP4 needs K % 16 == 0")
    N = int(n_rows)
    q = _out(q, "q", torch.uint8, (N, K // 2), h)
    sb = _out(sb, "sb", torch.uint8, (N, K // 16), h)
    st = _out(st, "st", torch.float32, (N,), h)
    status = _out(status, "status", torch.int32, (1,), h)
    _check("nv_quantize_nvfp4_per_token_scatter",
           lib().nv_quantize_nvfp4_per_token_scatter(_ptr(h), T, K, _ptr(dst_rows), top_k, N, _ptr(q), _ptr(sb),
                                                     _ptr(st), _ptr(status), _stream(stream)))
    return q, sb, st, status


def nv_quantize_nvfp4_2d(x: torch.Tensor, group_offsets: torch.Tensor, q=None, sb=None, s_group=None,
                         status=None, stream=None):
    """NVFP4 of a weight x [R, K] bf16 with one E4M3 scale per 16x16 tile under one FP32
    scale per row group (group_offsets int64 [G+1] on the GPU, multiples of 16).  Returns
    (q [R, K/2], sb [R/16, K/16], s_group [G] f32, status)."""
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    R, K = x.shape
    _dev_tensor(x, "x", torch.bfloat16, (R, K))
    if group_offsets.dim() != 1 or group_offsets.numel() < 2:
        raise ValueError("group_offsets must be int64 [G+1] with G >= 1")
    G = group_offsets.numel() - 1
    _dev_tensor(group_offsets, "group_offsets", torch.int64, (G + 1,))
    if R % 16 or K % 16:
        raise ValueError("16x16 tiles need R % 16 == 0 and K % 16 == 0")
    q = _out(q, "q", torch.uint8, (R, K // 2), x)
    sb = _out(sb, "sb", torch.uint8, (R // 16, K // 16), x)
    s_group = _out(s_group, "s_group", torch.float32, (G,), x)
    status = _out(status, "status", torch.int32, (1,), x)
    _check("nv_quantize_nvfp4_2d",
           lib().nv_quantize_nvfp4_2d(_ptr(x), R, K, _ptr(group_offsets), G, _ptr(q), _ptr(sb), _ptr(s_group),
                                      _ptr(status), _stream(stream)))
    return q, sb, s_group, status


def nv_dequantize_2d(q: torch.Tensor, sb: torch.Tensor, s_group: torch.Tensor, group_offsets: torch.Tensor,
                     y=None, stream=None) -> torch.Tensor:
    """BF16 [R, K] from the 16x16-tile NVFP4 layout."""
    if q.dim() != 2:
        raise ValueError("q must be 2-D")
    R, half = q.shape
    K = 2 * half
    _dev_tensor(q, "q", torch.uint8, (R, half))
    if R % 16 or K % 16:
        raise ValueError("16x16 tiles need R % 16 == 0 and K % 16 == 0")
    G = group_offsets.numel() - 1
    _dev_tensor(group_offsets, "group_offsets", torch.int64, (G + 1,))
    _dev_tensor(sb, "sb", torch.uint8, (R // 16, K // 16))
    _dev_tensor(s_group, "s_group", torch.float32, (G,))
    y = _out(y, "y", torch.bfloat16, (R, K), q)
    _check("nv_dequantize_2d",
           lib().nv_dequantize_2d(_ptr(q), _ptr(sb), _ptr(s_group), _ptr(group_offsets), G, R, K, _ptr(y),
                                  _stream(stream)))
    return y
