"""Second implementation of the block-scaled quantizer contract in vectorized numpy.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): it pins the C oracle at the sizes of
the workloads, where the exact-rational verifier (``exact.py``) is far too slow.  It shares
no code with the C oracle or the HIP library: the format tables are built here from the
bit fields, "nearest value, ties to the even code" is a sorted-table search, every step
the contract states as one binary32 operation is one numpy float32 operation (IEEE,
round to nearest even, no fused multiply-add, subnormals kept), and exact steps are done
in float64, where every value involved is exact.

Passages followed (the page "Towards Blackwell-native 8-bit and 4-bit RL"):
* section "Format background": MXFP8 blocks of 32 E4M3 values with one E8M0 scale rounded
  up so the block maximum never clips; NVFP4 E2M1 values, one E4M3 scale per 16 values
  rounded to nearest, and a coarse FP32 scale whose scope is a recipe choice.
* section "Recipe 1: end-to-end MXFP8 RL": rowwise 1x32 and columnwise 32x1 copies, each
  from the BF16 input.
* section "Per-token activation scaling": one FP32 scale per token (row).
* section "High-precision and dequantized backward": BF16 dequantized operands.
The readings where the pages are silent are the ones the C oracle's header lists.
"""
from __future__ import annotations

import numpy as np

# ------------------------------------------------------------------ format tables

def _e4m3_table() -> np.ndarray:
    """Magnitudes of the E4M3 codes 0x00 .. 0x7E (0x7F is NaN), increasing."""
    out = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        out.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out, np.float64)


E4M3 = _e4m3_table()
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
FLT_MAX = np.float32(np.finfo(np.float32).max)


def _nearest(table: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Index of the table value nearest to a >= 0 (float64), ties to the even index;
    values beyond the last entry take the last one."""
    lo = np.searchsorted(table, a, side="right") - 1          # table[lo] <= a
    lo = np.clip(lo, 0, table.size - 1)
    hi = np.minimum(lo + 1, table.size - 1)
    dlo, dhi = a - table[lo], table[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0) & (hi != lo))
    return np.where(pick_hi, hi, lo)


def _encoder_tables(table: np.ndarray, sign: int):
    """Codes of every binary32 value by its top 16 bits.  Every boundary between two codes (a
    midpoint of neighbouring table values) is a value whose low 16 binary32 bits are zero,
    so a value whose low bits are zero takes the code of its top 16 bits read as a value
    (`exact`), and any other value the code of a point strictly inside the interval above
    that (`above`): no boundary lies inside the interval.  Both are found by the search
    above; NaN patterns are never looked up."""
    top = np.arange(1 << 16, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        lo_val = (top << 16).view(np.float32).astype(np.float64)
        step = (((top << 16) | 0x8000).view(np.float32).astype(np.float64))  # inside the interval
    mags = []
    for a in (np.abs(lo_val), np.abs(step)):
        a = np.where(np.isnan(a), 0.0, a)
        mags.append(_nearest(table, a).astype(np.uint8))
    neg = (top >> 15).astype(bool)
    return [np.where(neg, m | np.uint8(sign), m).astype(np.uint8) for m in mags]


_E4M3_EXACT, _E4M3_ABOVE = _encoder_tables(E4M3, 0x80)
_E2M1_EXACT, _E2M1_ABOVE = _encoder_tables(E2M1, 0x8)


def _encode(v: np.ndarray, exact: np.ndarray, above: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    top = u >> 16
    return np.where((u & 0xFFFF) == 0, exact[top], above[top])


def enc_e4m3(v: np.ndarray) -> np.ndarray:
    """E4M3 codes of binary32 values (not NaN): nearest finite value, ties to the even code,
    sign kept."""
    return _encode(v, _E4M3_EXACT, _E4M3_ABOVE)


def enc_e2m1(v: np.ndarray) -> np.ndarray:
    return _encode(v, _E2M1_EXACT, _E2M1_ABOVE)


_DEC_E4M3 = np.concatenate([np.append(E4M3, np.nan), -np.append(E4M3, np.nan)])   # all 256 codes
_DEC_E2M1 = np.concatenate([E2M1, -E2M1])                                             # all 16 codes


def dec_e4m3(c: np.ndarray) -> np.ndarray:
    return _DEC_E4M3[c]


def dec_e2m1(c: np.ndarray) -> np.ndarray:
    return _DEC_E2M1[c]


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    """BF16 bits of float32 values, nearest with ties to even; NaN -> 0x7FC0."""
    u = v.astype(np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(np.isnan(v), np.uint16(0x7FC0), r)


# ------------------------------------------------------------------ MXFP8

def e8m0_codes(amax: np.ndarray) -> np.ndarray:
    """Smallest e >= -127 with amax <= 448 * 2^e, as e + 127; 0 for amax == 0 (float64)."""
    with np.errstate(divide="ignore"):
        e = np.ceil(np.log2(amax / 448.0))
    e = np.where(amax > 0, e, -127.0)
    e = np.clip(e, -127.0, 127.0)
    # the logarithm is approximate: settle e with exact comparisons of powers of two
    e = np.where(np.ldexp(448.0, e.astype(np.int64)) < amax, e + 1, e)
    e = np.where((e > -127) & (np.ldexp(448.0, e.astype(np.int64) - 1) >= amax), e - 1, e)
    return (e + 127).astype(np.uint8)


def mx_quantize_rowwise(x_bits: np.ndarray):
    """x [M][K] BF16 bits, K % 32 == 0 -> (q [M][K] E4M3, s [M][K/32] E8M0)."""
    M, K = x_bits.shape
    v = bf16_to_f32(x_bits).reshape(M, K // 32, 32)
    amax = np.abs(v).max(axis=2).astype(np.float64)
    c = e8m0_codes(amax)
    inv = np.ldexp(np.float32(1), 127 - c.astype(np.int32)).astype(np.float32)   # 2^-e, normal
    # |x 2^-e| <= 448: the binary32 product is exact down to 2^-126, and anything smaller
    # encodes to a signed zero whichever way it was rounded
    with np.errstate(under="ignore"):
        return enc_e4m3(v * inv[:, :, None]).reshape(M, K), c


def mx_quantize_colwise(x_bits: np.ndarray):
    """32x1 blocks down the columns, stored transposed: (q [K][M], s [K][M/32])."""
    return mx_quantize_rowwise(np.ascontiguousarray(x_bits.T))


def mx_dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """BF16 bits of DEC(q) * 2^(c - 127) (exact, then nearest-even to BF16)."""
    rows, cols = q.shape
    sc = np.where(s == 0xFF, np.nan, np.ldexp(1.0, s.astype(np.int64) - 127))
    y = dec_e4m3(q).reshape(rows, cols // 32, 32) * sc[:, :, None]
    with np.errstate(over="ignore"):
        return f32_to_bf16(y.reshape(rows, cols).astype(np.float32))


# ------------------------------------------------------------------ NVFP4

def _nv_blocks(v32: np.ndarray, s: np.ndarray):
    """Blocks v32 [..., n] (float32) under FP32 scales s [...] -> (block scale codes, codes)."""
    amax_b = np.abs(v32).max(axis=-1)
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        p = np.float32(6) * s
        t = amax_b / p
        sb = np.where(s == 0, np.uint8(0), enc_e4m3(np.where(s == 0, np.float32(0), t)))
        d = dec_e4m3(sb).astype(np.float32) * s
        f = np.where(d == 0, np.float32(0), np.minimum(np.float32(1) / d, FLT_MAX)).astype(np.float32)
        q = enc_e2m1(v32 * f[..., None])
    return sb.astype(np.uint8), q


def _pack(codes: np.ndarray) -> np.ndarray:
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def nv_quantize_per_token(x_bits: np.ndarray):
    """x [R][K] BF16 bits, K % 16 == 0 -> (q [R][K/2], sb [R][K/16], st [R] float32)."""
    R, K = x_bits.shape
    v = bf16_to_f32(x_bits)
    st = np.abs(v).max(axis=1) / np.float32(2688)
    sb, q = _nv_blocks(v.reshape(R, K // 16, 16), st[:, None])
    return _pack(q.reshape(R, K)), sb, st.astype(np.float32)


def nv_quantize_per_group(x_bits: np.ndarray, offsets):
    """One FP32 scale per row group [o_g, o_g+1) -> (q, sb, s_group float32 [G])."""
    R, K = x_bits.shape
    v = bf16_to_f32(x_bits)
    row_amax = np.abs(v).max(axis=1) if R else np.zeros(0, np.float32)
    off = np.asarray(offsets, np.int64)
    sg = np.array([row_amax[a:b].max() if b > a else 0 for a, b in zip(off[:-1], off[1:])], np.float32)
    sg = (sg / np.float32(2688)).astype(np.float32)
    s_row = np.repeat(sg, np.diff(off))
    sb, q = _nv_blocks(v.reshape(R, K // 16, 16), s_row[:, None])
    return _pack(q.reshape(R, K)), sb, sg


def nv_quantize_2d(x_bits: np.ndarray, offsets):
    """16x16 tiles under per-group FP32 scales -> (q [R][K/2], sb [R/16][K/16], s_group)."""
    R, K = x_bits.shape
    v = bf16_to_f32(x_bits)
    off = np.asarray(offsets, np.int64)
    row_amax = np.abs(v).max(axis=1)
    sg = np.array([row_amax[a:b].max() if b > a else 0 for a, b in zip(off[:-1], off[1:])], np.float32)
    sg = (sg / np.float32(2688)).astype(np.float32)
    s_tile = np.repeat(sg, np.diff(off) // 16)                             # per tile row
    tiles = v.reshape(R // 16, 16, K // 16, 16).transpose(0, 2, 1, 3).reshape(R // 16, K // 16, 256)
    sb, q = _nv_blocks(tiles, s_tile[:, None])
    q = q.reshape(R // 16, K // 16, 16, 16).transpose(0, 2, 1, 3).reshape(R, K)
    return _pack(q), sb, sg


def nv_dequantize(q: np.ndarray, sb: np.ndarray, st: np.ndarray) -> np.ndarray:
    """BF16 bits of fl(exact(DEC(q) * DEC(sb)) * s_t) for the per-token layout."""
    R, half = q.shape
    K = 2 * half
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(R, K)
    inner = (dec_e2m1(codes).reshape(R, K // 16, 16) * dec_e4m3(sb)[:, :, None]).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        y = inner * st.astype(np.float32)[:, None, None]
    return f32_to_bf16(y.reshape(R, K))
