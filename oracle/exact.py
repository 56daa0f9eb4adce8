"""Exact-rational brute-force verifier for the block-scaled quantizer contract.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Used on tiny inputs to pin the C
oracle; never timed.  It shares no code with ``bsq_oracle.c``: every value is a
``fractions.Fraction`` built from the bit-field definition of its format, every
"nearest representable value" is found by scanning *all* codes of the format, and every
binary32 rounding is done from the IEEE definition (nearest value of the binary32 grid,
ties to even significand, gradual underflow, overflow to infinity).

Passages followed (the pages, "Towards Blackwell-native 8-bit and 4-bit RL"):
* section "Format background": MXFP8 blocks of 32 E4M3 values with one E8M0 scale
  rounded up so the block maximum never clips; NVFP4 E2M1 values with one E4M3 scale
  per 16 values rounded to nearest and a coarse FP32 scale.
* section "Per-token activation scaling": one FP32 scale per token.
* section "High-precision and dequantized backward": BF16 dequantized operands.
The readings where the pages are silent are the same as the C oracle's (its header
lists them); this file restates them independently.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Optional, Sequence, Tuple

INF = float("inf")


# ---------------------------------------------------------------------------------------
# Decoders from the bit-field definitions
# ---------------------------------------------------------------------------------------

def _pow2(e: int) -> Fraction:
    return Fraction(2) ** e


def bf16_value(bits: int) -> Tuple[int, Optional[Fraction]]:
    """(sign, magnitude) of a BF16 pattern; magnitude None for NaN/inf."""
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        return s, None
    if e == 0:
        return s, Fraction(m) * _pow2(-126 - 7)
    return s, (1 + Fraction(m, 128)) * _pow2(e - 127)


def e4m3_value(code: int) -> Optional[Fraction]:
    """Signed value of an OCP E4M3FN code; None for the two NaN codes."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return None
    v = Fraction(m, 8) * _pow2(-6) if e == 0 else (1 + Fraction(m, 8)) * _pow2(e - 7)
    return -v if s else v


def e2m1_value(code: int) -> Fraction:
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    v = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * _pow2(e - 1)
    return -v if s else v


def e8m0_value(code: int) -> Optional[Fraction]:
    return None if code == 0xFF else _pow2(code - 127)


def binary32_value(bits: int) -> Tuple[int, Optional[Fraction]]:
    s = (bits >> 31) & 1
    e = (bits >> 23) & 0xFF
    m = bits & 0x7FFFFF
    if e == 0xFF:
        return s, None
    if e == 0:
        return s, Fraction(m) * _pow2(-126 - 23)
    return s, (1 + Fraction(m, 1 << 23)) * _pow2(e - 127)


# ---------------------------------------------------------------------------------------
# Nearest-value rounding
# ---------------------------------------------------------------------------------------

def _floor_log2(a: Fraction) -> int:
    """Largest integer n with 2^n <= a, for a > 0."""
    n = a.numerator.bit_length() - a.denominator.bit_length()
    while _pow2(n) > a:
        n -= 1
    while _pow2(n + 1) <= a:
        n += 1
    return n


def _round_half_even(n: Fraction) -> int:
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def round_binary_float(a: Fraction, mant_bits: int, emin: int, emax: int):
    """Round a >= 0 to the nearest value of a binary format with ``mant_bits`` stored
    mantissa bits, normal exponents emin..emax, gradual underflow; ties to even
    significand; returns INF when the rounded magnitude reaches 2^(emax+1)."""
    if a == 0:
        return Fraction(0)
    ex = max(_floor_log2(a), emin)
    quantum = _pow2(ex - mant_bits)
    r = _round_half_even(a / quantum) * quantum
    if r >= _pow2(emax + 1):
        return INF
    return r


def rn_binary32(sign: int, a: Fraction):
    """Signed binary32 nearest to (-1)^sign * a; returns (sign, magnitude or INF)."""
    return sign, round_binary_float(a, 23, -126, 127)


def rn_bf16_bits(sign: int, a) -> int:
    """BF16 bit pattern nearest to (-1)^sign * a (a a Fraction >= 0, or INF)."""
    if a == INF:
        return (sign << 15) | 0x7F80
    r = round_binary_float(a, 7, -126, 127)
    if r == INF:
        return (sign << 15) | 0x7F80
    if r == 0:
        return sign << 15
    if r < _pow2(-126):
        return (sign << 15) | int(r / _pow2(-133))
    ex = _floor_log2(r)
    mant = int(r / _pow2(ex - 7)) - 128
    return (sign << 15) | ((ex + 127) << 7) | mant


def binary32_bits(sign: int, a) -> int:
    """Bit pattern of a binary32 value given exactly (a on the binary32 grid, or INF)."""
    if a == INF:
        return (sign << 31) | 0x7F800000
    if a == 0:
        return sign << 31
    if a < _pow2(-126):
        m = a / _pow2(-149)
        assert m.denominator == 1
        return (sign << 31) | int(m)
    ex = _floor_log2(a)
    m = a / _pow2(ex - 23) - (1 << 23)
    assert m.denominator == 1
    return (sign << 31) | ((ex + 127) << 23) | int(m)


_E4M3_POS = [(c, e4m3_value(c)) for c in range(0x00, 0x80) if e4m3_value(c) is not None]
_E2M1_POS = [(c, e2m1_value(c)) for c in range(0, 8)]


def _nearest_by_scan(a, table) -> int:
    """Code of the nearest finite table value to a >= 0 (INF allowed), ties to the even
    code, found by scanning every code."""
    if a == INF:
        return max(table, key=lambda cv: cv[1])[0]
    best = None
    for c, v in table:
        d = abs(a - v)
        if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
            best = (c, d)
    return best[0]


def enc_e4m3(sign: int, a) -> int:
    return _nearest_by_scan(a, _E4M3_POS) | (0x80 if sign else 0)


def enc_e2m1(sign: int, a) -> int:
    return _nearest_by_scan(a, _E2M1_POS) | (8 if sign else 0)


# ---------------------------------------------------------------------------------------
# MXFP8
# ---------------------------------------------------------------------------------------

def e8m0_code(amax: Fraction) -> int:
    """Smallest e >= -127 with amax <= 448 * 2^e, as e + 127; zero block -> 0.  Found by
    scanning every candidate exponent from -127 upwards."""
    if amax == 0:
        return 0
    for e in range(-127, 128):
        if amax <= 448 * _pow2(e):
            return e + 127
    raise ValueError("amax beyond every E8M0 scale")


def mx_block(bits: Sequence[int]) -> Tuple[int, List[int]]:
    """One block of 32 BF16 patterns -> (E8M0 code, 32 E4M3 codes)."""
    assert len(bits) == 32
    vals = [bf16_value(b) for b in bits]
    amax = max(v for _, v in vals)
    c = e8m0_code(amax)
    scale = _pow2(c - 127)
    return c, [enc_e4m3(s, v / scale) for s, v in vals]


def mx_quantize_rowwise(x: Sequence[Sequence[int]]):
    q, s = [], []
    for row in x:
        qr, sr = [], []
        for b in range(0, len(row), 32):
            c, codes = mx_block(row[b:b + 32])
            sr.append(c)
            qr.extend(codes)
        q.append(qr)
        s.append(sr)
    return q, s


def mx_quantize_colwise(x: Sequence[Sequence[int]]):
    """Columnwise blocks = rowwise blocks of the transpose, stored as the transpose."""
    xt = [list(col) for col in zip(*x)]
    return mx_quantize_rowwise(xt)


def mx_block_partial(bits: Sequence[int]) -> Tuple[int, List[int]]:
    """A block of 1 to 32 BF16 patterns (the last block of an expert segment may hold
    fewer than 32 rows) -> (E8M0 code, its E4M3 codes); the scale is set by the largest
    magnitude present."""
    assert 1 <= len(bits) <= 32
    vals = [bf16_value(b) for b in bits]
    amax = max(v for _, v in vals)
    c = e8m0_code(amax)
    scale = _pow2(c - 127)
    return c, [enc_e4m3(s, v / scale) for s, v in vals]


def mx_quantize_colwise_grouped(x: Sequence[Sequence[int]], offsets: Sequence[int]):
    """Grouped columnwise copy: for each expert, the columnwise blocks of that expert's
    rows alone, 32 rows at a time from the segment start (the last block partial).
    Returns (q_col as K lists of M codes, K lists of scale codes in expert order)."""
    M, K = len(x), len(x[0])
    q = [[None] * M for _ in range(K)]
    s = [[] for _ in range(K)]
    for e in range(len(offsets) - 1):
        lo, hi = offsets[e], offsets[e + 1]
        for k in range(K):
            column = [x[r][k] for r in range(lo, hi)]
            for b in range(0, hi - lo, 32):
                c, codes = mx_block_partial(column[b:b + 32])
                s[k].append(c)
                q[k][lo + b:lo + b + len(codes)] = codes
    return q, s


def mx_dequant_one(q: int, c: int) -> int:
    v = e4m3_value(q)
    sc = e8m0_value(c)
    if v is None or sc is None:
        return 0x7FC0
    sign = 1 if (q & 0x80) else 0
    return rn_bf16_bits(sign, abs(v) * sc)


# ---------------------------------------------------------------------------------------
# Per-token NVFP4
# ---------------------------------------------------------------------------------------

def _f32(sign: int, a: Fraction):
    """Round a signed exact value to binary32 (magnitude may come back as INF)."""
    return rn_binary32(sign, a)


def nv_block(blk, s):
    """One NVFP4 block -- a list of (sign, magnitude) pairs, the 16 values of a 1x16 block or
    the 256 of a 16x16 tile -- under the FP32 scale s (an exact binary32 magnitude) ->
    (E4M3 scale code, E2M1 codes in the block's order)."""
    amax_b = max(v for _, v in blk)
    if s == 0:
        sb = 0
    else:
        _, p = _f32(0, 6 * s)                            # fl(6 * s)
        _, t = _f32(0, amax_b / p)                       # fl(amax_b / p)
        sb = enc_e4m3(0, t)
    _, d = _f32(0, e4m3_value(sb) * s)                   # fl(DEC(sb) * s)
    if d == 0:
        f = Fraction(0)
    else:
        _, f = _f32(0, 1 / d)                            # fl(1 / D)
        if f == INF:
            f = (2 - _pow2(-23)) * _pow2(127)            # FLT_MAX
    codes = []
    for sg, v in blk:
        _, y = _f32(sg, v * f)                           # fl(x * f)
        codes.append(enc_e2m1(sg, y))
    return sb, codes


def _pack(codes: Sequence[int]) -> List[int]:
    return [codes[i] | (codes[i + 1] << 4) for i in range(0, len(codes), 2)]


def nv_row_under(bits: Sequence[int], s):
    """One row of BF16 patterns (len % 16 == 0) encoded in 1x16 blocks under the given FP32
    scale s (exact binary32 magnitude) -> (packed q bytes, sb codes)."""
    vals = [bf16_value(b) for b in bits]
    sbs, codes = [], []
    for b in range(0, len(vals), 16):
        sb, c = nv_block(vals[b:b + 16], s)
        sbs.append(sb)
        codes.extend(c)
    return _pack(codes), sbs


def nv_row(bits: Sequence[int]):
    """One row of BF16 patterns (len % 16 == 0) -> (packed q bytes, sb codes, s_t magnitude
    as an exact binary32 value)."""
    amax_t = max(bf16_value(b)[1] for b in bits)
    _, s_t = _f32(0, amax_t / 2688)                     # fl(amax_t / 2688)
    packed, sbs = nv_row_under(bits, s_t)
    return packed, sbs, s_t


# ---------------------------------------------------------------------------------------
# NVFP4 with one FP32 scale per row group, and with 16x16 weight tiles
# ---------------------------------------------------------------------------------------
#
# Section "Format background": the scope of the coarse FP32 scale (a tensor, a batch, a
# token) is a recipe choice; section "Per-token activation scaling": gate and up are
# quantized together so that both get one scale.  Page "NVIDIA verified the 4-bit NVFP4
# format on a Mamba-Transformer (12B) at 10 trillion tokens": two-dimensional block scaling
# of the weights.  Reading (the same as the C oracle's, restated here): a group of rows
# [o_g, o_{g+1}) gets s_g = fl(amax_g / 2688) over all its values (0 for an empty group);
# its blocks -- 1x16 along a row, or 16x16 tiles -- are encoded with the per-token steps
# under s_g.  These functions walk group by group, tile by tile, and index every output
# from that walk; the C oracle walks rows and looks each row's group up.

def group_scale(x: Sequence[Sequence[int]], lo: int, hi: int):
    """s_g = fl(amax over rows lo..hi-1 / 2688) as an exact binary32 magnitude."""
    amax = Fraction(0)
    for r in range(lo, hi):
        for b in x[r]:
            amax = max(amax, bf16_value(b)[1])
    return _f32(0, amax / 2688)[1]


def nv_quantize_per_group(x: Sequence[Sequence[int]], offsets: Sequence[int]):
    """Rows of BF16 patterns and group offsets -> (packed q rows, sb rows, [s_g])."""
    R = len(x)
    q, sb = [None] * R, [None] * R
    scales = []
    for g in range(len(offsets) - 1):
        lo, hi = offsets[g], offsets[g + 1]
        s = group_scale(x, lo, hi)
        scales.append(s)
        for r in range(lo, hi):
            q[r], sb[r] = nv_row_under(x[r], s)
    return q, sb, scales


def nv_quantize_2d(x: Sequence[Sequence[int]], offsets: Sequence[int]):
    """Rows of BF16 patterns (R and K multiples of 16, every group whole 16-row tiles) ->
    (packed q rows, tile scales sb[R/16][K/16], [s_g])."""
    R, K = len(x), len(x[0])
    codes = [[None] * K for _ in range(R)]
    sb = [[None] * (K // 16) for _ in range(R // 16)]
    scales = []
    for g in range(len(offsets) - 1):
        lo, hi = offsets[g], offsets[g + 1]
        assert lo % 16 == 0 and hi % 16 == 0
        s = group_scale(x, lo, hi)
        scales.append(s)
        for tr in range(lo // 16, hi // 16):
            for tc in range(K // 16):
                cells = [(16 * tr + i, 16 * tc + j) for i in range(16) for j in range(16)]
                code, c = nv_block([bf16_value(x[r][k]) for r, k in cells], s)
                sb[tr][tc] = code
                for (r, k), ck in zip(cells, c):
                    codes[r][k] = ck
    return [_pack(row) for row in codes], sb, scales


def _nibble(q_rows, r: int, k: int) -> int:
    byte = q_rows[r][k // 2]
    return (byte >> 4) & 0xF if k % 2 else byte & 0xF


def nv_dequantize_per_group(q_rows, sb_rows, scales, offsets):
    """BF16 patterns RNE_BF16(fl(exact(DEC(q) * DEC(sb[r][k/16])) * s_g)) of the per-group
    layout; scales are (sign, magnitude) pairs as binary32_value returns them."""
    R, K = len(q_rows), 2 * len(q_rows[0])
    y = [[None] * K for _ in range(R)]
    for g in range(len(offsets) - 1):
        sg, s = scales[g]
        for r in range(offsets[g], offsets[g + 1]):
            for k in range(K):
                y[r][k] = nv_dequant_one(_nibble(q_rows, r, k), sb_rows[r][k // 16], sg, s)
    return y


def nv_dequantize_2d(q_rows, sb_tiles, scales, offsets):
    """BF16 patterns of the 16x16-tile layout: every element of tile (tr, tc), in a row of
    group g, is RNE_BF16(fl(exact(DEC(q) * DEC(sb[tr][tc])) * s_g))."""
    R, K = len(q_rows), 2 * len(q_rows[0])
    y = [[None] * K for _ in range(R)]
    for g in range(len(offsets) - 1):
        sg, s = scales[g]
        for tr in range(offsets[g] // 16, offsets[g + 1] // 16):
            for tc in range(K // 16):
                t = sb_tiles[tr][tc]
                for i in range(16):
                    for j in range(16):
                        r, k = 16 * tr + i, 16 * tc + j
                        y[r][k] = nv_dequant_one(_nibble(q_rows, r, k), t, sg, s)
    return y


def nv_dequant_one(code: int, sb: int, s_t_sign: int, s_t) -> int:
    """BF16 pattern of RNE_BF16(fl(exact(DEC(code) * DEC(sb)) * s_t))."""
    vq = e2m1_value(code)
    vs = e4m3_value(sb)
    if vs is None or s_t is None:
        return 0x7FC0
    inner = vq * vs
    sign = ((1 if (code & 8) else 0) ^ (1 if (sb & 0x80) else 0) ^ s_t_sign)
    if s_t == INF:
        if inner == 0:
            return 0x7FC0
        return rn_bf16_bits(sign, INF)
    _, y = _f32(sign, abs(inner) * s_t)
    return rn_bf16_bits(sign, y)
