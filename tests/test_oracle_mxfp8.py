"""Pins of the oracle's MXFP8 quantize/dequantize.

Passages ("Towards Blackwell-native 8-bit and 4-bit RL"):
* section "Format background": 32 consecutive E4M3 values share one E8M0 scale, blocks
  are one-dimensional, the decoded scale is rounded up so the block maximum never clips;
* section "Recipe 1: end-to-end MXFP8 RL": rowwise 1x32 and columnwise 32x1 blocks are
  numerically different, and both copies are quantized from full precision;
* section "Bit-exact quantizer contract": test data of the kinds random, boundary, zeros
  and maxes.
"""
from fractions import Fraction
import os

import numpy as np
import pytest

import oracle
import workloads
from oracle import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(vals) -> np.ndarray:
    """BF16 bits of values that are exact in BF16 (asserted)."""
    f = np.asarray(vals, dtype=np.float32)
    b = workloads.bf16_bits_from_f32(f)
    assert np.array_equal(workloads.f32_from_bf16_bits(b), f)
    return b


def _read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, *v = line.split()
            out[k] = v
    return out


# --------------------------------------------------------------------------- E8M0 choice

def test_e8m0_code_every_positive_bf16_is_smallest_non_clipping_exponent():
    """For all 32639 positive finite BF16 amax values: amax <= 448*2^e and, unless the
    -127 clamp applies, amax > 448*2^(e-1)."""
    for b in range(1, 0x7F80):
        _, amax = exact.bf16_value(b)
        c = oracle.e8m0_code(float(amax))
        e = c - 127
        assert amax <= 448 * Fraction(2) ** e, hex(b)
        assert e == -127 or amax > 448 * Fraction(2) ** (e - 1), hex(b)
        assert c <= 247


def test_e8m0_code_integer_closed_form():
    """Closed form on the BF16 fields: c = max(E - 8 + [mantissa > 0x60], 0), since
    (1 + m/128) <= 1.75 exactly when m <= 96."""
    for b in range(1, 0x7F80):
        E, m = b >> 7, b & 0x7F
        want = max(E - 8 + (1 if m > 0x60 else 0), 0)
        assert oracle.e8m0_code(oracle.bf16_to_float(b)) == want, hex(b)
    assert oracle.e8m0_code(0.0) == 0


# --------------------------------------------------------------------------- handmade

def test_rowwise_differs_from_colwise_handmade_example():
    g = _read_golden("mx_rowwise_vs_colwise.txt")
    h = lambda k: int(g[k][0], 16)
    x = np.full((32, 32), h("input_other_bf16"), np.uint16)
    x[0, :] = h("input_row0_bf16")
    q_r, s_r = oracle.mx_quantize_rowwise(x)
    q_c, s_c = oracle.mx_quantize_colwise(x)
    assert s_r[0, 0] == h("row_scale_row0") and np.all(s_r[1:, 0] == h("row_scale_other"))
    assert np.all(q_r[0] == h("row_code_row0")) and np.all(q_r[1:] == h("row_code_other"))
    assert np.all(s_c == h("col_scale"))
    assert np.all(q_c[:, 0] == h("col_code_row0")) and np.all(q_c[:, 1:] == h("col_code_other"))
    y_r = oracle.mx_dequantize(q_r, s_r)
    y_c = oracle.mx_dequantize(q_c, s_c)
    assert np.all(y_r[0] == h("row_dequant_row0")) and np.all(y_r[1:] == h("row_dequant_other"))
    assert np.all(y_c[:, 0] == h("col_dequant_row0")) and np.all(y_c[:, 1:] == h("col_dequant_other"))
    assert not np.array_equal(y_r, y_c.T)              # the two copies really differ


# --------------------------------------------------------------------------- exact verifier

def _random_blocks(rng, n):
    """Blocks of the four kinds named on the pages: random, boundary, zeros, maxes."""
    blocks = []
    for i in range(n):
        kind = i % 6
        if kind == 0:       # random, random magnitude anywhere in the BF16 range
            v = rng.standard_normal(32) * np.exp2(rng.integers(-130, 120))
            blocks.append(workloads.bf16_bits_from_f32(v.astype(np.float32)))
        elif kind == 1:     # random bit patterns (finite)
            b = rng.integers(0, 1 << 16, 32).astype(np.uint16)
            b[(b & 0x7F80) == 0x7F80] &= np.uint16(0xBFFF)
            blocks.append(b)
        elif kind == 2:     # zeros, with signs
            b = np.zeros(32, np.uint16)
            b[rng.random(32) < 0.5] = 0x8000
            blocks.append(b)
        elif kind == 3:     # maxes: 448*2^k, BF16 max, and neighbours
            k = int(rng.integers(-130, 118))
            v = np.full(32, 448.0 * 2.0 ** k)
            b = workloads.bf16_bits_from_f32(v.astype(np.float32))
            b[rng.integers(32)] = 0x7F7F if rng.random() < 0.3 else b[0] + 1
            b[rng.random(32) < 0.3] |= np.uint16(0x8000)
            blocks.append(b)
        elif kind == 4:     # boundary: E4M3 midpoints times the block scale
            e = int(rng.integers(-120, 110))
            mids = [(exact.e4m3_value(c) + exact.e4m3_value(c + 1)) / 2 for c in range(0x7E)]
            pick = rng.integers(0, len(mids), 31)
            vals = [float(mids[p]) * 2.0 ** e for p in pick] + [448.0 * 2.0 ** e]
            f = np.array(vals, np.float32)
            b = workloads.bf16_bits_from_f32(f)
            blocks.append(b)
        else:               # BF16 subnormals (scale clamps at 2^-127)
            b = rng.integers(0, 0x80, 32).astype(np.uint16)
            b[rng.random(32) < 0.5] |= np.uint16(0x8000)
            blocks.append(b)
    return blocks


def test_mx_oracle_matches_exact_verifier_on_tiny_blocks():
    rng = np.random.default_rng(21)
    blocks = _random_blocks(rng, 240)
    x = np.stack(blocks).reshape(-1, 64)            # two blocks per row
    q, s = oracle.mx_quantize_rowwise(x)
    for r in range(x.shape[0]):
        for b in range(2):
            c, codes = exact.mx_block([int(v) for v in x[r, 32 * b:32 * b + 32]])
            assert s[r, b] == c
            assert list(q[r, 32 * b:32 * b + 32]) == codes


def test_colwise_is_rowwise_of_the_transpose():
    x = workloads.config2(seed=5, rows=96, cols=160)["x"]
    q_c, s_c = oracle.mx_quantize_colwise(x)
    q_t, s_t = oracle.mx_quantize_rowwise(np.ascontiguousarray(x.T))
    assert np.array_equal(q_c, q_t) and np.array_equal(s_c, s_t)
    e_q, e_s = exact.mx_quantize_colwise([[int(v) for v in row] for row in x[:32, :8]])
    assert np.array_equal(q_c[:8, :32], np.array(e_q)) and np.array_equal(s_c[:8, :1], np.array(e_s))


# --------------------------------------------------------------------------- invariants

def _block_amax(x):
    a = np.abs(workloads.f32_from_bf16_bits(x).astype(np.float64))
    return a.reshape(x.shape[0], -1, 32).max(axis=2)


def test_no_clip_and_minimal_scale_on_config_like_data():
    x = workloads.config2(seed=6, rows=512)["x"]
    q, s = oracle.mx_quantize_rowwise(x)
    amax = _block_amax(x)
    e = s.astype(np.int64) - 127
    assert np.all(amax * np.exp2(-e) <= 448.0)
    assert np.all((s == 0) | (amax * np.exp2(-(e - 1)) > 448.0))
    # no element ever saturates: dequant never exceeds the block max
    y = workloads.f32_from_bf16_bits(oracle.mx_dequantize(q, s)).astype(np.float64)
    assert np.all(np.abs(y).reshape(amax.shape + (32,)).max(axis=2) <= amax * 1.0625)


def test_dequant_requantizes_to_the_same_codes():
    """Every finite (code, scale) pair whose dequantized value is a normal BF16 comes back
    to the same code when re-encoded with the same scale (dequant is exact there)."""
    for c in range(0, 255):
        for code in range(256):
            if (code & 0x7F) == 0x7F:
                continue
            v = oracle.dec_e4m3(code) * 2.0 ** (c - 127)
            if v != 0 and not (2.0 ** -126 <= abs(v) < 2.0 ** 128):
                continue
            y = oracle.mx_dequantize(np.array([[code] * 32], np.uint8), np.array([[c]], np.uint8))
            yv = oracle.bf16_to_float(int(y[0, 0]))
            assert yv == v
            assert oracle.enc_e4m3(yv * 2.0 ** (127 - c)) == code


def test_dequant_every_code_and_scale_matches_exact():
    codes = np.arange(256, dtype=np.uint8)
    q = np.tile(codes, (256, 1))                          # row = scale, 8 blocks per row
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    y = oracle.mx_dequantize(q, s)
    for c in range(256):
        for code in range(256):
            assert y[c, code] == exact.mx_dequant_one(code, c), (c, code)


def test_dequant_overflow_to_inf():
    # a block holding BF16 max gets c = 247; its element 2^127*(2-2^-7)/2^120 rounds to 256
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = 0x7F7F
    q, s = oracle.mx_quantize_rowwise(x)
    assert s[0, 0] == 247 and q[0, 0] == 0x78
    assert oracle.mx_dequantize(q, s)[0, 0] == 0x7F80


def test_power_of_two_equivariance():
    rng = np.random.default_rng(22)
    v = (rng.standard_normal((64, 64)) * 3).astype(np.float32)
    x = workloads.bf16_bits_from_f32(v)
    q0, s0 = oracle.mx_quantize_rowwise(x)
    for k in (-20, -3, 1, 7, 40):
        xk = workloads.bf16_bits_from_f32(workloads.f32_from_bf16_bits(x) * np.float32(2.0 ** k))
        qk, sk = oracle.mx_quantize_rowwise(xk)
        nz = s0 > 0
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk[nz].astype(int), s0[nz].astype(int) + k)


def test_sign_symmetry():
    x = workloads.config2(seed=7, rows=64)["x"]
    q, s = oracle.mx_quantize_rowwise(x)
    qn, sn = oracle.mx_quantize_rowwise(x ^ np.uint16(0x8000))
    assert np.array_equal(s, sn) and np.array_equal(qn, q ^ np.uint8(0x80))


def test_config1_zero_block_and_outliers():
    cfg = workloads.config1()
    x = cfg["x"]
    q, s = oracle.mx_quantize_rowwise(x)
    r, b = cfg["zero_block"]
    assert s[r, b] == 0 and np.all((q[r, 32 * b:32 * b + 32] & 0x7F) == 0)
    # the x1000 outliers lift their blocks' scales about log2(1000) ~ 10 codes
    assert int(s.max()) - int(np.median(s)) >= 7


# --------------------------------------------------------------------------- grouped colwise

def _rand_bf16(rng, rows, cols):
    x = rng.integers(0, 1 << 16, size=(rows, cols), dtype=np.uint16)
    x[(x & 0x7F80) == 0x7F80] &= 0xBFFF                   # finite only
    return x


def _parse_ranges(items):
    out = {}
    for it in items:
        where, val = it.split(":")
        lo, _, hi = where.partition("-")
        for r in range(int(lo), int(hi or lo) + 1):
            out[r] = int(val, 16)
    return out


def test_grouped_colwise_golden():
    g = _read_golden("mx_grouped_colwise.txt")
    M = int(g["rows"][0])
    off = [int(v) for v in g["offsets"]]
    xr, codes = _parse_ranges(g["x_rows"]), _parse_ranges(g["codes"])
    x = np.array([[xr[r]] * 32 for r in range(M)], np.uint16)
    q, s, ok = oracle.mx_quantize_colwise_grouped(x, off)
    assert ok and s.shape == (32, 3)
    assert np.all(s == np.array([int(v, 16) for v in g["scales"]], np.uint8))
    assert np.all(q == np.array([codes[r] for r in range(M)], np.uint8))


def test_grouped_colwise_with_aligned_segments_is_the_flat_copy():
    rng = np.random.default_rng(11)
    x = _rand_bf16(rng, 256, 64)
    for off in ([0, 256], [0, 32, 32, 96, 256], [0, 0, 128, 128, 224, 256]):
        q, s, ok = oracle.mx_quantize_colwise_grouped(x, off)
        qf, sf = oracle.mx_quantize_colwise(x)
        assert ok
        assert np.array_equal(q, qf) and np.array_equal(s, sf)


def test_grouped_colwise_partial_block_equals_zero_padded_segment():
    """Zero rows never raise a block maximum, so an expert's partial last block has the
    scale and codes of the flat columnwise copy of its segment padded with zero rows."""
    rng = np.random.default_rng(12)
    off = [0, 5, 5, 45, 77, 109, 110]
    x = _rand_bf16(rng, off[-1], 32)
    q, s, ok = oracle.mx_quantize_colwise_grouped(x, off)
    assert ok
    blk = 0
    for e in range(len(off) - 1):
        lo, hi = off[e], off[e + 1]
        m = hi - lo
        if m == 0:
            continue
        pad = np.zeros(((m + 31) // 32 * 32, 32), np.uint16)
        pad[:m] = x[lo:hi]
        qf, sf = oracle.mx_quantize_colwise(pad)
        nb = sf.shape[1]
        assert np.array_equal(q[:, lo:hi], qf[:, :m]), e
        assert np.array_equal(s[:, blk:blk + nb], sf), e
        blk += nb
    assert blk == s.shape[1]


def test_grouped_colwise_matches_exact_verifier():
    rng = np.random.default_rng(13)
    off = [0, 3, 3, 40, 41, 75]
    x = _rand_bf16(rng, off[-1], 4)
    x[1] = 0                                              # an all-zero row inside a block
    q, s, ok = oracle.mx_quantize_colwise_grouped(x, off)
    eq, es = exact.mx_quantize_colwise_grouped(x.tolist(), off)
    assert ok
    assert q.tolist() == eq
    assert s.tolist() == es


def test_grouped_colwise_rejects_bad_offsets_and_short_scale_rows():
    x = np.zeros((64, 32), np.uint16)
    for off in ([1, 64], [0, 40, 30, 64], [0, 63], [0, 65]):
        assert oracle.mx_quantize_colwise_grouped(x, off)[2] is False
    # offsets [0, 1, 64]: ceil(1/32) + ceil(63/32) = 3 blocks per column
    assert oracle.mx_quantize_colwise_grouped(x, [0, 1, 64], s_ld=2)[2] is False
    q, s, ok = oracle.mx_quantize_colwise_grouped(x, [0, 1, 64], s_ld=3)
    assert ok and s.shape == (32, 3) and np.all(s == 0) and np.all(q == 0)
