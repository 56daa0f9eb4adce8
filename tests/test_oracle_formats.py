"""Pins of the oracle's format codecs against closed forms and brute force.

Closed forms come from the bit-field definitions of the formats the pages name
("Towards Blackwell-native 8-bit and 4-bit RL", section "Format background": E4M3
elements with E8M0 scales for MXFP8; E2M1 elements with E4M3 scales for NVFP4).  The
brute-force checks scan every code of a format, independently of the oracle's
bracketing search.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from oracle import exact


# --------------------------------------------------------------------------- E4M3

def test_e4m3_closed_forms():
    assert oracle.dec_e4m3(0x7E) == 448.0            # largest finite
    assert oracle.dec_e4m3(0x08) == 2.0 ** -6         # smallest normal
    assert oracle.dec_e4m3(0x01) == 2.0 ** -9         # smallest subnormal
    assert oracle.dec_e4m3(0x38) == 1.0
    assert oracle.dec_e4m3(0x00) == 0.0 and math.copysign(1, oracle.dec_e4m3(0x80)) < 0
    assert math.isnan(oracle.dec_e4m3(0x7F)) and math.isnan(oracle.dec_e4m3(0xFF))
    finite = [c for c in range(256) if not math.isnan(oracle.dec_e4m3(c))]
    assert len(finite) == 254
    pos = [oracle.dec_e4m3(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))   # increasing in the code
    for c in range(0x7F):
        assert oracle.dec_e4m3(c | 0x80) == -oracle.dec_e4m3(c)


def test_e4m3_decode_matches_exact_definition():
    for c in range(256):
        ev = exact.e4m3_value(c)
        ov = oracle.dec_e4m3(c)
        if ev is None:
            assert math.isnan(ov)
        else:
            assert Fraction(ov) == ev


def test_e4m3_encode_roundtrip_every_code():
    for c in range(256):
        if (c & 0x7F) == 0x7F:
            continue
        assert oracle.enc_e4m3(oracle.dec_e4m3(c)) == c


def test_e4m3_encode_midpoints_go_to_even_code():
    for c in range(0x7E):
        lo, hi = oracle.dec_e4m3(c), oracle.dec_e4m3(c + 1)
        mid = (lo + hi) / 2                             # exact in binary64
        even = c if c % 2 == 0 else c + 1
        assert oracle.enc_e4m3(mid) == even
        assert oracle.enc_e4m3(-mid) == even | 0x80
        assert oracle.enc_e4m3(np.nextafter(mid, 0)) == c
        assert oracle.enc_e4m3(np.nextafter(mid, 1e9)) == c + 1


def test_e4m3_saturates_to_448_and_keeps_sign_of_zero():
    for v in (448.0, 460.0, 464.0, 479.9, 480.0, 1e6, 3.4e38, math.inf):
        assert oracle.enc_e4m3(v) == 0x7E
        assert oracle.enc_e4m3(-v) == 0xFE
    assert oracle.enc_e4m3(0.0) == 0x00
    assert oracle.enc_e4m3(-0.0) == 0x80
    assert oracle.enc_e4m3(-2.0 ** -10) == 0x80       # tie with 0: even code 0
    assert oracle.enc_e4m3(-1e-30) == 0x80


def _structured_fp32_inputs():
    """Every binary32 pattern whose high 16 bits are arbitrary and whose low 16 bits are
    one of a few values: this holds every E4M3 and E2M1 value, every midpoint between
    consecutive values, and the binary32 neighbours on both sides of each."""
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    bits = bits[(bits & np.uint32(0x7F800000)) != np.uint32(0x7F800000)]   # finite only
    return bits.view(np.float32).astype(np.float64)


def _brute_force_nearest(v: np.ndarray, table: np.ndarray, sign_bit: int) -> np.ndarray:
    """Nearest table entry to |v| by scanning all entries (exact in binary64 for the
    magnitudes passed here), ties to the even code, sign of v kept."""
    a = np.abs(v)
    out = np.empty(v.size, np.int64)
    for s in range(0, v.size, 1 << 15):
        d = np.abs(a[s:s + (1 << 15), None] - table[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        # among equal distances take the even code (two candidates at most)
        even = cand & (np.arange(table.size)[None, :] % 2 == 0)
        pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
        out[s:s + (1 << 15)] = pick
    return out | np.where(np.signbit(v), sign_bit, 0)


def test_e4m3_encode_brute_force_structured_sweep():
    v = _structured_fp32_inputs()
    v = v[np.abs(v) <= 1024.0]
    table = np.array([oracle.dec_e4m3(c) for c in range(0x7F)])
    got = oracle.enc_e4m3_array(v).astype(np.int64)
    want = _brute_force_nearest(v, table, 0x80)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e4m3_encode_exact_scan_on_random_binary32():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, size=3000, dtype=np.uint64).astype(np.uint32)
    for b in bits:
        s, a = exact.binary32_value(int(b))
        if a is None:
            continue
        v = float(np.uint32(b).view(np.float32))
        assert oracle.enc_e4m3(v) == exact.enc_e4m3(s, a), hex(int(b))


# --------------------------------------------------------------------------- E2M1

def test_e2m1_grid_closed_form():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert [oracle.dec_e2m1(c) for c in range(8)] == grid
    assert [oracle.dec_e2m1(c | 8) for c in range(8)] == [-g for g in grid]
    for c in range(16):
        assert Fraction(oracle.dec_e2m1(c)) == exact.e2m1_value(c)
        assert oracle.enc_e2m1(oracle.dec_e2m1(c)) == c


def test_e2m1_midpoints_and_saturation():
    # midpoint between codes lo and lo+1 -> the even one of the two;
    # 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2.0, 2.5->2, 3.5->4, 5->4
    expect = {0.25: (0, 0), 0.75: (1, 2), 1.25: (2, 2), 1.75: (3, 4), 2.5: (4, 4),
              3.5: (5, 6), 5.0: (6, 6)}
    for v, (lo, even) in expect.items():
        assert oracle.enc_e2m1(v) == even
        assert oracle.enc_e2m1(-v) == even | 8
        assert oracle.enc_e2m1(np.nextafter(v, 0)) == lo
        assert oracle.enc_e2m1(np.nextafter(v, 100)) == lo + 1
    for v in (6.0, 6.5, 7.0, 100.0, 3.4e38, math.inf):
        assert oracle.enc_e2m1(v) == 7 and oracle.enc_e2m1(-v) == 15
    assert oracle.enc_e2m1(-0.0) == 8 and oracle.enc_e2m1(-0.1) == 8


def test_e2m1_encode_brute_force_structured_sweep():
    v = _structured_fp32_inputs()
    v = v[np.abs(v) <= 64.0]
    table = np.array([oracle.dec_e2m1(c) for c in range(8)])
    got = oracle.enc_e2m1_array(v).astype(np.int64)
    want = _brute_force_nearest(v, table, 8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (v[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_e2m1_encode_exact_scan_on_random_binary32():
    rng = np.random.default_rng(12)
    bits = rng.integers(0, 1 << 32, size=3000, dtype=np.uint64).astype(np.uint32)
    for b in bits:
        s, a = exact.binary32_value(int(b))
        if a is None:
            continue
        v = float(np.uint32(b).view(np.float32))
        assert oracle.enc_e2m1(v) == exact.enc_e2m1(s, a), hex(int(b))


# --------------------------------------------------------------------------- E8M0 / BF16

def test_e8m0_is_pure_power_of_two():
    for c in range(255):
        assert oracle.dec_e8m0(c) == 2.0 ** (c - 127)
    assert math.isnan(oracle.dec_e8m0(255))


def test_bf16_decode_every_pattern_matches_definition():
    for b in range(1 << 16):
        s, a = exact.bf16_value(b)
        v = oracle.bf16_to_float(b)
        if a is None:
            assert not math.isfinite(v)
            continue
        assert Fraction(abs(v)) == a and (math.copysign(1, v) < 0) == bool(s)


def test_bf16_rounding_matches_exact_definition():
    rng = np.random.default_rng(13)
    vals = list(rng.standard_normal(400) * np.exp2(rng.integers(-140, 128, 400)))
    # ties, neighbours of ties, subnormals, overflow threshold
    for b in rng.integers(0, 0x7F7F, 200):
        lo = oracle.bf16_to_float(int(b))
        hi = oracle.bf16_to_float(int(b) + 1)
        mid = (lo + hi) / 2
        vals += [mid, np.nextafter(mid, -1e300), np.nextafter(mid, 1e300)]
    big = (2 - 2 ** -8) * 2.0 ** 127
    vals += [big, np.nextafter(big, 0), 2.0 ** -133, 2.0 ** -134, 1.5 * 2.0 ** -134,
             3 * 2.0 ** -135, 2.0 ** -126 - 2.0 ** -134]
    for v in vals:
        for sv in (v, -v):
            sign = 1 if sv < 0 else 0
            assert oracle.rne_bf16(sv) == exact.rn_bf16_bits(sign, Fraction(abs(sv))), sv


def test_bf16_rounding_agrees_with_numpy_float32_path_where_float32_is_exact():
    # for binary32 inputs, RNE to BF16 is the usual 16-bit rounding of the pattern
    rng = np.random.default_rng(14)
    bits = rng.integers(0, 0x7F7FFFFF, size=20000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    want = ((bits + np.uint32(0x7FFF) + ((bits >> 16) & 1)) >> 16).astype(np.uint16)
    got = oracle.rne_bf16_array(f.astype(np.float64))
    assert np.array_equal(got, want)
