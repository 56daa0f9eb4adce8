"""Pins of the oracle's per-token NVFP4 quantize/dequantize.

Passages ("Towards Blackwell-native 8-bit and 4-bit RL"):
* section "Format background": E2M1 values, one E4M3 scale per 16 values rounded to the
  nearest representable value, plus a coarse FP32 scale whose scope is a recipe choice;
* section "Per-token activation scaling": one FP32 scale per token, computed online; a
  token's quantized bytes must not depend on the other tokens of the batch; gate and up
  projections are quantized together;
* section "High-precision and dequantized backward": BF16 dequantized operands.
And the NVIDIA NVFP4 pretraining note (Russian page): at least 6.25% of each block
(the block-amax element, 1 of 16) is represented at close to FP8 precision.
"""
from fractions import Fraction
import math
import os

import numpy as np
import pytest

import oracle
import workloads
from oracle import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


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


def _bf16_exact(vals) -> np.ndarray:
    f = np.array([float(v) for v in vals], dtype=np.float32)
    b = workloads.bf16_bits_from_f32(f)
    assert np.array_equal(workloads.f32_from_bf16_bits(b), f)
    # keep the sign of negative zero written as "-0"
    b[np.signbit(f)] |= np.uint16(0x8000)
    return b


def _unpack(q):
    lo = q & np.uint8(0xF)
    hi = q >> np.uint8(4)
    return np.stack([lo, hi], axis=-1).reshape(q.shape[0], -1)


# --------------------------------------------------------------------------- handmade

def test_handmade_row_matches_golden():
    g = _read_golden("nvfp4_handmade.txt")
    x = _bf16_exact(g["x"])[None, :]
    q, sb, st = oracle.nv_quantize_per_token(x)
    assert [int(c, 16) for c in g["codes"]] == list(_unpack(q)[0])
    assert [int(c, 16) for c in g["q"]] == list(q[0])
    assert [int(c, 16) for c in g["sb"]] == list(sb[0])
    assert st[0] == float(g["st"][0])
    y = oracle.nv_dequantize(q, sb, st)
    assert np.array_equal(y[0], _bf16_exact(g["y"]))


# --------------------------------------------------------------------------- exact verifier

def _rows_of_every_kind(rng, n, K):
    """Rows of the kinds the pages name for quantizer tests: random, boundary, zeros,
    maxes; plus BF16-subnormal rows and rows with one huge outlier."""
    rows = []
    for i in range(n):
        kind = i % 7
        if kind == 0:
            v = rng.standard_normal(K) * np.exp2(rng.integers(-126, 120))
            rows.append(workloads.bf16_bits_from_f32(v.astype(np.float32)))
        elif kind == 1:
            b = rng.integers(0, 1 << 16, K).astype(np.uint16)
            b[(b & 0x7F80) == 0x7F80] &= np.uint16(0xBFFF)
            rows.append(b)
        elif kind == 2:
            b = np.zeros(K, np.uint16)
            b[rng.random(K) < 0.5] = 0x8000
            if rng.random() < 0.5:
                b[rng.integers(K)] = 0x3F80      # one lone 1.0 in a zero row
            rows.append(b)
        elif kind == 3:                          # maxes: 2688*2^k and BF16 max
            k = int(rng.integers(-130, 115))
            v = np.full(K, 2688.0 * 2.0 ** k, np.float32)
            b = workloads.bf16_bits_from_f32(v)
            if rng.random() < 0.3:
                b[rng.integers(K)] = 0x7F7F
            b[rng.random(K) < 0.5] |= np.uint16(0x8000)
            rows.append(b)
        elif kind == 4:                          # boundary: E2M1 midpoints x block step
            v = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 4.0], K) * np.exp2(rng.integers(-20, 20))
            v *= np.where(rng.random(K) < 0.5, -1, 1)
            rows.append(workloads.bf16_bits_from_f32(v.astype(np.float32)))
        elif kind == 5:                          # BF16 subnormal row (tiny s_t)
            b = rng.integers(0, 0x100, K).astype(np.uint16)
            b[rng.random(K) < 0.5] |= np.uint16(0x8000)
            rows.append(b)
        else:                                    # one outlier: many blocks' scales underflow
            v = rng.standard_normal(K) * 1e-3
            v[rng.integers(K)] = 3e4
            rows.append(workloads.bf16_bits_from_f32(v.astype(np.float32)))
    return np.stack(rows)


def test_nv_oracle_matches_exact_verifier_on_tiny_rows():
    rng = np.random.default_rng(31)
    x = _rows_of_every_kind(rng, 140, 32)
    q, sb, st = oracle.nv_quantize_per_token(x)
    for r in range(x.shape[0]):
        packed, sbs, s_t = exact.nv_row([int(v) for v in x[r]])
        assert list(sb[r]) == sbs, r
        assert list(q[r]) == packed, r
        assert Fraction(float(st[r])) == s_t, r


def test_nv_dequant_every_code_and_scale_matches_exact():
    rng = np.random.default_rng(32)
    sts = [1.0, 2.0 ** -140, 3.1e-5, 7.7e30, 0.0, float(np.float32(1 / 3))]
    sts += list(np.float32(rng.standard_normal(4) * 10.0 ** rng.integers(-30, 30, 4)).astype(float))
    for s_t in sts:
        s_t = float(np.float32(abs(s_t)))
        # one row: 16 codes per block x 256 block scales (K = 4096)
        codes = np.tile(np.arange(16, dtype=np.uint8), 256)
        q = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
        sb = np.arange(256, dtype=np.uint8)[None, :]
        y = oracle.nv_dequantize(q, sb, np.array([s_t], np.float32))
        _, st_exact = exact.binary32_value(int(np.float32(s_t).view(np.uint32)))
        for j in range(4096):
            assert y[0, j] == exact.nv_dequant_one(int(codes[j]), j // 16, 0, st_exact), (s_t, j)


# --------------------------------------------------------------------------- invariants

def _block_amax(x, width):
    a = np.abs(workloads.f32_from_bf16_bits(x).astype(np.float64))
    return a.reshape(x.shape[0], -1, width).max(axis=2)


def test_block_amax_element_is_six_when_block_scale_is_normal():
    """The block-amax element lands on E2M1 6 (code 7) whenever DEC(sb) >= 2^-6: the
    '6.25% of values near FP8 precision' property."""
    x = workloads.config3(seed=33, tokens=256, materialize=False)["h"]
    q, sb, st = oracle.nv_quantize_per_token(x)
    codes = _unpack(q)
    xa = np.abs(workloads.f32_from_bf16_bits(x)).reshape(x.shape[0], -1, 16)
    arg = xa.argmax(axis=2)
    c = np.take_along_axis(codes.reshape(x.shape[0], -1, 16), arg[..., None], axis=2)[..., 0]
    dec = np.vectorize(oracle.dec_e4m3)(sb)
    normal = dec >= 2.0 ** -6
    assert normal.mean() > 0.9
    assert np.all((c[normal] & 7) == 7)


def test_block_holding_token_amax_gets_scale_448():
    x = workloads.config3(seed=34, tokens=256, materialize=False)["h"]
    q, sb, st = oracle.nv_quantize_per_token(x)
    amax_b = _block_amax(x, 16)
    hold = amax_b == amax_b.max(axis=1, keepdims=True)
    assert np.all(sb[hold] == 0x7E)
    assert np.all(sb[~hold] <= 0x7E)


def test_per_token_invariance():
    """A token's bytes do not depend on the rest of the batch: change, permute, split or
    duplicate the other rows and every row's (q, sb, s_t) stays identical."""
    rng = np.random.default_rng(35)
    x = workloads.config3(seed=35, tokens=64, materialize=False)["h"]
    q, sb, st = oracle.nv_quantize_per_token(x)
    perm = rng.permutation(x.shape[0])
    qp, sbp, stp = oracle.nv_quantize_per_token(x[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sbp, sb[perm]) and np.array_equal(stp, st[perm])
    y = x.copy()
    y[1::2] = workloads.bf16_bits_from_f32(rng.standard_normal((32, x.shape[1])).astype(np.float32) * 1e4)
    qy, sby, sty = oracle.nv_quantize_per_token(y)
    assert np.array_equal(qy[0::2], q[0::2]) and np.array_equal(sty[0::2], st[0::2])
    qa, sba, sta = oracle.nv_quantize_per_token(x[:17])
    assert np.array_equal(qa, q[:17]) and np.array_equal(sba, sb[:17])
    dup = np.repeat(x[:8], 8, axis=0)
    qd, sbd, std = oracle.nv_quantize_per_token(dup)
    assert np.array_equal(qd, np.repeat(q[:8], 8, axis=0))


def test_gate_up_joint_equals_separate_under_per_row_scales():
    e = workloads.config4_expert(0, ffn=64, hidden=128)
    gu = e["gate_up"]
    q, sb, st = oracle.nv_quantize_per_token(gu)
    qg, sbg, stg = oracle.nv_quantize_per_token(gu[:64])
    qu, sbu, stu = oracle.nv_quantize_per_token(gu[64:])
    assert np.array_equal(q, np.concatenate([qg, qu])) and np.array_equal(st, np.concatenate([stg, stu]))


def test_power_of_two_equivariance():
    rng = np.random.default_rng(36)
    x = workloads.bf16_bits_from_f32((rng.standard_normal((32, 256)) * 5).astype(np.float32))
    q0, sb0, st0 = oracle.nv_quantize_per_token(x)
    for k in (-30, -4, 3, 60):
        xk = workloads.bf16_bits_from_f32(workloads.f32_from_bf16_bits(x) * np.float32(2.0 ** k))
        qk, sbk, stk = oracle.nv_quantize_per_token(xk)
        assert np.array_equal(qk, q0) and np.array_equal(sbk, sb0)
        assert np.array_equal(stk, st0 * np.float32(2.0 ** k))


def test_sign_symmetry():
    x = workloads.config3(seed=37, tokens=32, materialize=False)["h"]
    q, sb, st = oracle.nv_quantize_per_token(x)
    qn, sbn, stn = oracle.nv_quantize_per_token(x ^ np.uint16(0x8000))
    assert np.array_equal(sbn, sb) and np.array_equal(stn, st)
    assert np.array_equal(qn, q ^ np.uint8(0x88))


def test_zero_row_and_zero_block():
    x = np.zeros((2, 64), np.uint16)
    x[1, :16] = 0x8000
    x[1, 16:32] = workloads.bf16_bits_from_f32(np.full(16, 3.0, np.float32))
    q, sb, st = oracle.nv_quantize_per_token(x)
    assert st[0] == 0.0 and np.all(sb[0] == 0) and np.all(q[0] == 0)
    assert np.all(_unpack(q)[1, :16] == 8)            # negative zeros keep their sign
    assert sb[1, 1] == 0x7E and np.all(sb[1, 2:] == 0)


def test_error_bound_exact():
    """|q*DEC(sb)*s_t - x| <= half the local E2M1 step * D * (1 + 2^-20), or the element
    saturated at 6 (checked in exact arithmetic on normal-range rows)."""
    x = workloads.config3(seed=38, tokens=24, materialize=False)["h"][:, :256]
    q, sb, st = oracle.nv_quantize_per_token(x)
    codes = _unpack(q)
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    for r in range(x.shape[0]):
        s_t = Fraction(float(st[r]))
        for k in range(x.shape[1]):
            c = int(codes[r, k])
            d = exact.e4m3_value(int(sb[r, k // 16])) * s_t
            _, xv = exact.bf16_value(int(x[r, k]))
            qv = grid[c & 7] * d
            step = grid[min((c & 7) + 1, 7)] - grid[c & 7] if (c & 7) < 7 else grid[7] - grid[6]
            assert abs(qv - xv) <= step / 2 * d * (1 + Fraction(1, 1 << 20)) or (c & 7) == 7, (r, k)


def test_grouped_is_flat_and_checks_offsets():
    cfg = workloads.config3(seed=39, tokens=40)
    x, off = cfg["x"], cfg["offsets"]
    q, sb, st, ok = oracle.nv_quantize_per_token_grouped(x, off)
    qf, sbf, stf = oracle.nv_quantize_per_token(x)
    assert ok and np.array_equal(q, qf) and np.array_equal(sb, sbf) and np.array_equal(st, stf)
    bad = off.copy()
    bad[3], bad[4] = bad[4] + 1, bad[3]
    assert not oracle.nv_quantize_per_token_grouped(x, bad)[3]
    short = off.copy()
    short[-1] = x.shape[0] - 1
    assert not oracle.nv_quantize_per_token_grouped(x, short)[3]
    first = off.copy()
    first[0] = 1
    assert not oracle.nv_quantize_per_token_grouped(x, first)[3]


# --------------------------------------------------------------------------- per-group scale

def _golden(name):
    out = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                k, *v = line.split()
                out[k] = [int(t, 16) for t in v]
    return out


def _rand_rows(rng, R, K):
    x = rng.integers(0, 1 << 16, size=(R, K), dtype=np.uint16)
    x[(x & 0x7F80) == 0x7F80] &= 0xBFFF                        # finite only
    return x


def test_per_group_golden():
    g = _golden("nvfp4_group_scale.txt")
    x = np.array([g["x_row0"], g["x_row1"] * 16], np.uint16)
    q, sb, s, ok = oracle.nv_quantize_per_group(x, [0, 2])
    assert ok
    assert s.view(np.uint32)[0] == g["group_scale_f32"][0]
    assert sb[0, 0] == g["sb_row0"][0] and sb[1, 0] == g["sb_row1"][0]
    assert q[0].tolist() == g["q_row0"] and np.all(q[1] == g["q_row1"][0])
    y = oracle.nv_dequantize(q, sb, np.repeat(s, 2))
    assert np.all(y[1] == g["dequant_row1"][0])
    tq, tsb, tst = oracle.nv_quantize_per_token(x)
    assert tsb[1, 0] == g["token_sb_row1"][0]
    assert np.all(oracle.nv_dequantize(tq, tsb, tst)[1] == g["token_dequant_row1"][0])


def test_per_group_with_one_row_per_group_is_per_token():
    rng = np.random.default_rng(21)
    x = _rand_rows(rng, 37, 96)
    q, sb, s, ok = oracle.nv_quantize_per_group(x, np.arange(38))
    tq, tsb, tst = oracle.nv_quantize_per_token(x)
    assert ok
    assert np.array_equal(q, tq) and np.array_equal(sb, tsb)
    assert np.array_equal(s.view(np.uint32), tst.view(np.uint32))


def test_per_group_scale_is_the_largest_token_scale_of_the_group():
    """fl(a / 2688) is non-decreasing in a, so the scale of the group maximum is the
    largest of the rows' per-token scales."""
    rng = np.random.default_rng(22)
    x = _rand_rows(rng, 60, 64)
    x[10:20] = 0                                               # an all-zero group
    off = [0, 10, 20, 20, 41, 60]                              # an empty group too
    q, sb, s, ok = oracle.nv_quantize_per_group(x, off)
    _, _, tst = oracle.nv_quantize_per_token(x)
    assert ok
    for g in range(len(off) - 1):
        lo, hi = off[g], off[g + 1]
        want = np.float32(0) if hi == lo else tst[lo:hi].max()
        assert s[g] == want, g
    assert s[1] == 0 and s[2] == 0


def test_per_group_equals_per_token_when_every_row_holds_the_group_maximum():
    """Put the group's largest magnitude into every row of the group: each row's own scale
    is then the group's, so the bytes must equal the per-token bytes."""
    rng = np.random.default_rng(23)
    x = _rand_rows(rng, 50, 48)
    off = [0, 7, 7, 30, 50]
    for g in range(len(off) - 1):
        lo, hi = off[g], off[g + 1]
        if hi == lo:
            continue
        mags = x[lo:hi] & 0x7FFF
        i, j = np.unravel_index(np.argmax(mags), mags.shape)
        x[lo:hi, 5] = x[lo + i, j]
    q, sb, s, ok = oracle.nv_quantize_per_group(x, off)
    tq, tsb, tst = oracle.nv_quantize_per_token(x)
    assert ok
    assert np.array_equal(q, tq) and np.array_equal(sb, tsb)


def test_per_group_rejects_bad_offsets():
    x = np.zeros((8, 16), np.uint16)
    for off in ([1, 8], [0, 5, 3, 8], [0, 7]):
        assert oracle.nv_quantize_per_group(x, off)[3] is False


# --------------------------------------------------------------------------- routed rows

def test_quantize_then_gather_equals_gather_then_quantize():
    """Per-token scaling is row-local ("Per-token activation scaling": no token's bytes
    depend on other tokens), so quantizing the tokens once and gathering the packed rows
    gives the bytes of quantizing the gathered BF16 rows."""
    rng = np.random.default_rng(31)
    T, K, k = 40, 96, 3
    h = _rand_rows(rng, T, K)
    tok = np.concatenate([rng.permutation(T) for _ in range(k)])     # each token k times
    dst = workloads.scatter_rows(tok, T, k)
    assert np.all(tok[dst] == np.arange(T)[:, None])
    q, sb, st, written = oracle.nv_quantize_per_token_routed(h, dst, T * k)
    assert written.all()
    hq, hsb, hst = oracle.nv_quantize_per_token(h)
    assert np.array_equal(q, hq[tok]) and np.array_equal(sb, hsb[tok])
    assert np.array_equal(st.view(np.uint32), hst[tok].view(np.uint32))
    gq, gsb, gst = oracle.nv_quantize_per_token(h[tok])
    assert np.array_equal(q, gq) and np.array_equal(sb, gsb)


# --------------------------------------------------------------------------- 16x16 tiles

def _unpack(q):
    lo, hi = q & 0xF, q >> 4
    return np.stack([lo, hi], axis=-1).reshape(q.shape[0], -1)


def test_2d_golden():
    g = _golden("nvfp4_2d_tile.txt")
    x = np.full((16, 16), g["x_other"][0], np.uint16)
    x[0, 0] = g["x00"][0]
    q, sb, s, ok = oracle.nv_quantize_2d(x, [0, 16])
    assert ok and sb.shape == (1, 1)
    assert s.view(np.uint32)[0] == g["group_scale_f32"][0] and sb[0, 0] == g["tile_sb"][0]
    assert q[0, 0] == g["q_byte0_row0"][0]
    rest = np.ones(q.shape, bool)
    rest[0, 0] = False
    assert np.all(q[rest] == g["q_other"][0])
    y = oracle.nv_dequantize_2d(q, sb, s, [0, 16])
    assert y[0, 0] == g["dequant00"][0]
    ym = np.ones(y.shape, bool)
    ym[0, 0] = False
    assert np.all(y[ym] == g["dequant_other"][0])
    q1, sb1, s1, _ = oracle.nv_quantize_per_group(x, [0, 16])
    assert np.all(sb1[1:, 0] == g["rowblock_sb_rows1to15"][0])
    assert np.all(oracle.nv_dequantize(q1, sb1, np.repeat(s1, 16))[1:] == g["rowblock_dequant_rows1to15"][0])


def test_2d_transpose_gives_transposed_codes_and_scales():
    """Square blocks: the weight and its transpose share codes and scales (the point of
    two-dimensional blocks is that one quantized copy serves both GEMM orientations)."""
    rng = np.random.default_rng(41)
    w = _rand_rows(rng, 48, 80)
    q, sb, s, ok = oracle.nv_quantize_2d(w, [0, 48])
    qt, sbt, st_, okt = oracle.nv_quantize_2d(np.ascontiguousarray(w.T), [0, 80])
    assert ok and okt
    assert np.array_equal(_unpack(q).T, _unpack(qt))
    assert np.array_equal(sb.T, sbt)
    assert s.view(np.uint32)[0] == st_.view(np.uint32)[0]


def test_2d_with_identical_rows_in_each_tile_equals_1x16_blocks():
    """When the 16 rows of every tile are equal, each 1x16 block has the tile's maximum,
    so the tile scale and codes are those of the per-group 1x16 layout."""
    rng = np.random.default_rng(42)
    base = _rand_rows(rng, 5, 64)
    w = np.repeat(base, 16, axis=0)                            # 80 rows, tiles of equal rows
    off = [0, 32, 32, 80]
    q, sb, s, ok = oracle.nv_quantize_2d(w, off)
    q1, sb1, s1, ok1 = oracle.nv_quantize_per_group(w, off)
    assert ok and ok1
    assert np.array_equal(q, q1)
    assert np.array_equal(np.repeat(sb, 16, axis=0), sb1)
    assert np.array_equal(s.view(np.uint32), s1.view(np.uint32))


def test_2d_rejects_partial_tiles():
    x = np.zeros((32, 32), np.uint16)
    assert oracle.nv_quantize_2d(x, [0, 8, 32])[3] is False              # group not whole tiles
    assert oracle.nv_quantize_2d(np.zeros((24, 32), np.uint16), [0, 24])[3] is False


# --------------------------------------------------------------------------- 16x16 tiles and row groups
# against the exact verifier and a hand-worked multi-tile fixture.  The C oracle walks rows
# and looks up each row's group and tile; exact.py walks group -> tile -> element.  The
# inputs span several tile rows and columns (sb not square) and several groups with
# distinct scales, one of them empty, so a transposed tile lookup or a group walk shifted
# by one row changes bytes (checked below on the same inputs).

def _f32_scales(s):
    return [exact.binary32_value(int(b)) for b in np.asarray(s, np.float32).view(np.uint32)]


def _np_rows(rows, dtype):
    return np.array(rows, dtype=dtype)


def test_2d_multitile_dequant_golden():
    g = _read_golden("nvfp4_2d_multitile.txt")              # strings: offsets are decimal
    off = [int(v) for v in g["offsets"]]
    s = np.array([int(v, 16) for v in g["group_scale_f32"]], np.uint32).view(np.float32)
    q = np.full((32, 24), int(g["q_byte"][0], 16), np.uint8)
    sb = np.array([[int(v, 16) for v in g["sb_row0"]], [int(v, 16) for v in g["sb_row1"]]], np.uint8)
    y = oracle.nv_dequantize_2d(q, sb, s, off)
    for tr in range(2):
        even = [int(v, 16) for v in g["dequant_tilerow%d_even" % tr]]
        odd = [int(v, 16) for v in g["dequant_tilerow%d_odd" % tr]]
        for tc in range(3):
            blk = y[16 * tr:16 * tr + 16, 16 * tc:16 * tc + 16]
            assert np.all(blk[:, 0::2] == even[tc]), (tr, tc)
            assert np.all(blk[:, 1::2] == odd[tc]), (tr, tc)
    assert np.array_equal(_np_rows(exact.nv_dequantize_2d(q.tolist(), sb.tolist(), _f32_scales(s), off),
                                   np.uint16), y)


def _tile_scaled_rows(rng, R, K, log2_range=12):
    """Random finite BF16 with every 16x16 tile scaled by its own power of two, so that
    neighbouring tiles get different E4M3 scales."""
    x = _rand_rows(rng, R, K)
    x &= np.uint16(0x83FF)                                     # exponent field 0..7 ...
    x |= np.uint16(0x3800)                                     # ... moved to 112..119
    shift = rng.integers(-log2_range, log2_range + 1, size=(R // 16, K // 16))
    e = ((x >> 7) & 0xFF).astype(np.int64) + np.repeat(np.repeat(shift, 16, 0), 16, 1)
    return ((x & np.uint16(0x807F)) | (e.astype(np.uint16) << 7)).astype(np.uint16)


def test_2d_quantize_multitile_multigroup_matches_exact():
    rng = np.random.default_rng(51)
    R, K = 48, 48
    x = _tile_scaled_rows(rng, R, K)
    x[16:32, 16:32] = 0                                        # an all-zero tile
    x[32, 40] = 0x4528                                         # 2688 in group 2
    off = [0, 16, 16, 48]                                      # an empty group in between
    q, sb, s, ok = oracle.nv_quantize_2d(x, off)
    assert ok and sb.shape == (3, 3)
    eq, esb, es = exact.nv_quantize_2d(x.tolist(), off)
    assert np.array_equal(q, _np_rows(eq, np.uint8))
    assert np.array_equal(sb, _np_rows(esb, np.uint8))
    assert [exact.binary32_value(int(b))[1] for b in s.view(np.uint32)] == es
    assert len(set(sb.ravel().tolist())) >= 6                  # tile scales differ
    assert len(set(s.tolist())) == 3                           # group scales differ
    y = oracle.nv_dequantize_2d(q, sb, s, off)
    assert np.array_equal(_np_rows(exact.nv_dequantize_2d(eq, esb, _f32_scales(s), off), np.uint16), y)


def _random_2d_layout(seed):
    rng = np.random.default_rng(seed)
    R, K = 64, 48                                              # 4 x 3 tiles
    q = rng.integers(0, 256, size=(R, K // 2), dtype=np.uint8)
    q[(q & 0x7) == 0] |= np.uint8(0x1)                         # no zero codes: every value shows its scale
    q[(q & 0x70) == 0] |= np.uint8(0x10)
    sb = rng.integers(0x08, 0x7F, size=(R // 16, K // 16), dtype=np.uint8)
    off = [0, 16, 16, 48, 64]
    s = np.array([0.75, 1024.0, 3.0 * 2.0 ** -20, 2.0 ** 90], np.float32)
    return q, sb, s, off


def test_2d_dequant_of_random_bytes_matches_exact():
    """Dequantization of arbitrary stored bytes (not only quantizer output): every tile scale
    code 0x08..0x7E, every E2M1 code, four group scales (one group empty)."""
    q, sb, s, off = _random_2d_layout(52)
    y = oracle.nv_dequantize_2d(q, sb, s, off)
    ey = exact.nv_dequantize_2d(q.tolist(), sb.tolist(), _f32_scales(s), off)
    assert np.array_equal(_np_rows(ey, np.uint16), y)


def test_2d_inputs_tell_the_plausible_index_mistakes_apart():
    """The random layout above really exercises the tile lookup and the group walk: a tile
    scale looked up transposed (flat index (k/16) * tiles_r + r/16), or a group walk that
    gives each group's first row to the group before it, changes the bytes."""
    q, sb, s, off = _random_2d_layout(52)
    right = _np_rows(exact.nv_dequantize_2d(q.tolist(), sb.tolist(), _f32_scales(s), off), np.uint16)
    tr, tc = sb.shape
    sb_transposed_lookup = sb.ravel().reshape(tc, tr).T
    wrong_tile = _np_rows(exact.nv_dequantize_2d(q.tolist(), sb_transposed_lookup.tolist(),
                                                 _f32_scales(s), off), np.uint16)
    assert not np.array_equal(wrong_tile, right)
    sb_rows = np.repeat(sb, 16, axis=0).repeat(16, axis=1)[:, ::16]
    shifted = [off[0]] + [o + 1 if 0 < o < off[-1] else o for o in off[1:]]
    wrong_group = _np_rows(exact.nv_dequantize_per_group(q.tolist(), sb_rows.tolist(),
                                                         _f32_scales(s), shifted), np.uint16)
    assert not np.array_equal(wrong_group, right)


def test_per_group_matches_exact():
    rng = np.random.default_rng(53)
    R, K = 40, 48
    x = _rand_rows(rng, R, K)
    x &= np.uint16(0x83FF)
    x |= np.uint16(0x3800)                                     # magnitudes 2^-15 .. 2^-8
    x[7:23] = (x[7:23] & np.uint16(0x807F)) | np.uint16(0x4400)    # group 2 far larger
    x[23:30] = 0                                               # zero rows in group 3
    x[35, 3] = 0x7F7F                                          # BF16 max in group 3
    off = [0, 7, 7, 23, 40]
    q, sb, s, ok = oracle.nv_quantize_per_group(x, off)
    assert ok
    eq, esb, es = exact.nv_quantize_per_group(x.tolist(), off)
    assert np.array_equal(q, _np_rows(eq, np.uint8))
    assert np.array_equal(sb, _np_rows(esb, np.uint8))
    assert [exact.binary32_value(int(b))[1] for b in s.view(np.uint32)] == es
    # the per-group dequant is the per-token one with each row's group scale
    y = oracle.nv_dequantize(q, sb, np.repeat(s, np.diff(off)))
    ey = exact.nv_dequantize_per_group(eq, esb, _f32_scales(s), off)
    assert np.array_equal(_np_rows(ey, np.uint16), y)
