"""GPU parity: every byte the HIP kernels write, through the C ABI, equals the CPU oracle's.

Shapes span several tiles with ragged tails (rows not a multiple of the tile, K not a
multiple of 128 or 512); outputs carry sentinel guard bytes on both sides to catch
out-of-range writes; inputs mix the four test-data kinds the pages name (random,
boundary, zeros, maxes) with BF16 subnormals and outliers.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import oracle
from gpu_helpers import Guarded, assert_same, bits, log, mixed_bf16, to_dev

pytestmark = pytest.mark.gpu


def _mx_gpu(x_np, mode):
    """Run mx_quantize_mxfp8 through the C ABI with guarded outputs."""
    M, K = x_np.shape
    x = to_dev(x_np)
    n = M * K
    qr, sr, qc, sc = Guarded(n), Guarded(n // 32), Guarded(n), Guarded(n // 32)
    st = bsq.lib().mx_quantize_mxfp8(x.data_ptr(), M, K, mode, qr.ptr, sr.ptr, qc.ptr, sc.ptr,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == bsq.BSQ_OK, bsq.status_string(st)
    torch.cuda.synchronize()
    return qr, sr, qc, sc


MX_ROW_SHAPES = [(1, 32), (3, 64), (7, 96), (33, 2048), (64, 4128), (257, 160), (5, 16384)]
MX_COL_SHAPES = [(32, 32), (64, 96), (96, 288), (160, 64), (256, 2048), (4128, 96), (32, 6176)]


@pytest.mark.parametrize("M,K", MX_ROW_SHAPES)
def test_mx_rowwise_matches_oracle(M, K):
    log("mx rowwise %dx%d" % (M, K))
    x = mixed_bf16(np.random.default_rng(M * 7919 + K), M, K)
    qr, sr, qc, sc = _mx_gpu(x, bsq.MX_ROWWISE)
    eq, es = oracle.mx_quantize_rowwise(x)
    assert_same("q_row", qr.payload().reshape(M, K), eq)
    assert_same("s_row", sr.payload().reshape(M, K // 32), es)
    assert np.all(qc.payload() == 0xA5) and np.all(sc.payload() == 0xA5)   # not touched


@pytest.mark.parametrize("mode", [bsq.MX_COLWISE, bsq.MX_BOTH])
@pytest.mark.parametrize("M,K", MX_COL_SHAPES)
def test_mx_colwise_and_both_match_oracle(M, K, mode):
    log("mx mode %d %dx%d" % (mode, M, K))
    x = mixed_bf16(np.random.default_rng(M * 31 + K + mode), M, K)
    qr, sr, qc, sc = _mx_gpu(x, mode)
    eqc, esc = oracle.mx_quantize_colwise(x)
    assert_same("q_col", qc.payload().reshape(K, M), eqc)
    assert_same("s_col", sc.payload().reshape(K, M // 32), esc)
    if mode == bsq.MX_BOTH:
        eqr, esr = oracle.mx_quantize_rowwise(x)
        assert_same("q_row", qr.payload().reshape(M, K), eqr)
        assert_same("s_row", sr.payload().reshape(M, K // 32), esr)
    else:
        assert np.all(qr.payload() == 0xA5) and np.all(sr.payload() == 0xA5)


@pytest.mark.parametrize("M,K", [(64, 8), (96, 40), (160, 72), (64, 6184), (8192, 4104)])
def test_mx_colwise_with_k_not_a_multiple_of_32(M, K):
    """The columnwise copy's blocks run along M, so it takes any K of whole 16-byte rows:
    the tile's last column group is ragged at 8-column granularity (and 8192 x 4104 runs
    the persistent form, 1088 tiles)."""
    log("mx colwise %dx%d" % (M, K))
    x = mixed_bf16(np.random.default_rng(M * 131 + K), M, K)
    qr, sr, qc, sc = _mx_gpu(x, bsq.MX_COLWISE)
    eqc, esc = oracle.mx_quantize_colwise(x)
    assert_same("q_col", qc.payload().reshape(K, M), eqc)
    assert_same("s_col", sc.payload().reshape(K, M // 32), esc)
    assert np.all(qr.payload() == 0xA5) and np.all(sr.payload() == 0xA5)
    y = bsq.mx_dequantize(torch.from_numpy(eqc).cuda(), torch.from_numpy(esc).cuda())
    assert_same("dequant", bits(y), oracle.mx_dequantize(eqc, esc))


@pytest.mark.parametrize("mode", [bsq.MX_COLWISE, bsq.MX_BOTH])
@pytest.mark.parametrize("M,K", [(65568, 2048), (8224, 2048), (65536, 2080)])
def test_mx_rows_or_columns_off_the_line_grid(M, K, mode):
    """M % 128 == 32 puts every q_col row off 128-byte line boundaries (the tile's columns are
    stored non-temporally only inside lines they cover whole); K % 128 == 32 does the same to
    q_row.  Full-size tensors, so nearly every workgroup has such shared lines."""
    log("mx mode %d %dx%d (off the line grid)" % (mode, M, K))
    x = mixed_bf16(np.random.default_rng(M + 7 * K + mode), M, K)
    qr, sr, qc, sc = _mx_gpu(x, mode)
    eqc, esc = oracle.mx_quantize_colwise(x)
    assert_same("q_col", qc.payload().reshape(K, M), eqc)
    assert_same("s_col", sc.payload().reshape(K, M // 32), esc)
    del eqc, esc
    if mode == bsq.MX_BOTH:
        eqr, esr = oracle.mx_quantize_rowwise(x)
        assert_same("q_row", qr.payload().reshape(M, K), eqr)
        assert_same("s_row", sr.payload().reshape(M, K // 32), esr)


def test_mx_both_on_a_tensor_with_tiles_beyond_31_bit_offsets():
    """M = 2^23 + 32 rows: a workgroup tile of the columnwise copy then spans more than
    2^31 bytes of q_col, so the kernel addresses with 64-bit offsets (and the tile grid
    is ragged in both directions)."""
    M, K = (1 << 23) + 32, 32
    log("mx both %dx%d" % (M, K))
    rng = np.random.default_rng(23)
    x = rng.integers(0, 1 << 16, size=(M, K), dtype=np.uint16)
    x[(x & 0x7F80) == 0x7F80] &= 0xBFFF                       # finite inputs only
    x[rng.integers(0, M, size=4096)] = 0                       # some all-zero rows
    qr, sr, qc, sc = _mx_gpu(x, bsq.MX_BOTH)
    eqc, esc = oracle.mx_quantize_colwise(x)
    assert_same("q_col", qc.payload().reshape(K, M), eqc)
    assert_same("s_col", sc.payload().reshape(K, M // 32), esc)
    del eqc, esc
    eqr, esr = oracle.mx_quantize_rowwise(x)
    assert_same("q_row", qr.payload().reshape(M, K), eqr)
    assert_same("s_row", sr.payload().reshape(M, K // 32), esr)


def test_mx_rowwise_differs_from_colwise_on_gpu():
    """The handmade 32x32 example: row 0 all 1024, the rest 0.01 (see tests/golden)."""
    x = np.full((32, 32), 0x3C24, np.uint16)
    x[0] = 0x4480
    q_row, s_row, q_col, s_col = bsq.mx_quantize_mxfp8(to_dev(x), "both")
    assert np.all(bits(s_row)[1:] == 0x70) and np.all(bits(q_row)[1:] == 0x7A)
    assert np.all(bits(s_col) == 0x81) and np.all(bits(q_col)[:, 1:] == 0x01)
    assert np.all(bits(q_row)[0] == 0x78) and np.all(bits(q_col)[:, 0] == 0x78)


def test_mx_dequant_every_code_and_scale():
    """All 256 E4M3 codes x all 256 E8M0 codes (NaN codes included)."""
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))          # [scale][code]
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    qd, sd = torch.from_numpy(q).cuda(), torch.from_numpy(s).cuda()
    y = Guarded(256 * 256 * 2)
    st = bsq.lib().mx_dequantize(qd.data_ptr(), sd.data_ptr(), 256, 256, y.ptr,
                                 torch.cuda.current_stream().cuda_stream)
    assert st == bsq.BSQ_OK
    torch.cuda.synchronize()
    got = y.payload().view(np.uint16).reshape(256, 256)
    assert_same("mx dequant", got, oracle.mx_dequantize(q, s))


@pytest.mark.parametrize("M,K", [(1, 32), (33, 2048), (130, 96), (64, 6176)])
def test_mx_dequant_round_trip_matches_oracle(M, K):
    x = mixed_bf16(np.random.default_rng(5 + M + K), M, K)
    q_row, s_row, _, _ = bsq.mx_quantize_mxfp8(to_dev(x), "rowwise")
    y = bsq.mx_dequantize(q_row, s_row)
    eq, es = oracle.mx_quantize_rowwise(x)
    assert_same("mx dequant", bits(y), oracle.mx_dequantize(eq, es))


# short rows go two to a wave: odd row counts leave a one-row tail span, and even counts
# with K = 256, 512, 768 fill whole register slots
NV_SHAPES = [(1, 16), (5, 32), (3, 48), (8, 64), (6, 256), (9, 512), (10, 512), (17, 768),
             (16, 768), (2, 768), (4, 1040), (33, 2048), (2, 4096), (3, 4112), (2, 8208),
             (4096, 1040), (8229, 1040),   # one-row spans dealt to the XCDs in 512-row chunks, and a tail
             (4096, 512), (8197, 768)]     # two-row spans, the same chunks, a tail and an odd last row


@pytest.mark.parametrize("R,K", NV_SHAPES)
def test_nv_quant_matches_oracle(R, K):
    log("nv quant %dx%d" % (R, K))
    x = mixed_bf16(np.random.default_rng(R * 131 + K), R, K, block=16)
    xd = to_dev(x)
    q, sb, st = Guarded(R * K // 2), Guarded(R * K // 16), Guarded(R * 4)
    rc = bsq.lib().nv_quantize_nvfp4_per_token(xd.data_ptr(), R, K, q.ptr, sb.ptr, st.ptr,
                                               torch.cuda.current_stream().cuda_stream)
    assert rc == bsq.BSQ_OK
    torch.cuda.synchronize()
    eq, esb, est = oracle.nv_quantize_per_token(x)
    assert_same("st", st.payload().view(np.uint32), est.view(np.uint32))
    assert_same("sb", sb.payload().reshape(R, K // 16), esb)
    assert_same("q", q.payload().reshape(R, K // 2), eq)


def test_nv_dequant_every_code_scale_and_token_scale():
    codes = np.tile(np.arange(16, dtype=np.uint8), 256)
    qrow = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    st_vals = np.array([1.0, 2.0 ** -140, 3.1e-5, 7.7e30, 0.0, 1 / 3, 2.0 ** -126, 1e-45,
                        3.0e38, np.inf, np.nan, 123.456], np.float32)
    R = st_vals.size
    q = np.tile(qrow, (R, 1))
    sb = np.tile(np.arange(256, dtype=np.uint8), (R, 1))
    y = bsq.nv_dequantize(torch.from_numpy(q).cuda(), torch.from_numpy(sb).cuda(),
                          torch.from_numpy(st_vals).cuda())
    assert_same("nv dequant", bits(y), oracle.nv_dequantize(q, sb, st_vals))


@pytest.mark.parametrize("R,K", [(7, 768), (33, 2048), (3, 4112)])
def test_nv_dequant_round_trip_matches_oracle(R, K):
    x = mixed_bf16(np.random.default_rng(R + K), R, K, block=16)
    q, sb, st = bsq.nv_quantize_nvfp4_per_token(to_dev(x))
    y = bsq.nv_dequantize(q, sb, st)
    eq, esb, est = oracle.nv_quantize_per_token(x)
    assert_same("nv dequant", bits(y), oracle.nv_dequantize(eq, esb, est))


def test_nv_grouped_equals_flat_and_reports_offsets():
    rng = np.random.default_rng(3)
    R, K, E = 300, 2048, 16
    x = mixed_bf16(rng, R, K, block=16)
    xd = to_dev(x)
    counts = rng.multinomial(R, np.ones(E) / E)
    counts[3] = 0                                              # an empty expert
    counts[4] += R - counts.sum()
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    qf, sbf, stf = bsq.nv_quantize_nvfp4_per_token(xd)
    q, sb, st, status = bsq.nv_quantize_nvfp4_per_token_grouped(xd, torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    assert torch.equal(q, qf) and torch.equal(sb, sbf) and torch.equal(st.view(torch.int32), stf.view(torch.int32))
    for bad in ([1] + list(off[1:]), list(off[:-1]) + [R + 1], list(off[:5]) + [off[6], off[5]] + list(off[7:])):
        b = torch.tensor(bad, dtype=torch.int64, device="cuda")
        _, _, _, status = bsq.nv_quantize_nvfp4_per_token_grouped(xd, b)
        torch.cuda.synchronize()
        assert int(status.item()) == bsq.BSQ_ERR_OFFSETS, bad
    # zero rows: only the offsets are checked
    x0 = torch.empty(0, K, dtype=torch.bfloat16, device="cuda")
    _, _, _, status = bsq.nv_quantize_nvfp4_per_token_grouped(
        x0, torch.zeros(E + 1, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK


def test_per_token_invariance_on_gpu():
    rng = np.random.default_rng(4)
    x = mixed_bf16(rng, 64, 2048, block=16)
    q, sb, st = (bits(t) for t in bsq.nv_quantize_nvfp4_per_token(to_dev(x)))
    perm = rng.permutation(64)
    y = x[perm].copy()
    y[1::2] = mixed_bf16(rng, 32, 2048, block=16)            # change every other row
    q2, sb2, st2 = (bits(t) for t in bsq.nv_quantize_nvfp4_per_token(to_dev(y)))
    keep = perm[0::2]
    assert np.array_equal(q2[0::2], q[keep]) and np.array_equal(sb2[0::2], sb[keep])
    assert np.array_equal(st2[0::2], st[keep])


def test_deterministic_and_stream_independent():
    x = to_dev(mixed_bf16(np.random.default_rng(9), 512, 2048))
    a = bsq.mx_quantize_mxfp8(x, "both")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = bsq.mx_quantize_mxfp8(x, "both")
        c = bsq.nv_quantize_nvfp4_per_token(x)
    s.synchronize()
    d = bsq.nv_quantize_nvfp4_per_token(x)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    for u, v in zip(c, d):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))


def test_zero_sized_calls():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    q_row, s_row, q_col, s_col = bsq.mx_quantize_mxfp8(x, "both")
    assert q_row.shape == (0, 64) and q_col.shape == (64, 0)
    q, sb, st = bsq.nv_quantize_nvfp4_per_token(x)
    assert q.shape == (0, 32)
    torch.cuda.synchronize()
