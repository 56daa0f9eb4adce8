"""GPU parity of the grouped MXFP8 quantizer (32x1 blocks confined to expert segments, for
the MoE weight-gradient operand) against the CPU oracle, through the C ABI.

Reading of "Towards Blackwell-native 8-bit and 4-bit RL", section "Recipe 1: end-to-end
MXFP8 RL": experts run their weight-gradient GEMM in MXFP8 on the columnwise copy, each
over its own rows, so blocks never cross an expert boundary and an expert whose row count
is not a multiple of 32 ends with a partial block.  Every output carries sentinel guard
bytes; scale entries past the last block must stay untouched.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import oracle
from gpu_helpers import SENTINEL, Guarded, assert_same, log, mixed_bf16

pytestmark = pytest.mark.gpu


def _grouped_gpu(x_np, off, mode, s_ld):
    M, K = x_np.shape
    x = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16).cuda()
    offd = torch.tensor(off, dtype=torch.int64, device="cuda")
    n = M * K
    qr, sr = Guarded(n), Guarded(n // 32)
    qc, sc = Guarded(n), Guarded(K * s_ld)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rc = bsq.lib().mx_quantize_mxfp8_grouped(x.data_ptr(), M, K, mode, offd.data_ptr(), len(off) - 1,
                                             qr.ptr, sr.ptr, qc.ptr, sc.ptr, s_ld, status.data_ptr(),
                                             torch.cuda.current_stream().cuda_stream)
    assert rc == bsq.BSQ_OK, bsq.status_string(rc)
    torch.cuda.synchronize()
    return qr, sr, qc, sc, int(status.item())


def _counts_offsets(counts):
    return [0] + np.cumsum(counts).tolist()


def _cases():
    rng = np.random.default_rng(2024)
    yield "aligned", 256, 64, _counts_offsets([32, 0, 96, 64, 64])
    yield "one_expert_partial_tail", 70, 64, [0, 70]
    yield "unaligned", 200, 96, _counts_offsets([3, 0, 37, 1, 34, 0, 45, 80])
    tiny = _counts_offsets(rng.integers(0, 6, size=24).tolist() + [0])
    yield "tiny_experts", tiny[-1], 256, tiny
    yield "empty_ends", 161, 288, _counts_offsets([0, 0, 33, 128, 0, 0])
    yield "many", 5000, 512, _counts_offsets(np.diff(np.sort(np.concatenate(
        [[0, 5000], rng.integers(0, 5000, size=36)]))).tolist())
    yield "aligned_16", 1024, 256, _counts_offsets([16, 48, 112, 0, 336, 512])
    # whole 128-row windows and 256-column groups, segments off the 32-row grid whose blocks
    # all hold 16 rows or more: blocks reach across windows on both sides, from one segment
    # or from two
    counts = rng.integers(40, 400, size=40)
    counts = np.where((counts % 32 > 0) & (counts % 32 < 16), counts + 16, counts)
    counts = counts[np.cumsum(counts) <= 8192 - 48].tolist()
    counts.append(8192 - sum(counts))
    yield "whole_windows_off_grid", 8192, 512, _counts_offsets(counts)
    # the same segments over eight 256-column groups
    yield "whole_windows_off_grid_wide", 8192, 2048, _counts_offsets(counts)
    # M % 128 == 32: the q_col rows start off line boundaries, so each window's run of a
    # column shares its first and last line with the neighbouring windows (stored the
    # ordinary way, the covered lines non-temporally)
    cut = _counts_offsets(counts)
    cut = [min(o, 8192 - 96) for o in cut]
    yield "rows_off_line_grid_wide", 8192 - 96, 2048, cut


CASES = list(_cases())


def _check_grouped(x, off, mode):
    M, K = x.shape
    nb = int(oracle.mx_group_blocks(off).sum())
    s_ld = nb + 3                                              # room past the last block
    qr, sr, qc, sc, status = _grouped_gpu(x, off, mode, s_ld)
    assert status == bsq.BSQ_OK
    eq, es, ok = oracle.mx_quantize_colwise_grouped(x, off)
    assert ok
    assert_same("q_col", qc.payload().reshape(K, M), eq)
    s = sc.payload().reshape(K, s_ld)
    assert_same("s_col", s[:, :nb], es)
    assert np.all(s[:, nb:] == SENTINEL), "scale entries past the last block were written"
    if mode == bsq.MX_BOTH:
        eqr, esr = oracle.mx_quantize_rowwise(x)
        assert_same("q_row", qr.payload().reshape(M, K), eqr)
        assert_same("s_row", sr.payload().reshape(M, K // 32), esr)
    else:
        assert np.all(qr.payload() == SENTINEL) and np.all(sr.payload() == SENTINEL)
    if all((b - a) % 32 == 0 for a, b in zip(off[:-1], off[1:])):
        fq, fs = oracle.mx_quantize_colwise(x)                 # aligned segments: the flat copy
        assert_same("q_col vs flat", qc.payload().reshape(K, M), fq)
        assert_same("s_col vs flat", s[:, :nb], fs)


@pytest.mark.parametrize("mode", [bsq.MX_COLWISE, bsq.MX_BOTH])
@pytest.mark.parametrize("name,M,K,off", CASES, ids=[c[0] for c in CASES])
def test_grouped_matches_oracle(name, M, K, off, mode):
    assert off[-1] == M
    log("mx grouped %s %dx%d E=%d mode %d" % (name, M, K, len(off) - 1, mode))
    x = mixed_bf16(np.random.default_rng(M * 13 + K + mode), M, K)
    _check_grouped(x, off, mode)


def _random_counts(rng, M):
    """Segment lengths mixing the cases the kernel tells apart: empty experts, 1-15 rows,
    16-31 rows, a few rows either side of a multiple of 32, and long segments."""
    counts, total = [], 0
    while total < M:
        kind = int(rng.integers(0, 5))
        if kind == 0:
            c = 0
        elif kind == 1:
            c = int(rng.integers(1, 16))
        elif kind == 2:
            c = int(rng.integers(16, 32))
        elif kind == 3:
            c = int(32 * rng.integers(1, 5) + rng.integers(-2, 3))
        else:
            c = int(rng.integers(33, 300))
        c = min(c, M - total)
        counts.append(c)
        total += c
    return counts


@pytest.mark.parametrize("mode", [bsq.MX_COLWISE, bsq.MX_BOTH])
@pytest.mark.parametrize("seed", range(8))
def test_grouped_random_segments(seed, mode):
    """Random segment mixes over whole and ragged windows and column groups."""
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.choice([640, 1024, 1500, 2048, 3001]))
    K = int(rng.choice([32, 160, 256, 512]))
    off = _counts_offsets(_random_counts(rng, M))
    log("mx grouped random seed %d %dx%d E=%d mode %d" % (seed, M, K, len(off) - 1, mode))
    x = mixed_bf16(rng, M, K)
    _check_grouped(x, off, mode)


@pytest.mark.parametrize("mode", [bsq.MX_COLWISE, bsq.MX_BOTH])
def test_grouped_more_than_2_pow_23_rows(mode):
    """q_col past 2^31 bytes from its base with 1000 segments of random length (most not
    multiples of 32): 64-bit addressing in both modes of the grouped kernel."""
    M, K = (1 << 23) + 48, 32
    log("mx grouped large %dx%d mode %d" % (M, K, mode))
    rng = np.random.default_rng(29)
    x = rng.integers(0, 1 << 16, size=(M, K), dtype=np.uint16)
    x[(x & 0x7F80) == 0x7F80] &= 0xBFFF                       # finite inputs only
    off = [0] + np.sort(rng.choice(np.arange(1, M), size=999, replace=False)).tolist() + [M]
    nb = int(oracle.mx_group_blocks(off).sum())
    qr, sr, qc, sc, status = _grouped_gpu(x, off, mode, nb)
    assert status == bsq.BSQ_OK
    eq, es, ok = oracle.mx_quantize_colwise_grouped(x, off)
    assert ok
    assert_same("q_col", qc.payload().reshape(K, M), eq)
    assert_same("s_col", sc.payload().reshape(K, nb), es)
    del eq, es
    if mode == bsq.MX_BOTH:
        eqr, esr = oracle.mx_quantize_rowwise(x)
        assert_same("q_row", qr.payload().reshape(M, K), eqr)
        assert_same("s_row", sr.payload().reshape(M, K // 32), esr)


@pytest.mark.parametrize("mode", [bsq.MX_COLWISE, bsq.MX_BOTH])
@pytest.mark.parametrize("off", [[1, 30, 64], [0, 40, 30, 64], [0, 30, 63], [0, 30, 70]],
                         ids=["first", "decreasing", "short_end", "long_end"])
def test_grouped_reports_bad_offsets_and_stays_in_bounds(off, mode):
    M, K = 64, 64
    x = mixed_bf16(np.random.default_rng(7), M, K)
    qr, sr, qc, sc, status = _grouped_gpu(x, off, mode, 8)
    assert status == bsq.BSQ_ERR_OFFSETS
    for g in (qr, sr, qc, sc):
        g.payload()                                            # guard bytes intact


def test_grouped_reports_too_few_scale_entries():
    M, K = 96, 64
    off = _counts_offsets([1, 1, 1, 93])                       # 1 + 1 + 1 + 3 = 6 blocks
    x = mixed_bf16(np.random.default_rng(8), M, K)
    qr, sr, qc, sc, status = _grouped_gpu(x, off, bsq.MX_COLWISE, 3)   # ceil(96/32) = 3 < 6
    assert status == bsq.BSQ_ERR_OFFSETS
    sc.payload()                                               # nothing past s_ld
    eq, es, ok = oracle.mx_quantize_colwise_grouped(x, off)
    assert_same("first blocks", sc.payload().reshape(K, 3), es[:, :3])


def test_grouped_status_for_an_empty_tensor():
    x = np.zeros((0, 64), np.uint16)
    x_d = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    for off, want in (([0, 0, 0], bsq.BSQ_OK), ([0, 1, 0], bsq.BSQ_ERR_OFFSETS)):
        offd = torch.tensor(off, dtype=torch.int64, device="cuda")
        status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        dummy = torch.empty(16, dtype=torch.uint8, device="cuda")
        rc = bsq.lib().mx_quantize_mxfp8_grouped(x_d.data_ptr(), 0, 64, bsq.MX_COLWISE, offd.data_ptr(),
                                                 len(off) - 1, None, None, dummy.data_ptr(),
                                                 dummy.data_ptr(), 0, status.data_ptr(),
                                                 torch.cuda.current_stream().cuda_stream)
        assert rc == bsq.BSQ_OK
        torch.cuda.synchronize()
        assert int(status.item()) == want
    del x


def test_grouped_binding_round_trip():
    M, K = 130, 64
    off = [0, 5, 130]
    x = mixed_bf16(np.random.default_rng(9), M, K)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    q_row, s_row, q_col, s_col, status = bsq.mx_quantize_mxfp8_grouped(
        xd, torch.tensor(off, dtype=torch.int64, device="cuda"), "both")
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    assert s_col.shape == (K, bsq.mx_group_scale_entries(M, 2))
    eq, es, _ = oracle.mx_quantize_colwise_grouped(x, off)
    assert_same("q_col", q_col.cpu().numpy(), eq)
    assert_same("s_col", s_col.cpu().numpy()[:, :es.shape[1]], es)
