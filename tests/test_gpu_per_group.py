"""GPU parity of standard NVFP4 with one FP32 scale per row group (a tensor, or an expert's
tensor with gate and up together) against the CPU oracle, through the C ABI.

Reading of "Towards Blackwell-native 8-bit and 4-bit RL", sections "Format background"
(the coarse FP32 scale may cover a tensor instead of a token) and "Per-token activation
scaling" (gate and up share one FP32 scale in export): s_g = fl(amax_g / 2688) over the
group, then the per-token steps under s_g.  Outputs carry sentinel guard bytes.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import oracle
from gpu_helpers import Guarded, assert_same, log, mixed_bf16

pytestmark = pytest.mark.gpu


def _per_group_gpu(x_np, off):
    R, K = x_np.shape
    G = len(off) - 1
    x = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16).cuda()
    offd = torch.tensor(off, dtype=torch.int64, device="cuda")
    q, sb, s = Guarded(R * K // 2), Guarded(R * K // 16), Guarded(4 * G)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rc = bsq.lib().nv_quantize_nvfp4_per_group(x.data_ptr(), R, K, offd.data_ptr(), G, q.ptr, sb.ptr, s.ptr,
                                               status.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == bsq.BSQ_OK, bsq.status_string(rc)
    y = Guarded(R * K * 2)
    rc = bsq.lib().nv_dequantize_per_group(q.ptr, sb.ptr, s.ptr, offd.data_ptr(), G, R, K, y.ptr,
                                           torch.cuda.current_stream().cuda_stream)
    assert rc == bsq.BSQ_OK, bsq.status_string(rc)
    torch.cuda.synchronize()
    return q, sb, s, y, int(status.item())


def _counts_offsets(counts):
    return [0] + np.cumsum(counts).tolist()


def _cases():
    rng = np.random.default_rng(77)
    yield "one_tensor", 96, 2048, [0, 96]
    yield "experts_gate_up", 4 * 48, 512, _counts_offsets([48] * 4)       # K = 512: two rows a wave
    yield "pairs_split_by_groups", 45, 768, _counts_offsets([3, 0, 7, 1, 20, 14])
    yield "odd_rows_short", 33, 48, _counts_offsets([10, 23])
    yield "wide_rows", 7, 8208, _counts_offsets([2, 0, 5])                # two-pass long rows
    yield "k_1536", 40, 1536, _counts_offsets([16, 24])
    tiny = _counts_offsets(rng.integers(0, 4, size=150).tolist())
    yield "tiny_groups", tiny[-1], 64, tiny


CASES = list(_cases())


def _many_groups():
    counts = np.random.default_rng(78).integers(0, 4, size=1500)
    return ("many_groups_in_hbm", int(counts.sum()), 64, _counts_offsets(counts.tolist()))


def _groups_at_lds_starts_limit():
    counts = np.random.default_rng(81).integers(0, 3, size=2048)
    return ("groups_at_lds_starts_limit", int(counts.sum()), 16, _counts_offsets(counts.tolist()))


def _groups_beyond_lds_starts():
    counts = np.random.default_rng(80).integers(0, 3, size=3000)
    return ("groups_beyond_lds_starts", int(counts.sum()), 32, _counts_offsets(counts.tolist()))


def _groups_beyond_lds_table():
    counts = np.random.default_rng(79).integers(0, 3, size=9000)
    return ("groups_beyond_lds_table", int(counts.sum()), 16, _counts_offsets(counts.tolist()))


CASES.append(_many_groups())                  # G <= 2048: group starts and maxima table in LDS
CASES.append(_groups_at_lds_starts_limit())   # G == 2048, the largest LDS-staged count
CASES.append(_groups_beyond_lds_starts())     # 2048 < G <= 8192: maxima table in LDS, starts read from HBM
CASES.append(_groups_beyond_lds_table())      # G > 8192: maxima straight to HBM


@pytest.mark.parametrize("name,R,K,off", CASES, ids=[c[0] for c in CASES])
def test_per_group_matches_oracle(name, R, K, off):
    assert off[-1] == R
    log("nv per group %s %dx%d G=%d" % (name, R, K, len(off) - 1))
    x = mixed_bf16(np.random.default_rng(R * 3 + K), R, K, block=16)
    q, sb, s, y, status = _per_group_gpu(x, off)
    assert status == bsq.BSQ_OK
    eq, esb, es, ok = oracle.nv_quantize_per_group(x, off)
    assert ok
    assert_same("s_group", s.payload().view(np.uint32), es.view(np.uint32))
    assert_same("sb", sb.payload().reshape(R, K // 16), esb)
    assert_same("q", q.payload().reshape(R, K // 2), eq)
    st = np.repeat(es, np.diff(off))                           # each row's group scale
    assert_same("dequant", y.payload().view(np.uint16).reshape(R, K), oracle.nv_dequantize(eq, esb, st))


@pytest.mark.parametrize("off", [[1, 30, 64], [0, 40, 30, 64], [0, 63]], ids=["first", "decreasing", "end"])
def test_per_group_reports_bad_offsets_and_stays_in_bounds(off):
    x = mixed_bf16(np.random.default_rng(5), 64, 256, block=16)
    q, sb, s, y, status = _per_group_gpu(x, off)
    assert status == bsq.BSQ_ERR_OFFSETS


def test_per_group_empty_tensor_gives_zero_scales():
    offd = torch.zeros(4, dtype=torch.int64, device="cuda")
    s = torch.full((3,), 7.0, dtype=torch.float32, device="cuda")
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rc = bsq.lib().nv_quantize_nvfp4_per_group(None, 0, 64, offd.data_ptr(), 3, None, None, s.data_ptr(),
                                               status.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == bsq.BSQ_OK
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK and torch.all(s == 0)


def test_per_group_binding_round_trip():
    R, K = 64, 256
    x = mixed_bf16(np.random.default_rng(6), R, K, block=16)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    off = torch.tensor([0, 20, 64], dtype=torch.int64, device="cuda")
    q, sb, s, status = bsq.nv_quantize_nvfp4_per_group(xd, off)
    y = bsq.nv_dequantize_per_group(q, sb, s, off)
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    eq, esb, es, _ = oracle.nv_quantize_per_group(x, [0, 20, 64])
    assert_same("q", q.cpu().numpy(), eq)
    assert_same("y", y.view(torch.int16).cpu().numpy().view(np.uint16),
                oracle.nv_dequantize(eq, esb, np.repeat(es, [20, 44])))
