"""GPU parity of NVFP4 with 16x16 weight tiles (two-dimensional block scaling) under one
FP32 scale per row group, against the CPU oracle, through the C ABI.

Reading of the pages: two-dimensional block scaling of the weights is one of the four
parts of NVIDIA's NVFP4 pretraining recipe (page "NVIDIA verified the 4-bit NVFP4 format
on a Mamba-Transformer (12B) at 10 trillion tokens"), turned off in Miles ("Towards
Blackwell-native 8-bit and 4-bit RL", section "Try the NVFP4 recipe in Miles"): one E4M3
scale per 16x16 tile, the per-token steps under the group's FP32 scale.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import oracle
from gpu_helpers import Guarded, assert_same, log, mixed_bf16

pytestmark = pytest.mark.gpu


def _two_d_gpu(x_np, off):
    R, K = x_np.shape
    G = len(off) - 1
    x = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).view(torch.bfloat16).cuda()
    offd = torch.tensor(off, dtype=torch.int64, device="cuda")
    q, sb, s = Guarded(R * K // 2), Guarded(R * K // 256), Guarded(4 * G)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rc = bsq.lib().nv_quantize_nvfp4_2d(x.data_ptr(), R, K, offd.data_ptr(), G, q.ptr, sb.ptr, s.ptr,
                                        status.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == bsq.BSQ_OK, bsq.status_string(rc)
    y = Guarded(R * K * 2)
    rc = bsq.lib().nv_dequantize_2d(q.ptr, sb.ptr, s.ptr, offd.data_ptr(), G, R, K, y.ptr,
                                    torch.cuda.current_stream().cuda_stream)
    assert rc == bsq.BSQ_OK, bsq.status_string(rc)
    torch.cuda.synchronize()
    return q, sb, s, y, int(status.item())


CASES = [("one_tile", 16, 16, [0, 16]), ("ragged_k", 48, 80, [0, 48]),
         ("full_strips", 256, 2048, [0, 256]), ("experts", 4 * 64, 768, [0, 64, 128, 128, 192, 256]),
         ("k_4112", 32, 4112, [0, 16, 32]),
         ("many_groups_in_hbm", 1100 * 16, 64, list(range(0, 1100 * 16 + 1, 16)))]


@pytest.mark.parametrize("name,R,K,off", CASES, ids=[c[0] for c in CASES])
def test_2d_matches_oracle(name, R, K, off):
    log("nv 2d %s %dx%d G=%d" % (name, R, K, len(off) - 1))
    x = mixed_bf16(np.random.default_rng(R + 5 * K), R, K, block=16)
    q, sb, s, y, status = _two_d_gpu(x, off)
    assert status == bsq.BSQ_OK
    eq, esb, es, ok = oracle.nv_quantize_2d(x, off)
    assert ok
    assert_same("s_group", s.payload().view(np.uint32), es.view(np.uint32))
    assert_same("sb", sb.payload().reshape(R // 16, K // 16), esb)
    assert_same("q", q.payload().reshape(R, K // 2), eq)
    assert_same("dequant", y.payload().view(np.uint16).reshape(R, K), oracle.nv_dequantize_2d(eq, esb, es, off))


def test_2d_transposed_weight_on_gpu():
    """The GPU's codes and tile scales of W^T are the transposes of those of W."""
    R, K = 96, 160
    w = mixed_bf16(np.random.default_rng(9), R, K, block=16)
    q, sb, s, _, st1 = _two_d_gpu(w, [0, R])
    qt, sbt, s_t, _, st2 = _two_d_gpu(np.ascontiguousarray(w.T), [0, K])
    assert st1 == st2 == bsq.BSQ_OK
    unpack = lambda b, r: np.stack([b & 0xF, b >> 4], axis=-1).reshape(r, -1)
    assert_same("codes", unpack(q.payload().reshape(R, K // 2), R).T, unpack(qt.payload().reshape(K, R // 2), K))
    assert_same("tile scales", sb.payload().reshape(R // 16, K // 16).T, sbt.payload().reshape(K // 16, R // 16))


@pytest.mark.parametrize("off", [[0, 8, 32], [0, 32, 16, 32], [0, 16]], ids=["not_16", "decreasing", "end"])
def test_2d_reports_bad_offsets_and_stays_in_bounds(off):
    x = mixed_bf16(np.random.default_rng(10), 32, 64, block=16)
    q, sb, s, y, status = _two_d_gpu(x, off)
    assert status == bsq.BSQ_ERR_OFFSETS


def test_2d_binding_round_trip():
    R, K = 64, 256
    x = mixed_bf16(np.random.default_rng(11), R, K, block=16)
    xd = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    off = torch.tensor([0, 32, 64], dtype=torch.int64, device="cuda")
    q, sb, s, status = bsq.nv_quantize_nvfp4_2d(xd, off)
    y = bsq.nv_dequantize_2d(q, sb, s, off)
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    eq, esb, es, _ = oracle.nv_quantize_2d(x, [0, 32, 64])
    assert_same("q", q.cpu().numpy(), eq)
    assert_same("y", y.view(torch.int16).cpu().numpy().view(np.uint16), oracle.nv_dequantize_2d(eq, esb, es, [0, 32, 64]))
