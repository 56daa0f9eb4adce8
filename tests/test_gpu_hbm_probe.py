"""The byte-moving probes that `bench.py --hbm-ceiling` times (tests/probes/hbm_probe.hip)
move the bytes they claim to: the copy reproduces its input, the write stores its pattern,
and the two access-pattern probes write the output arrays of the quantizers they stand for
(NVFP4 codes, block and token scales, the dequantized rows and the routed rows of the
scatter; MXFP8 rowwise and columnwise codes and scales), with
the values they are stated to write where those are simple, and nothing around them."""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

from gpu_helpers import log

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "probes"))
import build_probe  # noqa: E402


def _lib():
    if not os.path.exists(build_probe.HBM_LIB):
        pytest.fail("tests/probes/libhbmprobe.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(build_probe.HBM_LIB)


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def test_copy_write_and_read_probes():
    log("hbm probe copy/write/read, 4096 pieces")
    hp = _lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n16 = 4096
    x = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda")
    for nt in (0, 1):
        y = torch.zeros_like(x)
        assert hp.hbm_probe_copy(_p(x), _p(y), ctypes.c_int64(n16), nt, s) == 0
        torch.cuda.synchronize()
        assert torch.equal(x, y)
        assert hp.hbm_probe_write(_p(y), ctypes.c_int64(n16), nt, s) == 0
        torch.cuda.synchronize()
        t = np.arange(n16, dtype=np.uint32)
        want = np.stack([t, t ^ 1, t ^ 2, t ^ 3], axis=1).reshape(-1)
        assert np.array_equal(y.cpu().numpy().view(np.uint32), want)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    assert hp.hbm_probe_read(_p(x), ctypes.c_int64(n16), _p(sink), s) == 0
    assert hp.hbm_probe_copy(_p(x), _p(x), ctypes.c_int64(n16 + 1), 1, s) != 0   # not a multiple of 256
    torch.cuda.synchronize()


def test_nv_pattern_probe_writes_the_quantizers_bytes():
    log("hbm probe NVFP4 pattern, 8256 rows")
    hp = _lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    R, K, pad = 8256, 2048, 4096                   # two rounds of 512-row chunks on 8 XCDs, and 64 more
    x = torch.randint(0, 0x7F80, (R * K,), dtype=torch.int32, device="cuda").to(torch.int16)
    q = torch.full((R * K // 2 + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    sb = torch.full((R * K // 16 + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    st = torch.full((R + 2 * pad // 4,), -7.0, dtype=torch.float32, device="cuda")
    qv, sbv, stv = q[pad:pad + R * K // 2], sb[pad:pad + R * K // 16], st[pad // 4:pad // 4 + R]
    assert hp.hbm_probe_nv_pattern(_p(x), ctypes.c_int64(R), _p(qv), _p(sbv), _p(stv), s) == 0
    torch.cuda.synchronize()
    qh, sbh, sth = q.cpu().numpy(), sb.cpu().numpy(), st.cpu().numpy()
    assert np.all(qh[:pad] == 0xA5) and np.all(qh[pad + R * K // 2:] == 0xA5)
    assert np.all(sbh[:pad] == 0xA5) and np.all(sbh[pad + R * K // 16:] == 0xA5)
    assert np.all(sth[:pad // 4] == -7.0) and np.all(sth[pad // 4 + R:] == -7.0)
    # every code byte written: the probe stores the XOR of each lane's four loaded dwords
    xw = x.cpu().numpy().view(np.uint32).reshape(R, 256, 4)
    want = np.bitwise_xor.reduce(xw, axis=2).astype(np.uint32)
    assert np.array_equal(qh[pad:pad + R * K // 2].view(np.uint32).reshape(R, 256), want)


def test_mx_dual_pattern_probe_writes_both_copies():
    log("hbm probe MXFP8 dual pattern, 256 x 512")
    hp = _lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    M, K, pad = 256, 512, 4096
    x = torch.randint(0, 0x7F80, (M * K,), dtype=torch.int32, device="cuda").to(torch.int16)
    bufs = [torch.full((n + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
            for n in (M * K, M * K // 32, M * K, M * K // 32)]
    views = [b[pad:b.numel() - pad] for b in bufs]
    assert hp.hbm_probe_mx_dual_pattern(_p(x), ctypes.c_int64(M), ctypes.c_int64(K), *map(_p, views), s) == 0
    assert hp.hbm_probe_mx_dual_pattern(_p(x), ctypes.c_int64(M + 32), ctypes.c_int64(K), *map(_p, views), s) != 0
    torch.cuda.synchronize()
    for b in bufs:
        h = b.cpu().numpy()
        assert np.all(h[:pad] == 0xA5) and np.all(h[-pad:] == 0xA5)
    # rowwise copy: 8 bytes a 16-byte piece, the XORs of its dword pairs
    xw = x.cpu().numpy().view(np.uint32).reshape(M, K // 8, 4)
    want = np.stack([xw[..., 0] ^ xw[..., 1], xw[..., 2] ^ xw[..., 3]], axis=-1).reshape(M, K // 4)
    assert np.array_equal(views[0].cpu().numpy().view(np.uint32).reshape(M, K // 4), want)


def test_nv_dequant_pattern_probe_writes_every_piece():
    log("hbm probe NVFP4 dequant pattern, 33 x 2048")
    hp = _lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    R, K, pad = 33, 2048, 4096                     # 8448 half blocks: a partial last workgroup
    q = torch.randint(-2**31, 2**31 - 1, (R * K // 8,), dtype=torch.int32, device="cuda")
    sb = torch.randint(0, 256, (R * K // 16,), dtype=torch.uint8, device="cuda")
    st = torch.randn(R, device="cuda")
    y = torch.full((R * K * 2 + 2 * pad,), 0xA5, dtype=torch.uint8, device="cuda")
    yv = y[pad:pad + R * K * 2]
    assert hp.hbm_probe_nv_dequant_pattern(_p(q), _p(sb), _p(st), ctypes.c_int64(R), ctypes.c_int64(K),
                                           _p(yv), s) == 0
    assert hp.hbm_probe_nv_dequant_pattern(_p(q), _p(sb), _p(st), ctypes.c_int64(R), ctypes.c_int64(K + 8),
                                           _p(yv), s) != 0
    torch.cuda.synchronize()
    yh = y.cpu().numpy()
    assert np.all(yh[:pad] == 0xA5) and np.all(yh[-pad:] == 0xA5)
    h = np.arange(R * K // 8)
    a = (q.cpu().numpy().view(np.uint32) ^ sb.cpu().numpy()[h >> 1].astype(np.uint32)
         ^ st.cpu().numpy().view(np.uint32)[h // (K // 8)])
    want = np.stack([a, a + 1, a + 2, a + 3], axis=1).astype(np.uint32)
    assert np.array_equal(yv.cpu().numpy().view(np.uint32).reshape(-1, 4), want)


def test_scatter_pattern_probe_writes_only_named_rows():
    log("hbm probe scatter pattern, 40 tokens x 2048, top 3 of 130 rows")
    hp = _lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    T, K, k, N = 40, 2048, 3, 130
    rng = np.random.default_rng(5)
    dst_np = rng.permutation(N)[:T * k].reshape(T, k).astype(np.int64)
    dst_np[0, 1] = -1                                    # a dropped choice
    dst_np[1, 2] = N + 3                                 # outside the rows: skipped
    written = np.zeros(N, bool)
    written[dst_np[(dst_np >= 0) & (dst_np < N)]] = True
    x = torch.randint(0, 0x7F80, (T * K,), dtype=torch.int32, device="cuda").to(torch.int16)
    dst = torch.from_numpy(dst_np).cuda()
    q = torch.full((N * K // 2,), 0xA5, dtype=torch.uint8, device="cuda")
    sb = torch.full((N * K // 16,), 0xA5, dtype=torch.uint8, device="cuda")
    st = torch.full((N,), -7.0, dtype=torch.float32, device="cuda")
    assert hp.hbm_probe_scatter_pattern(_p(x), ctypes.c_int64(T), _p(dst), k, ctypes.c_int64(N),
                                        _p(q), _p(sb), _p(st), s) == 0
    assert hp.hbm_probe_scatter_pattern(_p(x), ctypes.c_int64(T), _p(dst), 65, ctypes.c_int64(N),
                                        _p(q), _p(sb), _p(st), s) != 0
    torch.cuda.synchronize()
    qh = q.cpu().numpy().reshape(N, K // 2)
    assert np.all(qh[~written] == 0xA5) and np.all(sb.cpu().numpy().reshape(N, K // 16)[~written] == 0xA5)
    assert np.all(st.cpu().numpy()[~written] == -7.0)
    # each named row holds its token's codes: the XOR of each lane's four loaded dwords
    xw = x.cpu().numpy().view(np.uint32).reshape(T, 256, 4)
    want = np.bitwise_xor.reduce(xw, axis=2).astype(np.uint32)
    for t in range(T):
        for d in dst_np[t]:
            if 0 <= d < N:
                assert np.array_equal(qh[d].view(np.uint32), want[t])
