"""The library inside a captured HIP graph: it allocates, clears and synchronises nothing
itself (flags and maxima are cleared by its own kernels), so a whole step of calls can be
captured once and replayed.  Every replay, with eager work and synchronisations between
the replays, must reproduce the eager results byte for byte."""
import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import workloads
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def test_captured_step_replays_match_eager():
    rng = np.random.default_rng(61)
    M, K = 4096, 1024
    x = _bf16(workloads.bf16_bits_from_f32((rng.standard_normal((M, K)) * 3).astype(np.float32)))
    cuts = np.sort(rng.choice(np.arange(1, M), 39, replace=False))    # 40 segments, most off 32-row lines
    off_np = np.concatenate([[0], cuts, [M]]).astype(np.int64)
    off = torch.from_numpy(off_np).cuda()
    T, k = 512, 8
    h = x[:T].contiguous()
    dst = torch.from_numpy(rng.permutation(T * k).reshape(T, k).astype(np.int64)).cuda()
    u8, f32 = torch.uint8, torch.float32
    s_ld = bsq.mx_group_scale_entries(M, len(off_np) - 1)
    n_blocks = int(sum((b - a + 31) // 32 for a, b in zip(off_np[:-1], off_np[1:])))
    outs = {
        "mx": [torch.empty(M, K, dtype=u8, device="cuda"), torch.empty(M, K // 32, dtype=u8, device="cuda"),
               torch.empty(K, M, dtype=u8, device="cuda"), torch.empty(K, M // 32, dtype=u8, device="cuda")],
        "mxg": [torch.empty(M, K, dtype=u8, device="cuda"), torch.empty(M, K // 32, dtype=u8, device="cuda"),
                torch.empty(K, M, dtype=u8, device="cuda"), torch.empty(K, s_ld, dtype=u8, device="cuda"),
                torch.empty(1, dtype=torch.int32, device="cuda")],
        "nv": [torch.empty(M, K // 2, dtype=u8, device="cuda"), torch.empty(M, K // 16, dtype=u8, device="cuda"),
               torch.empty(M, dtype=f32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda")],
        "pg": [torch.empty(M, K // 2, dtype=u8, device="cuda"), torch.empty(M, K // 16, dtype=u8, device="cuda"),
               torch.empty(len(off_np) - 1, dtype=f32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda")],
        "sc": [torch.empty(T * k, K // 2, dtype=u8, device="cuda"), torch.empty(T * k, K // 16, dtype=u8, device="cuda"),
               torch.empty(T * k, dtype=f32, device="cuda"), torch.empty(1, dtype=torch.int32, device="cuda")],
        "y": [torch.empty(M, K, dtype=torch.bfloat16, device="cuda"), torch.empty(K, M, dtype=torch.bfloat16, device="cuda"),
              torch.empty(M, K, dtype=torch.bfloat16, device="cuda"), torch.empty(M, K, dtype=torch.bfloat16, device="cuda")],
    }

    def step(stream):
        mx, mxg, nv, pg, sc, y = (outs[n] for n in ("mx", "mxg", "nv", "pg", "sc", "y"))
        bsq.mx_quantize_mxfp8(x, "both", *mx, stream=stream)
        bsq.mx_quantize_mxfp8_grouped(x, off, "both", s_ld, *mxg, stream=stream)
        bsq.nv_quantize_nvfp4_per_token_grouped(x, off, *nv, stream=stream)
        bsq.nv_quantize_nvfp4_per_group(x, off, *pg, stream=stream)
        bsq.nv_quantize_nvfp4_per_token_scatter(h, dst, T * k, *sc, stream=stream)
        bsq.mx_dequantize(mx[0], mx[1], y[0], stream=stream)
        bsq.mx_dequantize(mx[2], mx[3], y[1], stream=stream)
        bsq.nv_dequantize(nv[0], nv[1], nv[2], y[2], stream=stream)
        bsq.nv_dequantize_per_group(pg[0], pg[1], pg[2], off, y[3], stream=stream)

    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        step(side)                                         # eager, also warms up
    torch.cuda.synchronize()
    eager = {n: [t.clone() for t in ts] for n, ts in outs.items()}
    for n in ("mxg", "nv", "pg", "sc"):
        assert int(eager[n][-1].item()) == bsq.BSQ_OK, n

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        step(torch.cuda.current_stream())
    for rep in range(3):
        for ts in outs.values():                           # eager work between the replays
            for t in ts:
                t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log("graph replay %d" % rep)
        for n, ts in outs.items():
            for i, (t, e) in enumerate(zip(ts, eager[n])):
                if n == "mxg" and i == 3:                      # entries past the last block are not written
                    t, e = t[:, :n_blocks], e[:, :n_blocks]
                assert torch.equal(t.view(torch.uint8), e.view(torch.uint8)), "replay %d: %s[%d]" % (rep, n, i)
