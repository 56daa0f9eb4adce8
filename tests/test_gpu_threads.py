"""Calls from several host threads at once, each on its own stream.  The library keeps no
state between calls (no allocation, no synchronisation, no global buffers), so concurrent
calls on different streams must give exactly the bytes of one call at a time."""
import threading

import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
from gpu_helpers import log, mixed_bf16

pytestmark = pytest.mark.gpu


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


GROUPED_S_COL = 10                                         # index of the grouped s_col in _run_all's list


def _run_all(x, off, stream):
    """One call of every kind on x; returns the outputs as uint8 tensors."""
    outs = []
    outs += bsq.mx_quantize_mxfp8(x, "both", stream=stream)
    q, sb, st = bsq.nv_quantize_nvfp4_per_token(x, stream=stream)
    outs += [q, sb, st.view(torch.uint8)]
    qr, sr, qc, sc, status = bsq.mx_quantize_mxfp8_grouped(x, off, "both", stream=stream)
    outs += [qr, sr, qc, sc]
    outs.append(bsq.mx_dequantize(outs[0], outs[1], stream=stream).view(torch.uint8))
    outs.append(bsq.nv_dequantize(q, sb, st, stream=stream).view(torch.uint8))
    return outs


def test_concurrent_host_threads_match_sequential_calls():
    n_threads, reps = 4, 3
    rng = np.random.default_rng(77)
    inputs = []
    for i in range(n_threads):
        M, K = 1024 + 128 * i, 512
        cuts = np.sort(rng.choice(np.arange(1, M), 15, replace=False))
        off = torch.from_numpy(np.concatenate([[0], cuts, [M]]).astype(np.int64)).cuda()
        inputs.append((_bf16(mixed_bf16(rng, M, K)), off))
    main = torch.cuda.current_stream()
    expected = [[t.clone() for t in _run_all(x, off, main)] for x, off in inputs]
    torch.cuda.synchronize()

    results, errors = [None] * n_threads, []

    def run(i):
        try:
            s = torch.cuda.Stream()
            x, off = inputs[i]
            with torch.cuda.stream(s):
                for _ in range(reps):
                    got = _run_all(x, off, s)
            s.synchronize()
            results[i] = got
        except Exception as e:            # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(n_threads)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    torch.cuda.synchronize()
    log("threads done")
    for i in range(n_threads):
        assert results[i] is not None
        off = inputs[i][1].cpu().numpy()
        nb = int(((np.diff(off) + 31) // 32).sum())
        for j, (u, v) in enumerate(zip(results[i], expected[i])):
            if j == GROUPED_S_COL:                         # entries past the last block are not written
                u, v = u[:, :nb], v[:, :nb]
            assert torch.equal(u.view(torch.uint8), v.view(torch.uint8)), (i, j)
