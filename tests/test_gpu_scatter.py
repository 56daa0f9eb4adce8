"""GPU parity of quantize-then-scatter for routed rows (per-token NVFP4 of X[dst[t, j]] =
H[t] without gathering X) against the CPU oracle's gather-then-quantize, through the C ABI.

Page "Towards Blackwell-native 8-bit and 4-bit RL", section "Per-token activation
scaling": a token's bytes depend on that token only, so the two orders give the same bytes.
Outputs carry sentinel guard bytes; rows that no entry names must stay untouched.
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import oracle
import workloads
from gpu_helpers import SENTINEL, Guarded, assert_same, log, mixed_bf16

pytestmark = pytest.mark.gpu


def _scatter_gpu(h_np, dst, N):
    T, K = h_np.shape
    h = torch.from_numpy(np.ascontiguousarray(h_np).view(np.int16)).view(torch.bfloat16).cuda()
    dd = torch.from_numpy(np.ascontiguousarray(dst, dtype=np.int64)).cuda()
    q, sb, st = Guarded(N * K // 2), Guarded(N * K // 16), Guarded(4 * N)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    rc = bsq.lib().nv_quantize_nvfp4_per_token_scatter(h.data_ptr(), T, K, dd.data_ptr(), dst.shape[1], N,
                                                       q.ptr, sb.ptr, st.ptr, status.data_ptr(),
                                                       torch.cuda.current_stream().cuda_stream)
    assert rc == bsq.BSQ_OK, bsq.status_string(rc)
    torch.cuda.synchronize()
    return q, sb, st, int(status.item())


def _routing(rng, T, k, drop=0.0, spare=0):
    """Each token to k distinct rows of a routed layout of T*k + spare rows (random order);
    a fraction `drop` of the choices is dropped (-1)."""
    N = T * k + spare
    dst = rng.permutation(N)[:T * k].reshape(T, k).astype(np.int64)
    if drop:
        dst[rng.random(dst.shape) < drop] = -1
    return dst, N


CASES = [("k2048", 33, 2048, 8, 0.0, 0), ("k768_pairs_odd", 45, 768, 4, 0.0, 0),
         ("k48_dropped", 64, 48, 3, 0.25, 17), ("k8208_long", 5, 8208, 2, 0.0, 3),
         ("k1536", 40, 1536, 8, 0.1, 0), ("k256_pairs_even", 50, 256, 6, 0.0, 0),
         # more than 32 destinations a token: the destination rows are read in chunks of 32
         ("k2048_top40", 9, 2048, 40, 0.1, 5), ("k768_pairs_top33", 11, 768, 33, 0.0, 0),
         ("k512_pairs_top64", 6, 512, 64, 0.2, 1)]


@pytest.mark.parametrize("name,T,K,k,drop,spare", CASES, ids=[c[0] for c in CASES])
def test_scatter_matches_gather_then_quantize(name, T, K, k, drop, spare):
    log("nv scatter %s T=%d K=%d top_k=%d" % (name, T, K, k))
    rng = np.random.default_rng(T * 7 + K)
    h = mixed_bf16(rng, T, K, block=16)
    dst, N = _routing(rng, T, k, drop, spare)
    q, sb, st, status = _scatter_gpu(h, dst, N)
    assert status == bsq.BSQ_OK
    eq, esb, est, written = oracle.nv_quantize_per_token_routed(h, dst, N)
    gq, gsb, gst = q.payload().reshape(N, K // 2), sb.payload().reshape(N, K // 16), st.payload().view(np.uint32)
    assert_same("q", gq[written], eq[written])
    assert_same("sb", gsb[written], esb[written])
    assert_same("st", gst[written], est.view(np.uint32)[written])
    assert np.all(gq[~written] == SENTINEL) and np.all(gsb[~written] == SENTINEL)
    assert np.all(st.payload().reshape(N, 4)[~written] == SENTINEL)


def test_scatter_reports_rows_beyond_n_and_skips_them():
    rng = np.random.default_rng(3)
    T, K, k = 16, 256, 2
    h = mixed_bf16(rng, T, K, block=16)
    dst, N = _routing(rng, T, k)
    dst[3, 1] = N + 5
    q, sb, st, status = _scatter_gpu(h, dst, N)
    assert status == bsq.BSQ_ERR_OFFSETS
    dst[3, 1] = -1
    eq, esb, est, written = oracle.nv_quantize_per_token_routed(h, dst, N)
    assert_same("q", q.payload().reshape(N, K // 2)[written], eq[written])


def test_scatter_binding_and_workload_map():
    rng = np.random.default_rng(4)
    T, K, k = 64, 512, 8
    tok, _ = workloads.zipf_routing(rng, T, 128, k)
    dst = workloads.scatter_rows(tok, T, k)
    h = mixed_bf16(rng, T, K, block=16)
    hd = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).cuda()
    q, sb, st, status = bsq.nv_quantize_nvfp4_per_token_scatter(hd, torch.from_numpy(dst).cuda(), T * k)
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    eq, esb, est = oracle.nv_quantize_per_token(h[tok])       # gather, then quantize
    assert_same("q", q.cpu().numpy(), eq)
    assert_same("sb", sb.cpu().numpy(), esb)
