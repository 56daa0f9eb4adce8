"""GPU parity at the full sizes of the five workloads (seeded synthetic inputs shaped like
a Qwen3-30B-A3B-class MoE layer; recipes in workloads/__init__.py), with the same launch
configuration the benchmark times.  Every output byte is compared with the CPU oracle
(the quantize-then-scatter rows against the grouped path on every byte, and against the
oracle on a seeded sample of rows).
"""
import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import oracle
import workloads
from gpu_helpers import assert_same, bits, log, to_dev

pytestmark = pytest.mark.gpu


def _check_mx(name, x_np, xd, mode):
    M, K = x_np.shape
    q_row, s_row, q_col, s_col = bsq.mx_quantize_mxfp8(xd, mode)
    if q_row is not None:
        eq, es = oracle.mx_quantize_rowwise(x_np)
        assert_same(name + " q_row", bits(q_row), eq)
        assert_same(name + " s_row", bits(s_row), es)
        assert_same(name + " dequant row", bits(bsq.mx_dequantize(q_row, s_row)),
                    oracle.mx_dequantize(eq, es))
    if q_col is not None:
        eq, es = oracle.mx_quantize_colwise(x_np)
        assert_same(name + " q_col", bits(q_col), eq)
        assert_same(name + " s_col", bits(s_col), es)
        assert_same(name + " dequant col", bits(bsq.mx_dequantize(q_col, s_col)),
                    oracle.mx_dequantize(eq, es))


def _check_nv(name, x_np, q, sb, st, y):
    eq, esb, est = oracle.nv_quantize_per_token(x_np)
    assert_same(name + " st", bits(st), est.view(np.uint32))
    assert_same(name + " sb", bits(sb), esb)
    assert_same(name + " q", bits(q), eq)
    assert_same(name + " dequant", bits(y), oracle.nv_dequantize(eq, esb, est))


def test_config1_mxfp8_rowwise_256x2048():
    log("config1")
    x = workloads.config1()["x"]
    _check_mx("config1", x, to_dev(x), "rowwise")


def test_config2_mxfp8_dual_8192x2048_and_dequant():
    log("config2")
    x = workloads.config2()["x"]
    _check_mx("config2", x, to_dev(x), "both")


def test_config3_nvfp4_grouped_131072x2048():
    log("config3: generating")
    cfg = workloads.config3()
    x, off = cfg["x"], cfg["offsets"]
    assert x.shape == (131072, 2048) and off.shape == (129,)
    xd = to_dev(x)
    q, sb, st, status = bsq.nv_quantize_nvfp4_per_token_grouped(xd, torch.from_numpy(off).cuda())
    y = bsq.nv_dequantize(q, sb, st)
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    log("config3: comparing")
    _check_nv("config3", x, q, sb, st, y)


def test_config4_weight_export_128_experts():
    log("config4: generating")
    cfg = workloads.config4()
    for key, shape in (("gate_up", (196608, 2048)), ("down", (262144, 768))):
        w = cfg[key]
        assert w.shape == shape
        wd = to_dev(w)
        log("config4 %s: nvfp4" % key)
        q, sb, st = bsq.nv_quantize_nvfp4_per_token(wd)
        y = bsq.nv_dequantize(q, sb, st)
        _check_nv("config4 " + key, w, q, sb, st, y)
        del q, sb, st, y
        log("config4 %s: mxfp8 rowwise" % key)
        _check_mx("config4 " + key, w, wd, "rowwise")
        del wd


def test_config4_weight_export_one_scale_per_expert():
    """Standard NVFP4 export of the 128 experts with one FP32 scale per expert tensor: the
    fused gate/up projection of an expert is one group (1536 rows, gate and up sharing one
    scale), the down projection another (2048 rows).  Every output byte is compared."""
    log("config4 per-expert scale: generating")
    cfg = workloads.config4()
    for key, rows in (("gate_up", 1536), ("down", 2048)):
        w = cfg[key]
        off = np.arange(0, w.shape[0] + 1, rows, dtype=np.int64)
        assert off[-1] == w.shape[0] and off.size == 129
        offd = torch.from_numpy(off).cuda()
        log("config4 %s: nvfp4 per expert" % key)
        q, sb, s, status = bsq.nv_quantize_nvfp4_per_group(to_dev(w), offd)
        y = bsq.nv_dequantize_per_group(q, sb, s, offd)
        torch.cuda.synchronize()
        assert int(status.item()) == bsq.BSQ_OK
        eq, esb, es, ok = oracle.nv_quantize_per_group(w, off)
        assert ok
        assert_same(key + " s_group", bits(s), es.view(np.uint32))
        assert_same(key + " sb", bits(sb), esb)
        assert_same(key + " q", bits(q), eq)
        assert_same(key + " dequant", bits(y), oracle.nv_dequantize(eq, esb, np.repeat(es, rows)))
        del q, sb, s, y


def test_config4_weight_export_16x16_tiles():
    """The 128 experts' weights with 16x16 tiles and one FP32 scale per expert tensor (gate
    and up together).  Every output byte is compared."""
    log("config4 2d: generating")
    cfg = workloads.config4()
    for key, rows in (("gate_up", 1536), ("down", 2048)):
        w = cfg[key]
        off = np.arange(0, w.shape[0] + 1, rows, dtype=np.int64)
        offd = torch.from_numpy(off).cuda()
        log("config4 %s: nvfp4 16x16" % key)
        q, sb, s, status = bsq.nv_quantize_nvfp4_2d(to_dev(w), offd)
        y = bsq.nv_dequantize_2d(q, sb, s, offd)
        torch.cuda.synchronize()
        assert int(status.item()) == bsq.BSQ_OK
        eq, esb, es, ok = oracle.nv_quantize_2d(w, off)
        assert ok
        assert_same(key + " s_group", bits(s), es.view(np.uint32))
        assert_same(key + " sb", bits(sb), esb)
        assert_same(key + " q", bits(q), eq)
        assert_same(key + " dequant", bits(y), oracle.nv_dequantize_2d(eq, esb, es, off))
        del q, sb, s, y


def test_config5_layer_step_stream():
    log("config5: generating")
    cfg = workloads.config5()
    a, w, tok, off = cfg["a"], cfg["w"], cfg["token_idx"], cfg["offsets"]
    assert a.shape == (65536, 2048) and w.shape == (2048, 6144) and tok.shape == (524288,)
    ad, wd = to_dev(a), to_dev(w)
    tokd = torch.from_numpy(tok).cuda()
    xd = ad.index_select(0, tokd)                      # routed rows, gathered on the device
    # the step: MX dual on A and W, NV grouped on X, then dequant of every output
    a_q = bsq.mx_quantize_mxfp8(ad, "both")
    w_q = bsq.mx_quantize_mxfp8(wd, "both")
    q, sb, st, status = bsq.nv_quantize_nvfp4_per_token_grouped(xd, torch.from_numpy(off).cuda())
    ya_r, ya_c = bsq.mx_dequantize(a_q[0], a_q[1]), bsq.mx_dequantize(a_q[2], a_q[3])
    yw_r, yw_c = bsq.mx_dequantize(w_q[0], w_q[1]), bsq.mx_dequantize(w_q[2], w_q[3])
    yx = bsq.nv_dequantize(q, sb, st)
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK

    log("config5: comparing W")
    ew = oracle.mx_quantize_rowwise(w), oracle.mx_quantize_colwise(w)
    assert_same("W q_row", bits(w_q[0]), ew[0][0])
    assert_same("W s_row", bits(w_q[1]), ew[0][1])
    assert_same("W q_col", bits(w_q[2]), ew[1][0])
    assert_same("W s_col", bits(w_q[3]), ew[1][1])
    assert_same("W dequant row", bits(yw_r), oracle.mx_dequantize(*ew[0]))
    assert_same("W dequant col", bits(yw_c), oracle.mx_dequantize(*ew[1]))

    log("config5: comparing A")
    er = oracle.mx_quantize_rowwise(a)
    assert_same("A q_row", bits(a_q[0]), er[0])
    assert_same("A s_row", bits(a_q[1]), er[1])
    assert_same("A dequant row", bits(ya_r), oracle.mx_dequantize(*er))
    del er
    ec = oracle.mx_quantize_colwise(a)
    assert_same("A q_col", bits(a_q[2]), ec[0])
    assert_same("A s_col", bits(a_q[3]), ec[1])
    assert_same("A dequant col", bits(ya_c), oracle.mx_dequantize(*ec))
    del ec

    log("config5: comparing all 524288 routed rows")
    eq, esb, est = oracle.nv_quantize_per_token(a[tok])
    assert_same("X st", bits(st), est.view(np.uint32))
    assert_same("X sb", bits(sb), esb)
    assert_same("X q", bits(q), eq)
    assert_same("X dequant", bits(yx), oracle.nv_dequantize(eq, esb, est))
    del eq, esb, est
    # duplicated tokens (a token routed to 8 experts) give byte-identical rows
    first = {}
    for i, t in enumerate(tok[:4096]):
        first.setdefault(int(t), i)
    pairs = [(first[int(t)], i) for i, t in enumerate(tok[:4096]) if first[int(t)] != i][:256]
    if pairs:
        i0 = torch.tensor([p[0] for p in pairs], device="cuda")
        i1 = torch.tensor([p[1] for p in pairs], device="cuda")
        assert torch.equal(q.index_select(0, i0), q.index_select(0, i1))


def test_config5_routed_rows_mxfp8_grouped_by_expert():
    """The layer step's 524288 routed rows as the MoE weight-gradient operand: MXFP8 with
    32x1 blocks confined to each of the 128 expert segments (Zipf-routed, so nearly every
    segment ends with a partial block), rowwise copy fused.  Every byte compared."""
    log("config5 grouped: generating")
    cfg = workloads.config5()
    a, tok, off = cfg["a"], cfg["token_idx"], cfg["offsets"]
    xd = to_dev(a).index_select(0, torch.from_numpy(tok).cuda())
    q_row, s_row, q_col, s_col, status = bsq.mx_quantize_mxfp8_grouped(
        xd, torch.from_numpy(off).cuda(), "both")
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    assert np.count_nonzero(np.diff(off) % 32) > 100           # partial blocks everywhere
    del xd
    log("config5 grouped: comparing every column")
    x = a[tok]
    eq, es, ok = oracle.mx_quantize_colwise_grouped(x, off)
    assert ok
    assert_same("X q_col", bits(q_col), eq)
    assert_same("X s_col", bits(s_col)[:, :es.shape[1]], es)
    del eq, es
    log("config5 grouped: comparing every row")
    er, esr = oracle.mx_quantize_rowwise(x)
    assert_same("X q_row", bits(q_row), er)
    assert_same("X s_row", bits(s_row), esr)


def test_config5_routed_rows_by_quantize_then_scatter():
    """The layer step's 524288 routed rows produced from the 65536 tokens directly: each
    token quantized once and written to its 8 routed rows.  Compared with the CPU oracle
    (gather, then quantize) on a seeded sample of rows, and with the direct path (gather in
    BF16, grouped quantize) on every byte."""
    log("config5 scatter: generating")
    cfg = workloads.config5()
    a, tok, off = cfg["a"], cfg["token_idx"], cfg["offsets"]
    dst = workloads.scatter_rows(tok, a.shape[0], 8)
    ad = to_dev(a)
    q, sb, st, status = bsq.nv_quantize_nvfp4_per_token_scatter(ad, torch.from_numpy(dst).cuda(), tok.size)
    xq, xsb, xst, xstatus = bsq.nv_quantize_nvfp4_per_token_grouped(
        ad.index_select(0, torch.from_numpy(tok).cuda()), torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK and int(xstatus.item()) == bsq.BSQ_OK
    assert torch.equal(q, xq) and torch.equal(sb, xsb) and torch.equal(st.view(torch.int32), xst.view(torch.int32))
    log("config5 scatter: comparing sampled rows")
    rows = np.sort(np.random.default_rng(58).choice(tok.size, 8192, replace=False))
    eq, esb, est = oracle.nv_quantize_per_token(a[tok[rows]])
    rows_d = torch.from_numpy(rows).cuda()
    assert_same("scatter q", bits(q.index_select(0, rows_d)), eq)
    assert_same("scatter sb", bits(sb.index_select(0, rows_d)), esb)
    assert_same("scatter st", bits(st.index_select(0, rows_d)), est.view(np.uint32))
