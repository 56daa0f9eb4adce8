"""The C oracle against a second, independent implementation at the sizes of the workloads.

``oracle/numpy_ref.py`` is written separately from the same format definitions and
readings (vectorized numpy, binary32 steps as numpy float32 operations); the exact-rational
verifier pins the C oracle on tiny inputs, this one on the workloads' own tensors: workloads
1 and 2 whole, and for 3-5 samples chosen so that every kind of block is present -- every
8th routed row of workload 3, whole experts of workload 4 (gate_up and down), every 16th
32-row stripe of workload 5's activations (whole 32x1 blocks), its weights whole and 1% of
its routed rows.  Every output byte (codes, scales, token scales, dequantized BF16) must be
equal.  Passages: page "Towards Blackwell-native 8-bit and 4-bit RL", sections "Format
background", "Recipe 1: end-to-end MXFP8 RL", "Per-token activation scaling" and
"High-precision and dequantized backward"; two-dimensional weight blocks: page "NVIDIA
verified the 4-bit NVFP4 format on a Mamba-Transformer (12B) at 10 trillion tokens".
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle import numpy_ref as nr


def _same(name, a, b):
    assert a.shape == b.shape, (name, a.shape, b.shape)
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b)
        raise AssertionError("%s: %d entries differ, first at %s" % (name, len(bad), bad[0].tolist()))


def _mx_both(x):
    qr, sr = nr.mx_quantize_rowwise(x)
    qc, sc = nr.mx_quantize_colwise(x)
    eqr, esr = oracle.mx_quantize_rowwise(x)
    eqc, esc = oracle.mx_quantize_colwise(x)
    _same("q_row", qr, eqr); _same("s_row", sr, esr)
    _same("q_col", qc, eqc); _same("s_col", sc, esc)
    _same("dequant row", nr.mx_dequantize(eqr, esr), oracle.mx_dequantize(eqr, esr))
    _same("dequant col", nr.mx_dequantize(eqc, esc), oracle.mx_dequantize(eqc, esc))


def _nv(x):
    q, sb, st = nr.nv_quantize_per_token(x)
    eq, esb, est = oracle.nv_quantize_per_token(x)
    _same("q", q, eq); _same("sb", sb, esb); _same("st", st.view(np.uint32), est.view(np.uint32))
    _same("nv dequant", nr.nv_dequantize(eq, esb, est), oracle.nv_dequantize(eq, esb, est))


def test_workload1_whole():
    x = workloads.config1()["x"]
    q, s = nr.mx_quantize_rowwise(x)
    eq, es = oracle.mx_quantize_rowwise(x)
    _same("q_row", q, eq); _same("s_row", s, es)
    _same("dequant", nr.mx_dequantize(eq, es), oracle.mx_dequantize(eq, es))


def test_workload2_whole():
    x = workloads.config2()["x"]
    _mx_both(x)
    _nv(x)                                                 # the same activations under NVFP4


def test_workload3_every_8th_routed_row():
    c3 = workloads.config3(materialize=False)
    x = c3["h"][c3["token_idx"][::8]]
    _nv(x)


@pytest.mark.parametrize("expert", [0, 77, 127])
def test_workload4_whole_experts(expert):
    e = workloads.config4_expert(expert)
    for key in ("gate_up", "down"):
        w = e[key]
        _nv(w)
        q, s = nr.mx_quantize_rowwise(w)
        eq, es = oracle.mx_quantize_rowwise(w)
        _same(key + " q_row", q, eq); _same(key + " s_row", s, es)
        _same(key + " dequant", nr.mx_dequantize(eq, es), oracle.mx_dequantize(eq, es))
        # one FP32 scale for the whole tensor (gate and up together), 1x16 and 16x16 blocks
        off = [0, w.shape[0]]
        for numpy_fn, c_fn in ((nr.nv_quantize_per_group, oracle.nv_quantize_per_group),
                               (nr.nv_quantize_2d, oracle.nv_quantize_2d)):
            q, sb, sg = numpy_fn(w, off)
            eq, esb, esg, ok = c_fn(w, off)
            assert ok
            _same(key + " group q", q, eq); _same(key + " group sb", sb, esb)
            _same(key + " group s", sg.view(np.uint32), esg.view(np.uint32))


def test_workload5_samples():
    c5 = workloads.config5(materialize=False)
    a = c5["a"]
    stripes = a.reshape(-1, 32, a.shape[1])[::16]           # every 16th 32-row stripe
    _mx_both(np.ascontiguousarray(stripes.reshape(-1, a.shape[1])))
    _mx_both(c5["w"])
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(c5["token_idx"].size, size=c5["token_idx"].size // 100, replace=False))
    _nv(a[c5["token_idx"][rows]])


def test_per_group_and_2d_on_several_groups():
    """Several groups of different magnitudes (gate_up of three experts stacked), checked
    against the C oracle's per-group and 16x16-tile layouts."""
    parts = [workloads.config4_expert(e)["gate_up"] for e in (1, 2, 3)]
    parts[1] = (parts[1] & np.uint16(0x807F)) | np.uint16(0x3C00)     # a group of larger values
    w = np.concatenate(parts)
    off = [0, 1536, 3072, 4608]
    for numpy_fn, c_fn in ((nr.nv_quantize_per_group, oracle.nv_quantize_per_group),
                           (nr.nv_quantize_2d, oracle.nv_quantize_2d)):
        q, sb, sg = numpy_fn(w, off)
        eq, esb, esg, ok = c_fn(w, off)
        assert ok
        _same("q", q, eq); _same("sb", sb, esb); _same("s", sg.view(np.uint32), esg.view(np.uint32))
    # the 16x16 layout dequantizes as 1x16 blocks that repeat each tile's scale on its 16 rows
    q, sb, sg = nr.nv_quantize_2d(w, off)
    _same("2d dequant", oracle.nv_dequantize_2d(q, sb, sg, off),
          nr.nv_dequantize(q, np.repeat(sb, 16, axis=0), np.repeat(sg, np.diff(off))))
