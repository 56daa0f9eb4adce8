"""The C oracle against the numpy implementation on whole workloads (opt-in).

The default CPU suite compares the two implementations on samples of workloads 3-5
(``test_oracle_numpy.py``).  With ``BSQ_FULL_WORKLOADS=1`` this file compares them on every
byte of the workloads instead: every routed row of workload 3, all 128 experts of workload 4
(gate_up and down: per-row NVFP4, rowwise MXFP8, one FP32 scale per tensor with 1x16 and 16x16
blocks, and the dequantizations), and workload 5 whole (both MXFP8 copies of the activations
and of the weights, every routed row in NVFP4).  It takes several minutes on 8 cores; rows are
processed in chunks, which is exact because every step is local to a row (per-token NVFP4,
rowwise MXFP8) or to a 32-row stripe (columnwise MXFP8).  Passages as in
``test_oracle_numpy.py``.
"""
import os

import numpy as np
import pytest

import oracle
import workloads
from oracle import numpy_ref as nr
from test_oracle_numpy import _mx_both, _nv, _same

pytestmark = pytest.mark.skipif(os.environ.get("BSQ_FULL_WORKLOADS") != "1",
                                reason="whole-workload comparison is opt-in (BSQ_FULL_WORKLOADS=1)")

CHUNK = 16384          # rows per comparison (a multiple of 32)


def test_workload3_every_routed_row():
    c3 = workloads.config3(materialize=False)
    h, idx = c3["h"], c3["token_idx"]
    for r0 in range(0, idx.size, CHUNK):
        _nv(h[idx[r0:r0 + CHUNK]])


def test_workload4_every_expert():
    for expert in range(workloads.EXPERTS):
        e = workloads.config4_expert(expert)
        for key in ("gate_up", "down"):
            w = e[key]
            _nv(w)
            q, s = nr.mx_quantize_rowwise(w)
            eq, es = oracle.mx_quantize_rowwise(w)
            _same(key + " q_row", q, eq)
            _same(key + " s_row", s, es)
            _same(key + " dequant", nr.mx_dequantize(eq, es), oracle.mx_dequantize(eq, es))
            off = [0, w.shape[0]]
            for numpy_fn, c_fn in ((nr.nv_quantize_per_group, oracle.nv_quantize_per_group),
                                   (nr.nv_quantize_2d, oracle.nv_quantize_2d)):
                q, sb, sg = numpy_fn(w, off)
                eq, esb, esg, ok = c_fn(w, off)
                assert ok
                _same(key + " group q", q, eq)
                _same(key + " group sb", sb, esb)
                _same(key + " group s", sg.view(np.uint32), esg.view(np.uint32))


def test_workload5_whole():
    c5 = workloads.config5(materialize=False)
    a, w, idx = c5["a"], c5["w"], c5["token_idx"]
    for r0 in range(0, a.shape[0], CHUNK):
        _mx_both(np.ascontiguousarray(a[r0:r0 + CHUNK]))
    _mx_both(w)
    for r0 in range(0, idx.size, CHUNK):
        _nv(a[idx[r0:r0 + CHUNK]])
