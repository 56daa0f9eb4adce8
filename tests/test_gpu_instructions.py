"""Exhaustive evidence for each gfx950 conversion instruction the kernels use, against the
CPU oracle (the pages' contract: exact byte-level agreement, section "Bit-exact quantizer
contract" of "Towards Blackwell-native 8-bit and 4-bit RL").

* FP4 encode helper (v_cvt_scalef32_pk_fp4_f32, scale 1.0): all 2^32 binary32 inputs.
* BF16 rounding helper (v_cvt_pk_bf16_f32): all 2^32 binary32 inputs.
* MXFP8 encode (v_cvt_scalef32_pk_fp8_bf16): every BF16 value at every E8M0 scale at which
  it can occur in a block, through the rowwise kernel and through the columnwise path of
  the dual kernel (which pairs rows with byte permutes first).
* MXFP8 decode (v_cvt_scalef32_pk_bf16_fp8) and NVFP4 decode (v_cvt_scalef32_pk_f32_fp4)
  have small input spaces and are covered exhaustively by test_gpu_parity.py.
NaN inputs are outside the contract and skipped.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import oracle
from gpu_helpers import assert_same, bits, log, to_dev

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CHUNK = 1 << 28


@pytest.fixture(scope="module")
def probe():
    path = os.path.join(HERE, "probes", "libcvtprobe.so")
    if not os.path.exists(path):
        import sys
        sys.path.insert(0, os.path.join(HERE, "probes"))
        import build_probe
        build_probe.build()
    L = ctypes.CDLL(path)
    for name in ("probe_sweep_e2m1", "probe_sweep_bf16"):
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p]
    return L


NAN_RANGES = [(0x7F800001, 0x80000000), (0xFF800001, 0x100000000)]   # [lo, hi) patterns


def _first_mismatch(got, want, start):
    """Index of the first differing non-NaN input pattern of the chunk, or None."""
    diff = got != want
    for lo, hi in NAN_RANGES:
        a, b = max(lo, start) - start, min(hi, start + got.size) - start
        if a < b:
            diff[a:b] = False
    bad = np.flatnonzero(diff)
    return None if bad.size == 0 else int(bad[0])


def test_fp4_encode_helper_every_binary32(probe):
    out = torch.empty(CHUNK // 2, dtype=torch.uint8, device="cuda")
    for k in range((1 << 32) // CHUNK):
        start = k * CHUNK
        log("fp4 sweep chunk %d" % k)
        assert probe.probe_sweep_e2m1(start, CHUNK, out.data_ptr()) == 0
        h = out.cpu().numpy()
        got = np.stack([h & 0xF, h >> 4], axis=1).reshape(-1)
        want = oracle.enc_e2m1_f32_range(start, CHUNK)
        i = _first_mismatch(got, want, start)
        assert i is None, ("fp4", hex(start + i), got[i], want[i])


def test_bf16_rounding_helper_every_binary32(probe):
    out = torch.empty(CHUNK // 2, dtype=torch.int32, device="cuda")
    for k in range((1 << 32) // CHUNK):
        start = k * CHUNK
        log("bf16 sweep chunk %d" % k)
        assert probe.probe_sweep_bf16(start, CHUNK, out.data_ptr()) == 0
        got = out.cpu().numpy().view(np.uint16)          # little endian: element order kept
        want = oracle.rne_bf16_f32_range(start, CHUNK)
        i = _first_mismatch(got, want, start)
        assert i is None, ("bf16", hex(start + i), hex(got[i]), hex(want[i]))


def _every_value_at_every_scale():
    """Blocks of 32 BF16: for each E8M0 code c in 0..247 one block-maximum element with
    code c (BF16 fields E = c + 7, m = 0x7F; 0x0460 for c = 0) followed by all BF16 values
    whose magnitude does not exceed it, both signs, 31 per block (zero padded)."""
    rows = []
    for c in range(248):
        amax = 0x0460 if c == 0 else ((c + 7) << 7) | 0x7F
        mags = np.arange(0, amax + 1, dtype=np.uint16)
        vals = np.concatenate([mags, mags | np.uint16(0x8000)])
        pad = (-vals.size) % 31
        vals = np.concatenate([vals, np.zeros(pad, np.uint16)]).reshape(-1, 31)
        lead = np.full((vals.shape[0], 1), amax, np.uint16)
        rows.append(np.concatenate([lead, vals], axis=1))
    z = np.concatenate(rows)
    z = np.concatenate([z, np.zeros(((-z.shape[0]) % 32, 32), np.uint16)])
    return z


def test_mxfp8_encode_every_bf16_at_every_scale():
    z = _every_value_at_every_scale()
    log("mx exhaustive: %d blocks" % z.shape[0])
    eq, es = oracle.mx_quantize_rowwise(z)
    assert sorted(set(es[:, 0].tolist())) == list(range(248))
    q_row, s_row, _, _ = bsq.mx_quantize_mxfp8(to_dev(z), "rowwise")
    assert_same("rowwise s", bits(s_row), es)
    assert_same("rowwise q", bits(q_row), eq)
    zt = np.ascontiguousarray(z.T)                       # [32, nblocks]: blocks down columns
    q_row2, s_row2, q_col, s_col = bsq.mx_quantize_mxfp8(to_dev(zt), "both")
    assert_same("colwise s", bits(s_col), es)
    assert_same("colwise q", bits(q_col), eq)
    er, esr = oracle.mx_quantize_rowwise(zt)
    assert_same("dual rowwise q", bits(q_row2), er)
    assert_same("dual rowwise s", bits(s_row2), esr)
