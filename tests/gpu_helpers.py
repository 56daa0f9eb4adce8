"""Helpers of the GPU parity tests: device transfer of BF16 bit patterns, outputs with
sentinel guard bytes, and input mixtures covering the test-data kinds the pages name for
quantizer tests (random, boundary, zeros, maxes; page "Towards Blackwell-native 8-bit and
4-bit RL", section "Bit-exact quantizer contract")."""
from __future__ import annotations

import sys

import numpy as np
import torch

import workloads

SENTINEL = 0xA5
GUARD = 256


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x_bits: np.ndarray) -> torch.Tensor:
    """numpy uint16 BF16 bit patterns -> torch.bfloat16 on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16))
    return t.view(torch.bfloat16).to("cuda:0")


def bits(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy bit patterns (uint16 for 2-byte dtypes, uint32 for f32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype in (torch.bfloat16, torch.float16, torch.int16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float32, torch.int32):
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.numpy()


def assert_same(name: str, got: np.ndarray, want: np.ndarray) -> None:
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if not np.array_equal(got, want):
        bad = np.argwhere(got != want)
        i = tuple(bad[0])
        raise AssertionError("%s: %d of %d entries differ; first at %s: got %s want %s"
                             % (name, len(bad), got.size, list(i), got[i], want[i]))


class Guarded:
    """A device byte buffer with GUARD sentinel bytes on each side of the payload."""

    def __init__(self, nbytes: int):
        self.n = nbytes
        self.buf = torch.full((nbytes + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda:0")

    @property
    def ptr(self) -> int:
        return self.buf.data_ptr() + GUARD

    def payload(self) -> np.ndarray:
        h = self.buf.cpu().numpy()
        assert np.all(h[:GUARD] == SENTINEL) and np.all(h[GUARD + self.n:] == SENTINEL), \
            "write outside the output buffer"
        return h[GUARD:GUARD + self.n]


# ---------------------------------------------------------------------------------------

def _mids(values):
    v = np.asarray(values, dtype=np.float64)
    return (v[:-1] + v[1:]) / 2


E4M3_POS = np.array([(m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
                     for e in range(16) for m in range(8)][:127])
E2M1_POS = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def mixed_bf16(rng, rows: int, cols: int, block: int = 32) -> np.ndarray:
    """BF16 bit patterns [rows, cols] mixing, per row, one of: random normal with a random
    binade, random finite bit patterns, zeros (signed), maxes (448*2^k / 2688*2^k / BF16
    max), E4M3 or E2M1 midpoints times a power of two, BF16 subnormals, and sparse
    outliers."""
    out = np.empty((rows, cols), np.uint16)
    for r in range(rows):
        kind = r % 8
        if kind == 0:
            v = rng.standard_normal(cols) * np.exp2(rng.integers(-125, 120))
            out[r] = workloads.bf16_bits_from_f32(v.astype(np.float32))
        elif kind == 1:
            b = rng.integers(0, 1 << 16, cols).astype(np.uint16)
            b[(b & 0x7F80) == 0x7F80] &= np.uint16(0xBFFF)
            out[r] = b
        elif kind == 2:
            b = np.zeros(cols, np.uint16)
            b[rng.random(cols) < 0.5] = 0x8000
            out[r] = b
        elif kind == 3:
            base = 448.0 if rng.random() < 0.5 else 2688.0
            v = np.full(cols, base * 2.0 ** int(rng.integers(-128, 115)), np.float32)
            b = workloads.bf16_bits_from_f32(v)
            if rng.random() < 0.4:
                b[rng.integers(cols)] = 0x7F7F
            b[rng.random(cols) < 0.5] |= np.uint16(0x8000)
            out[r] = b
        elif kind == 4:   # E4M3 midpoints with the block max fixing the scale at 2^e
            e = int(rng.integers(-120, 110))
            v = rng.choice(_mids(E4M3_POS), cols) * 2.0 ** e
            v[::block] = 448.0 * 2.0 ** e
            v *= np.where(rng.random(cols) < 0.5, -1, 1)
            out[r] = workloads.bf16_bits_from_f32(v.astype(np.float32))
        elif kind == 5:   # E2M1 midpoints and grid values
            v = rng.choice(np.concatenate([_mids(E2M1_POS), E2M1_POS]), cols)
            v = v * 2.0 ** int(rng.integers(-30, 30))
            v *= np.where(rng.random(cols) < 0.5, -1, 1)
            out[r] = workloads.bf16_bits_from_f32(v.astype(np.float32))
        elif kind == 6:   # BF16 subnormals
            b = rng.integers(0, 0x80, cols).astype(np.uint16)
            b[rng.random(cols) < 0.5] |= np.uint16(0x8000)
            out[r] = b
        else:             # small values with sparse huge outliers
            v = rng.standard_normal(cols) * 1e-3
            k = max(1, cols // 97)
            v[rng.integers(0, cols, k)] = rng.standard_normal(k) * 3e4
            out[r] = workloads.bf16_bits_from_f32(v.astype(np.float32))
    return out
