"""Seeded synthetic inputs for the block-scaled quantizer contract.

This module only makes input tensors.  It holds none of the quantizer's arithmetic, so
both the HIP path and the CPU oracle can consume exactly the same tensors.  BF16 tensors
are numpy ``uint16`` arrays of bit patterns.

The shapes follow a Qwen3-30B-A3B-class MoE layer (hidden 2048, 128 routed experts,
top-8 routing, expert FFN width 768 so gate_up is 1536 wide), the workload the pages'
ablation runs on (section "Results: Qwen3-30B-A3B recipe ablation on 8x B200").  The
dataset and trained weights of that ablation are not used: these are stand-ins with the
same shapes and with value distributions chosen to exercise the format (wide per-row
dynamic range, outliers, all-zero blocks, heavy-tailed token magnitudes, skewed expert
load).

Recipes (all draws from ``numpy.random.default_rng``; float32 arithmetic; the final
float32 value is rounded to BF16 with round-to-nearest-even):

* ``config1``  seed 0: X[256,2048] ~ N(0,1); 8 distinct uniform positions scaled x1000;
  then one uniform (row, 32-column block) set to zero.
* ``config2``  seed 1: X[8192,2048] = N(0,1) * sigma_r, sigma_r = 10^U(-3,2) per row;
  round(0.001 * numel) distinct uniform positions scaled x100.
* ``config3``  seed 2: H[16384,2048] = N(0,1) * m_t, m_t ~ LogNormal(0, 2) per token;
  router logits N(0,1)[16384,128]; each token goes to its 8 largest logits (the top-8 of
  the softmax; ties to the lower expert id); the routed rows are H gathered in (expert,
  token) order -> X[131072,2048]; offsets int64[129] = exclusive cumsum of expert counts.
* ``config4``  seed 3: for each of 128 experts (own stream ``default_rng([3, e])``):
  gate_up W[1536,2048] and down W[2048,768] ~ N(0, 0.02), round(1e-4 * numel) distinct
  positions scaled x50 per tensor; stacked to [128*1536, 2048] and [128*2048, 768].
* ``config5``  seed 4: activations A[65536,2048] as config2's recipe; weights
  W[2048,6144] as config4's recipe; each token picks 8 distinct experts with probability
  proportional to Zipf(1.1) over expert id (Gumbel-top-8 of log p), routed rows gathered
  from A in (expert, token) order -> X[524288,2048] plus offsets int64[129].
"""
from __future__ import annotations

import numpy as np

HIDDEN = 2048
EXPERTS = 128
TOP_K = 8
FFN = 768


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (nearest, ties to even) and return the bit patterns.
    Inputs here are always finite."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float32 (for building test inputs)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _scale_positions(rng, x: np.ndarray, count: int, factor: float) -> None:
    flat = x.reshape(-1)
    pos = rng.choice(flat.size, size=count, replace=False)
    flat[pos] *= np.float32(factor)


# ---------------------------------------------------------------------------------------

def config1(seed: int = 0, rows: int = 256, cols: int = HIDDEN) -> dict:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    _scale_positions(rng, x, 8, 1000.0)
    r = int(rng.integers(rows))
    b = int(rng.integers(cols // 32))
    x[r, b * 32:(b + 1) * 32] = 0.0
    return {"x": bf16_bits_from_f32(x), "zero_block": (r, b)}


def activations(rng, rows: int, cols: int) -> np.ndarray:
    """config2's activation recipe: per-row std 10^U(-3,2), 0.1% outliers x100 (float32)."""
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    sigma = np.power(np.float32(10.0), rng.uniform(-3.0, 2.0, size=rows).astype(np.float32))
    x *= sigma[:, None]
    _scale_positions(rng, x, int(round(0.001 * x.size)), 100.0)
    return x


def config2(seed: int = 1, rows: int = 8192, cols: int = HIDDEN) -> dict:
    rng = np.random.default_rng(seed)
    return {"x": bf16_bits_from_f32(activations(rng, rows, cols))}


def _group_by_expert(token_of_choice: np.ndarray, expert_of_choice: np.ndarray, experts: int):
    order = np.lexsort((token_of_choice, expert_of_choice))
    token_idx = token_of_choice[order].astype(np.int64)
    counts = np.bincount(expert_of_choice, minlength=experts)
    offsets = np.zeros(experts + 1, np.int64)
    np.cumsum(counts, out=offsets[1:])
    return token_idx, offsets


def top_k_stable(keys: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest keys per row; ties go to the lower index."""
    return np.argsort(-keys, axis=1, kind="stable")[:, :k]


def config3(seed: int = 2, tokens: int = 16384, cols: int = HIDDEN,
            experts: int = EXPERTS, top_k: int = TOP_K, materialize: bool = True) -> dict:
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((tokens, cols), dtype=np.float32)
    m = rng.lognormal(0.0, 2.0, size=tokens).astype(np.float32)
    h *= m[:, None]
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    chosen = top_k_stable(logits, top_k)
    tok = np.repeat(np.arange(tokens), top_k)
    token_idx, offsets = _group_by_expert(tok, chosen.reshape(-1), experts)
    hb = bf16_bits_from_f32(h)
    out = {"h": hb, "token_idx": token_idx, "offsets": offsets}
    if materialize:
        out["x"] = hb[token_idx]
    return out


def weight(rng, rows: int, cols: int) -> np.ndarray:
    """config4's weight recipe: N(0, 0.02) with 0.01% entries x50 (float32)."""
    w = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(0.02)
    _scale_positions(rng, w, int(round(1e-4 * w.size)), 50.0)
    return w


def config4_expert(e: int, seed: int = 3, ffn: int = FFN, hidden: int = HIDDEN) -> dict:
    """One expert of config4: gate_up [2*ffn, hidden] and down [hidden, ffn] (BF16 bits)."""
    rng = np.random.default_rng([seed, e])
    gu = weight(rng, 2 * ffn, hidden)
    dn = weight(rng, hidden, ffn)
    return {"gate_up": bf16_bits_from_f32(gu), "down": bf16_bits_from_f32(dn)}


def config4(seed: int = 3, experts: int = EXPERTS, ffn: int = FFN, hidden: int = HIDDEN) -> dict:
    parts = [config4_expert(e, seed, ffn, hidden) for e in range(experts)]
    return {"gate_up": np.concatenate([p["gate_up"] for p in parts]),
            "down": np.concatenate([p["down"] for p in parts])}


def zipf_routing(rng, tokens: int, experts: int, top_k: int, a: float = 1.1):
    """Each token picks top_k distinct experts with probability proportional to
    (id+1)^-a, sampled without replacement as the Gumbel-top-k of log p."""
    logp = -a * np.log(np.arange(1, experts + 1, dtype=np.float64))
    u = rng.random((tokens, experts))
    g = -np.log(-np.log(u))
    chosen = top_k_stable(logp[None, :] + g, top_k)
    tok = np.repeat(np.arange(tokens), top_k)
    return _group_by_expert(tok, chosen.reshape(-1), experts)


def config5(seed: int = 4, tokens: int = 65536, hidden: int = HIDDEN, w_cols: int = 6144,
            experts: int = EXPERTS, top_k: int = TOP_K, materialize: bool = False) -> dict:
    """Layer-step stream.  Routed rows are returned as (token_idx, offsets) into ``a``;
    ``x = a[token_idx]`` is materialised only on request (it is 2 GiB at full size)."""
    rng = np.random.default_rng(seed)
    a = bf16_bits_from_f32(activations(rng, tokens, hidden))
    w = bf16_bits_from_f32(weight(rng, hidden, w_cols))
    token_idx, offsets = zipf_routing(rng, tokens, experts, top_k)
    out = {"a": a, "w": w, "token_idx": token_idx, "offsets": offsets}
    if materialize:
        out["x"] = a[token_idx]
    return out


def scatter_rows(token_idx: np.ndarray, tokens: int, top_k: int) -> np.ndarray:
    """Inverse of a routed-row gather: dst[t, j] = the routed row holding token t's j-th
    occurrence in token_idx (each token appears exactly top_k times)."""
    tok = np.asarray(token_idx, dtype=np.int64)
    assert tok.size == tokens * top_k
    order = np.argsort(tok, kind="stable")                   # routed rows grouped by token
    assert np.array_equal(tok[order], np.repeat(np.arange(tokens), top_k))
    return order.reshape(tokens, top_k).astype(np.int64)
