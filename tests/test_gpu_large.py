"""GPU parity on a tensor past 2^31 elements: 1081349 x 2048 BF16 (4.4 GB), quantized to
per-token NVFP4, to rowwise and to both MXFP8 copies at full size on the GPU and dequantized
again, scattered as tokens to routed rows, and quantized with one scale per row group (1x16
and 16x16 blocks), then
compared with the oracle on sampled rows (and sampled 32-row blocks of the columnwise copy);
and the NVFP4 dequantizers on tensors large enough to be split into several launches.  Per-token NVFP4 and rowwise MXFP8 are
row-local (page "Towards Blackwell-native 8-bit and 4-bit RL", sections "Format background"
and "Per-token activation scaling": a row's codes and scales depend on that row only), so
the oracle's result on a subset of the rows is that subset of its result on the whole
tensor; a columnwise block depends on its 32 rows only.  The sampled rows lie at the start,
on both sides of element 2^31 (row 2^20), at seeded random places and in the last rows;
element and byte offsets there need more than 31 bits.  The per-token and rowwise outputs
carry guard bytes on both sides, checked on the device."""
import numpy as np
import pytest
import torch

import block_scaled_precision_mxfp8_amd as bsq
import oracle
from gpu_helpers import GUARD, SENTINEL, assert_same, bits, log

pytestmark = pytest.mark.gpu

R, K = (1 << 20) + (1 << 15) + 5, 2048
ROWS = np.unique(np.concatenate([np.arange(4), np.arange((1 << 20) - 3, (1 << 20) + 3),
                                 np.random.default_rng(31).integers(0, R, 24), np.arange(R - 5, R)]))


def _input():
    """Normal values times a per-row power of two in [2^-20, 2^19], drawn on the GPU in
    chunks (seeded), rounded to BF16: a wide spread of token scales and every element code."""
    g = torch.Generator(device="cuda").manual_seed(2 ** 31 + 1)
    x = torch.empty(R, K, dtype=torch.bfloat16, device="cuda")
    step = 1 << 17
    for a in range(0, R, step):
        b = min(a + step, R)
        e = torch.randint(-20, 20, (b - a, 1), generator=g, device="cuda").float()
        x[a:b] = (torch.randn(b - a, K, generator=g, device="cuda") * torch.exp2(e)).to(torch.bfloat16)
    return x


def _guarded(n):
    return torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device="cuda")


def _guards_intact(buf):
    return bool((buf[:GUARD] == SENTINEL).all()) and bool((buf[-GUARD:] == SENTINEL).all())


def _rows(t2d):
    return bits(t2d[torch.from_numpy(ROWS).cuda()])


@pytest.fixture(scope="module")
def big():
    x = _input()
    xs = _rows(x)
    yield x, xs
    del x
    torch.cuda.empty_cache()


def test_nv_per_token_past_2_pow_31_elements(big):
    x, xs = big
    log("nv per-token + dequant %dx%d (%d elements)" % (R, K, R * K))
    assert R * K > 2 ** 31
    qb, sbb, stb = _guarded(R * K // 2), _guarded(R * K // 16), _guarded(4 * R)
    q = qb[GUARD:GUARD + R * K // 2].view(R, K // 2)
    sb = sbb[GUARD:GUARD + R * K // 16].view(R, K // 16)
    st = stb[GUARD:GUARD + 4 * R].view(torch.float32)
    bsq.nv_quantize_nvfp4_per_token(x, q, sb, st)
    y = bsq.nv_dequantize(q, sb, st)
    torch.cuda.synchronize()
    assert all(_guards_intact(b) for b in (qb, sbb, stb))
    eq, esb, est = oracle.nv_quantize_per_token(xs)
    assert_same("st", _rows(st.view(R, 1)).reshape(-1), est.view(np.uint32))
    assert_same("sb", _rows(sb), esb)
    assert_same("q", _rows(q), eq)
    assert_same("dequant", _rows(y), oracle.nv_dequantize(eq, esb, est))
    del y
    # grouped by expert: the same bytes as the flat call (row-local), offsets checked on the device
    off = torch.tensor([0, 7, (1 << 20) + 1, (1 << 20) + 1, R], dtype=torch.int64, device="cuda")
    q2, sb2, st2 = torch.empty_like(q), torch.empty_like(sb), torch.empty_like(st)
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    bsq.nv_quantize_nvfp4_per_token_grouped(x, off, q2, sb2, st2, status)
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    assert torch.equal(q2, q) and torch.equal(sb2, sb) and torch.equal(st2.view(torch.int32), st.view(torch.int32))
    del q, sb, st, qb, sbb, stb, q2, sb2, st2
    torch.cuda.empty_cache()


def test_mx_rowwise_past_2_pow_31_elements(big):
    x, xs = big
    log("mx rowwise + dequant %dx%d (%d elements)" % (R, K, R * K))
    qb, sb_ = _guarded(R * K), _guarded(R * K // 32)
    q = qb[GUARD:GUARD + R * K].view(R, K)
    s = sb_[GUARD:GUARD + R * K // 32].view(R, K // 32)
    bsq.mx_quantize_mxfp8(x, "rowwise", q, s)
    y = bsq.mx_dequantize(q, s)
    torch.cuda.synchronize()
    assert _guards_intact(qb) and _guards_intact(sb_)
    eq, es = oracle.mx_quantize_rowwise(xs)
    assert_same("s_row", _rows(s), es)
    assert_same("q_row", _rows(q), eq)
    assert_same("dequant", _rows(y), oracle.mx_dequantize(eq, es))
    del q, s, qb, sb_, y
    torch.cuda.empty_cache()


def test_scatter_to_routed_rows_past_2_pow_31_elements(big):
    """Quantize-then-scatter (page "Towards Blackwell-native 8-bit and 4-bit RL", section
    "Per-token activation scaling": a token's bytes do not depend on the other rows) of the
    first T = 2^17 + 3 rows as tokens to 8 distinct routed rows each among all R rows, in a
    seeded random order; rows that no entry names keep their sentinel bytes."""
    x, _ = big
    T, k = (1 << 17) + 3, 8
    log("nv scatter %d tokens x %d -> %d routed rows" % (T, K, R))
    dst_np = np.random.default_rng(37).permutation(R)[:T * k].reshape(T, k).astype(np.int64)
    src = np.full(R, -1, np.int64)                   # routed row -> token
    src[dst_np.reshape(-1)] = np.repeat(np.arange(T), k)
    unnamed = np.flatnonzero(src < 0)
    q = torch.full((R, K // 2), SENTINEL, dtype=torch.uint8, device="cuda")
    sb = torch.full((R, K // 16), SENTINEL, dtype=torch.uint8, device="cuda")
    st = torch.full((R,), -7.0, dtype=torch.float32, device="cuda")
    q, sb, st, status = bsq.nv_quantize_nvfp4_per_token_scatter(x[:T], torch.from_numpy(dst_np).cuda(), R, q, sb, st)
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    named = ROWS[src[ROWS] >= 0]
    assert named.size > 20 and named.max() >= (1 << 20)
    eq, esb, est = oracle.nv_quantize_per_token(bits(x[torch.from_numpy(src[named]).cuda()]))
    idx = torch.from_numpy(named).cuda()
    assert_same("st", bits(st[idx]), est.view(np.uint32))
    assert_same("sb", bits(sb[idx]), esb)
    assert_same("q", bits(q[idx]), eq)
    u = torch.from_numpy(unnamed[np.random.default_rng(41).integers(0, unnamed.size, 64)]).cuda()
    assert bool((q[u] == SENTINEL).all()) and bool((sb[u] == SENTINEL).all()) and bool((st[u] == -7.0).all())
    del q, sb, st
    torch.cuda.empty_cache()


def test_mx_both_past_2_pow_31_elements(big):
    """Both MXFP8 copies of the first M = 2^20 + 96 rows (the tile grid ragged in rows): the
    rowwise copy on the sampled rows, the columnwise copy on sampled 32-row blocks (a 32x1
    block depends only on its own 32 rows of one column; page "Towards Blackwell-native 8-bit
    and 4-bit RL", section "Recipe 1: end-to-end MXFP8 RL"), each dequantized as well."""
    x, _ = big
    M = (1 << 20) + 96
    log("mx both + dequant %dx%d (%d elements)" % (M, K, M * K))
    xm = x[:M]
    q_row, s_row, q_col, s_col = bsq.mx_quantize_mxfp8(xm, "both")
    y_col = bsq.mx_dequantize(q_col, s_col)
    torch.cuda.synchronize()
    rows = ROWS[ROWS < M]
    eq, es = oracle.mx_quantize_rowwise(bits(xm[torch.from_numpy(rows).cuda()]))
    assert_same("q_row", bits(q_row[torch.from_numpy(rows).cuda()]), eq)
    assert_same("s_row", bits(s_row[torch.from_numpy(rows).cuda()]), es)
    nb = M // 32
    blocks = np.unique(np.concatenate([[0, 1, (1 << 15) - 1, 1 << 15, (1 << 15) + 1, nb - 2, nb - 1],
                                       np.random.default_rng(43).integers(0, nb, 8)]))
    brows = (32 * blocks[:, None] + np.arange(32)[None, :]).reshape(-1)
    ec, esc = oracle.mx_quantize_colwise(bits(xm[torch.from_numpy(brows).cuda()]))   # [K][32 nb'], [K][nb']
    bi, bb = torch.from_numpy(brows).cuda(), torch.from_numpy(blocks).cuda()
    assert_same("q_col", bits(q_col[:, bi]), ec)
    assert_same("s_col", bits(s_col[:, bb]), esc)
    assert_same("dequant col", bits(y_col[:, bi]), oracle.mx_dequantize(ec, esc))
    del q_row, s_row, q_col, s_col, y_col
    torch.cuda.empty_cache()


def test_nv_per_group_past_2_pow_31_elements(big):
    """Standard NVFP4 with one FP32 scale per row group (page "Towards Blackwell-native 8-bit
    and 4-bit RL", section "Format background": the coarse FP32 scale's scope is a recipe
    choice) on the whole tensor in three groups, the last one starting past element 2^31.
    A row's bytes depend on its own values and its group's maximum only, so for each group
    the oracle runs on that group's sampled rows plus one row that holds the group's largest
    magnitude (located with torch on the GPU), as a group of its own: its scale is the
    group's, and the sampled rows' bytes must equal the GPU's."""
    x, _ = big
    off = np.array([0, 500000, (1 << 20) + 7, R], np.int64)
    log("nv per-group %dx%d, %d groups" % (R, K, off.size - 1))
    q, sb, s_group, status = bsq.nv_quantize_nvfp4_per_group(x, torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    sg = bits(s_group)
    for g in range(off.size - 1):
        a, b = int(off[g]), int(off[g + 1])
        rows = ROWS[(ROWS >= a) & (ROWS < b)]
        assert rows.size > 0
        top = a + int(torch.argmax(x[a:b].abs().amax(dim=1).float()).item())   # row of the group maximum
        sub = np.concatenate([rows, [top]])
        eq, esb, es, ok = oracle.nv_quantize_per_group(bits(x[torch.from_numpy(sub).cuda()]), [0, sub.size])
        assert ok
        assert_same("s_group[%d]" % g, sg[g:g + 1], es.view(np.uint32))
        ri = torch.from_numpy(rows).cuda()
        assert_same("sb group %d" % g, bits(sb[ri]), esb[:-1])
        assert_same("q group %d" % g, bits(q[ri]), eq[:-1])
    del q, sb, s_group
    torch.cuda.empty_cache()

def test_nv_2d_past_2_pow_31_elements(big):
    """NVFP4 with 16x16 tiles under one scale per row group (page "NVIDIA verified the 4-bit
    NVFP4 format on a Mamba-Transformer (12B) at 10 trillion tokens": 2-D block scaling of the
    weights) on the first 2^20 + 2^15 rows in three groups of whole tiles, the last starting
    past element 2^31.  A tile's bytes depend on its own values and its group's maximum only,
    so for each group the oracle runs on that group's sampled tiles plus the tile that holds
    the group's largest magnitude, as a group of its own."""
    x, _ = big
    R16 = R - R % 16
    off = np.array([0, 499984, (1 << 20) + 16, R16], np.int64)
    log("nv 16x16 tiles %dx%d, %d groups" % (R16, K, off.size - 1))
    xm = x[:R16]
    q, sb, s_group, status = bsq.nv_quantize_nvfp4_2d(xm, torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    assert int(status.item()) == bsq.BSQ_OK
    sg = bits(s_group)
    for g in range(off.size - 1):
        a, b = int(off[g]), int(off[g + 1])
        tiles = np.unique(ROWS[(ROWS >= a) & (ROWS < b)] // 16)
        assert tiles.size > 0
        top = a + int(torch.argmax(xm[a:b].abs().amax(dim=1).float()).item())
        sub_tiles = np.concatenate([tiles, [top // 16]])
        rows = (16 * sub_tiles[:, None] + np.arange(16)[None, :]).reshape(-1)
        eq, esb, es, ok = oracle.nv_quantize_2d(bits(xm[torch.from_numpy(rows).cuda()]), [0, rows.size])
        assert ok
        assert_same("s_group[%d]" % g, sg[g:g + 1], es.view(np.uint32))
        n = 16 * tiles.size
        assert_same("sb group %d" % g, bits(sb[torch.from_numpy(tiles).cuda()]), esb[:-1])
        assert_same("q group %d" % g, bits(q[torch.from_numpy(rows[:n]).cuda()]), eq[:n])
    del q, sb, s_group
    torch.cuda.empty_cache()

def test_nv_dequant_split_into_several_launches():
    """The NVFP4 dequantizers index half blocks (8 elements) with 32 bits, so a tensor of 2^31
    half blocks or more is dequantized in row ranges, one launch each: at K = 2048 a launch
    takes 2^23 rows.  R = 2^23 + 1000 rows of random codes, block scales (NaN codes included)
    and token scales (34 GB of BF16 output) cross that boundary; the per-token dequant and the
    per-group one (three groups, the middle one spanning the boundary) are compared with the
    oracle's dequant on sampled rows (the per-group one is the per-token formula with each
    row's group scale)."""
    Rb = (1 << 23) + 1000
    log("nv dequant %dx%d in several launches" % (Rb, K))
    g = torch.Generator(device="cuda").manual_seed(47)
    q = torch.randint(0, 256, (Rb, K // 2), generator=g, dtype=torch.uint8, device="cuda")
    sb = torch.randint(0, 256, (Rb, K // 16), generator=g, dtype=torch.uint8, device="cuda")
    st = torch.exp2(torch.randint(-30, 30, (Rb,), generator=g, device="cuda").float()) * \
        torch.rand(Rb, generator=g, device="cuda")
    rows = np.unique(np.concatenate([np.arange(3), np.arange((1 << 23) - 3, (1 << 23) + 3),
                                     np.random.default_rng(53).integers(0, Rb, 16), np.arange(Rb - 3, Rb)]))
    ri = torch.from_numpy(rows).cuda()
    qh, sbh, sth = bits(q[ri]), bits(sb[ri]), bits(st[ri]).view(np.float32)
    y = bsq.nv_dequantize(q, sb, st)
    torch.cuda.synchronize()
    assert_same("per-token dequant", bits(y[ri]), oracle.nv_dequantize(qh, sbh, sth))
    off = np.array([0, 1000, (1 << 23) + 500, Rb], np.int64)
    s_group = torch.tensor([0.75, 3.0e-3, 1.5e4], dtype=torch.float32, device="cuda")
    bsq.nv_dequantize_per_group(q, sb, s_group, torch.from_numpy(off).cuda(), y=y)
    torch.cuda.synchronize()
    st_rows = s_group.cpu().numpy()[np.searchsorted(off, rows, side="right") - 1]
    assert_same("per-group dequant", bits(y[ri]), oracle.nv_dequantize(qh, sbh, st_rows))
    del q, sb, st, y
    torch.cuda.empty_cache()


def test_nv_dequant_2d_split_into_several_launches():
    """The same split for the 16x16-tile dequant, whose row ranges are whole tiles: R = 2^23 +
    1008 rows of random codes, random tile scales and three groups (offsets multiples of 16,
    the middle group spanning the boundary at row 2^23).  Sampled 16-row tiles are compared
    with the oracle's 2-D dequant of those tiles alone, each as a group of its own with its
    group's scale (an element depends only on its code, its tile's scale and its group's
    scale)."""
    Rb = (1 << 23) + 1008
    log("nv dequant 2d %dx%d in several launches" % (Rb, K))
    g = torch.Generator(device="cuda").manual_seed(59)
    q = torch.randint(0, 256, (Rb, K // 2), generator=g, dtype=torch.uint8, device="cuda")
    sb = torch.randint(0, 256, (Rb // 16, K // 16), generator=g, dtype=torch.uint8, device="cuda")
    off = np.array([0, 1008, (1 << 23) + 496, Rb], np.int64)
    s_group = torch.tensor([2.5, 6.0e-5, 7.0e3], dtype=torch.float32, device="cuda")
    y = bsq.nv_dequantize_2d(q, sb, s_group, torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    nt = Rb // 16
    tiles = np.unique(np.concatenate([[0, 1, (1 << 19) - 1, 1 << 19, (1 << 19) + 1, nt - 1],
                                      np.random.default_rng(61).integers(0, nt, 8)]))
    rows = (16 * tiles[:, None] + np.arange(16)[None, :]).reshape(-1)
    ri, ti = torch.from_numpy(rows).cuda(), torch.from_numpy(tiles).cuda()
    sg = s_group.cpu().numpy()[np.searchsorted(off, 16 * tiles, side="right") - 1]
    want = oracle.nv_dequantize_2d(bits(q[ri]), bits(sb[ti]), sg.astype(np.float32),
                                   np.arange(0, 16 * tiles.size + 1, 16, dtype=np.int64))
    assert_same("2-D dequant", bits(y[ri]), want)
    del q, sb, y
    torch.cuda.empty_cache()
