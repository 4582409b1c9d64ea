"""Pins of the oracle's low-latency dispatch forms (CPU only): the padded
per-expert layout and the FP8 (e4m3) cast on dispatch with per-128-channel
scales (DeepEP repository dump, deep_ep.cpp, Buffer::low_latency_dispatch;
config.hpp, LowLatencyLayout). The cast's arithmetic is a reading of ours
(the kernel is not on the pages): amax/448 per block, at least 2^-126,
optionally rounded up to a power of two; e4m3 round-to-nearest-even,
saturating.
"""
import math

import numpy as np
import pytest
import torch

import moe_workloads as mw
from _util import bf16_bits_to_float


def _bits(a):
    return mw.bf16_bits_from_f32(np.asarray(a, np.float32))


# ---------------------------------------------------------------- layout ---

@pytest.mark.parametrize("seed", range(12))
def test_padded_layout_is_the_stable_layout_shifted(orc, seed):
    rng = np.random.default_rng(seed)
    N, K, E = int(rng.integers(0, 300)), int(rng.integers(1, 9)), int(rng.integers(1, 40))
    ids = rng.integers(-1, E + 2, size=(N, K)).astype(np.int32)
    M = int(rng.choice([N, max(1, N // 4), 3, 0])) if N else 2
    counts, pos, row_pair, (bad, dropped) = orc.layout_padded(ids, E, M)
    full_counts, offsets, full_pos, _, full_bad = orc.layout(ids, E)
    assert bad == full_bad
    assert (counts == np.minimum(full_counts, M)).all()
    assert dropped == int(np.maximum(full_counts - M, 0).sum())
    flat, fpos = ids.reshape(-1), full_pos.reshape(-1)
    for i, e in enumerate(flat):
        if fpos[i] < 0:
            assert pos.reshape(-1)[i] == -1
            continue
        rank = fpos[i] - offsets[e]                   # rank within the expert, (t, k) order
        expect = e * M + rank if rank < M else -1
        assert pos.reshape(-1)[i] == expect
    for e in range(E):
        seg = row_pair[e * M:(e + 1) * M]
        assert (seg[counts[e]:] == -1).all() and (np.diff(seg[:counts[e]]) > 0).all()


def test_padded_layout_hand_worked(orc):
    # N=4 K=2 E=3 (ids as in tests/golden/layout_hand.txt, case plain), M=2:
    # e0 pairs (0,1),(1,0),(3,1) -> rows 0,1 then dropped; e1 (2,0) -> row 2;
    # e2 (0,0),(1,1),(3,0) -> rows 4,5 then dropped.
    ids = np.array([[2, 0], [0, 2], [1, -1], [2, 0]], np.int32)
    counts, pos, row_pair, (bad, dropped) = orc.layout_padded(ids, 3, 2)
    assert counts.tolist() == [2, 1, 2]
    assert pos.reshape(-1).tolist() == [4, 0, 1, 5, 2, -1, -1, -1]
    assert row_pair.tolist() == [1, 2, 4, -1, 0, 3]
    assert (bad, dropped) == (0, 2)


# ------------------------------------------------------------------ e4m3 ---

def _torch_e4m3(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_padded_receive_metadata(orc, seed):
    """What the receive metadata must say, checked against the layout itself
    rather than against its formula: for each expert, the range's begin and
    count (in the packing this library reads into the int64, begin in the
    high half) cover exactly the rows of the expert's segment that hold a
    pair; the stats gain, over two calls, the rows each expert received, and
    one call's gains add up to the pairs that were neither masked, out of
    range nor dropped."""
    rng = np.random.default_rng(seed)
    N, K, E, M = 300, 8, 40, 50
    ids = rng.integers(-1, E + 1, size=(N, K)).astype(np.int32)
    counts, pos, row_pair, (nbad, ndrop) = orc.layout_padded(ids, E, M)
    start = rng.integers(0, 1000, size=E).astype(np.int32)
    rngs, stats = orc.padded_recv_meta(counts, start)
    begin, count = rngs >> 32, rngs & 0xFFFFFFFF
    filled = (row_pair.reshape(E, M) >= 0)
    for e in range(E):
        rows = np.flatnonzero(filled[e])
        assert np.array_equal(rows, np.arange(begin[e], begin[e] + count[e]))
    valid = int(((ids >= 0) & (ids < E)).sum())
    assert int((stats - start).sum()) == valid - ndrop
    ids2 = rng.integers(0, E, size=(17, K)).astype(np.int32)
    counts2 = orc.layout_padded(ids2, E, M)[0]
    _, stats2 = orc.padded_recv_meta(counts2, stats)
    assert np.array_equal(stats2 - start, counts.astype(np.int64) + counts2)
    empty = orc.layout_padded(np.zeros((0, K), np.int32), E, M)[0]
    r0, s0 = orc.padded_recv_meta(empty, stats2)
    assert (r0 == 0).all() and np.array_equal(s0, stats2)


def test_e4m3_matches_torch_in_range(orc):
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-4, 3, 20000),
                        rng.uniform(-463.9, 463.9, 5000)]).astype(np.float32)
    # exact ties between neighbouring e4m3 values
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    vals = np.array([orc.e4m3_to_f32(int(c)) for c in codes], np.float64)
    ties = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, ties, -ties, [0.0, -0.0, 2 ** -9, 2 ** -10, 448.0, -448.0]]).astype(np.float32)
    ours = np.array([orc.f32_to_e4m3(float(x)) for x in v], np.uint8)
    ref = _torch_e4m3(v)
    same = (ours == ref) | ((ours & 0x7F) == 0) & ((ref & 0x7F) == 0)   # +-0
    assert same.all(), v[~same][:10]


def test_e4m3_saturates_and_decodes(orc):
    for x, c in [(448.0, 0x7E), (449.0, 0x7E), (1e9, 0x7E), (-1e9, 0xFE), (float("inf"), 0x7E),
                 (float("nan"), 0x7F), (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (1.0, 0x38)]:
        assert orc.f32_to_e4m3(x) == c, x
    for c in range(256):
        v = orc.e4m3_to_f32(c)
        if (c & 0x7F) == 0x7F:
            assert math.isnan(v)
        else:
            assert orc.f32_to_e4m3(v) == c or (c & 0x7F) == 0


# ----------------------------------------------------------------- scale ---

def test_block_scale_rules(orc):
    """The scale rule of the reading the oracle takes, written out: amax/448
    as one fp32 division, raised to 2^-126 when smaller, and with round_scale
    the smallest power of two at or above it. The pages give the cast's
    inputs and outputs only, so the floor and the division form are parity
    unpinned; the property tests below pin what the scale must achieve."""
    rng = np.random.default_rng(1)
    for _ in range(200):
        blk = _bits(rng.standard_normal(128) * 10.0 ** rng.integers(-8, 4))
        amax = float(np.abs(bf16_bits_to_float(blk)).max())
        s = orc.fp8_block_scale(blk, False)
        assert s == max(float(np.float32(np.float32(amax) / np.float32(448.0))), 2.0 ** -126)
        r = orc.fp8_block_scale(blk, True)
        m, e = math.frexp(r)
        assert m == 0.5 and r >= s and r < 2 * s            # smallest power of two >= s
    assert orc.fp8_block_scale(np.zeros(128, np.uint16), False) == 2.0 ** -126


@pytest.mark.parametrize("round_scale", [False, True])
def test_block_scale_puts_amax_at_the_top_of_e4m3(orc, round_scale):
    """What a per-block scale is for, checked without its formula: the
    block's largest magnitude lands at the top of the e4m3 range, so no code
    saturates and none of the range is wasted. Without round_scale it encodes
    to 448 itself; with a power-of-two scale (the next power of two at or
    above the exact one) it lands in [224, 448]. Every other element stays
    within +-448, and no code is NaN."""
    rng = np.random.default_rng(11)
    for _ in range(300):
        f = rng.standard_normal(128) * 10.0 ** rng.integers(-30, 30)
        blk = _bits(f)
        codes, scales = orc.dispatch_fp8(blk.reshape(1, 128), np.zeros((1, 1), np.int32), 1,
                                         orc.SCALE_ROWS, 0, round_scale)
        dec = np.array([orc.e4m3_to_f32(int(c)) for c in codes[0]])
        assert not np.isnan(dec).any()
        assert (np.abs(dec) <= 448.0).all()
        top = abs(dec[int(np.argmax(np.abs(bf16_bits_to_float(blk))))])
        if round_scale:
            assert 224.0 <= top <= 448.0
            assert math.frexp(float(scales[0, 0]))[0] == 0.5
        else:
            assert top == 448.0


def test_all_zero_block_encodes_to_zero(orc):
    """An all-zero block has no magnitude to scale, so any positive finite
    scale (whatever floor keeps it off zero) gives codes that are all +0 and
    a dequantised block that is exactly zero. The value the oracle stores
    for that scale (2^-126) is its own reading: parity unpinned."""
    for round_scale in (False, True):
        codes, scales = orc.dispatch_fp8(np.zeros((1, 512), np.uint16), np.zeros((1, 1), np.int32),
                                         1, orc.SCALE_ROWS, 0, round_scale)
        assert (codes == 0).all()
        s = scales[0, :4]
        assert np.isfinite(s).all() and (s > 0).all()
    assert orc.e4m3_to_f32(0) == 0.0


@pytest.mark.parametrize("round_scale", [False, True])
def test_block_with_an_infinity(orc, round_scale):
    """amax = inf makes s = inf, and with round_scale it stays inf: there is
    no power of two above it. x / inf is then +-0 for finite x and NaN for
    +-inf, so the codes are 0x00 / 0x80 and 0x7F (NaN), and the UE8M0 byte is
    inf's exponent field, 0xFF."""
    blk = _bits(np.linspace(-3.0, 3.0, 128))
    blk[5], blk[9], blk[17] = 0x7F80, 0xFF80, 0x7FC0        # +inf, -inf, NaN
    s = orc.fp8_block_scale(blk, round_scale)
    assert math.isinf(s) and s > 0
    x = blk.reshape(1, 128)
    codes, scales = orc.dispatch_fp8(x, np.zeros((1, 1), np.int32), 1, orc.SCALE_ROWS, 0, round_scale)
    f = bf16_bits_to_float(blk)
    want = np.where(np.isfinite(f), np.where(np.signbit(f), 0x80, 0x00), 0x7F).astype(np.uint8)
    assert np.array_equal(codes[0], want)
    assert math.isinf(scales[0, 0])
    if round_scale:
        x4 = np.tile(blk, 4).reshape(1, 512)
        _, ue = orc.dispatch_fp8(x4, np.zeros((1, 1), np.int32), 1, orc.SCALE_UE8M0, 1, True)
        assert ue.view(np.uint8).reshape(-1).tolist() == [0xFF] * 4


def test_constant_block_maps_to_max_code(orc):
    for c in (1.0, -3.5, 1e-3, 7.0e4):
        x = np.tile(_bits([c] * 128), (1, 1))
        pos = np.zeros((1, 1), np.int32)
        codes, scales = orc.dispatch_fp8(x, pos, 1)
        assert (codes == (0xFE if c < 0 else 0x7E)).all()


@pytest.mark.parametrize("round_scale", [False, True])
def test_dequantisation_error_bound(orc, round_scale):
    rng = np.random.default_rng(2)
    N, H = 16, 512
    x = _bits(rng.standard_normal((N, H)) * np.exp(rng.standard_normal((N, 1)) * 3))
    pos = np.arange(N, dtype=np.int32).reshape(N, 1)
    codes, scales = orc.dispatch_fp8(x, pos, N, round_scale=round_scale)
    xf = bf16_bits_to_float(x).astype(np.float64)
    deq = np.vectorize(orc.e4m3_to_f32)(codes).astype(np.float64) * np.repeat(scales, 128, axis=1)
    blk_max = np.repeat(np.abs(xf).reshape(N, -1, 128).max(axis=2), 128, axis=1)
    # e4m3 keeps 3 mantissa bits: relative error <= 2^-4 in the normal range,
    # absolute error <= half the subnormal spacing (2^-10 times the scale) below it
    err = np.abs(deq - xf)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, np.repeat(scales, 128, axis=1) * 2.0 ** -10) * 1.0001
    assert (err <= bound).all()
    # the largest element of each block lands near the top of the e4m3 range
    top = np.abs(deq) >= blk_max * (1 - 2.0 ** -3)
    assert top.reshape(N, -1, 128).any(axis=2).all()


def test_scale_layouts_agree(orc):
    rng = np.random.default_rng(3)
    N, K, E, H, M = 40, 4, 8, 1024, 40
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    x = _bits(rng.standard_normal((N, H)))
    counts, pos, row_pair, _ = orc.layout_padded(ids, E, M)
    rows = E * M
    c_rows, s_rows = orc.dispatch_fp8(x, pos, rows, orc.SCALE_ROWS, M, True)
    c_cols, s_cols = orc.dispatch_fp8(x, pos, rows, orc.SCALE_COLS, M, True)
    c_ue, s_ue = orc.dispatch_fp8(x, pos, rows, orc.SCALE_UE8M0, M, True)
    assert np.array_equal(c_rows, c_cols) and np.array_equal(c_rows, c_ue)
    # column-major per expert is a transpose of the row-major scales
    assert np.array_equal(s_cols, s_rows.reshape(E, M, H // 128).transpose(0, 2, 1))
    # ue8m0 bytes are the biased exponents of the power-of-two scales
    exps = (s_rows.view(np.uint32) >> 23).astype(np.uint8).reshape(E, M, H // 512, 4)
    assert np.array_equal(s_ue.view(np.uint8).reshape(E, H // 512, M, 4), exps.transpose(0, 2, 1, 3))
    # every used row holds the codes of its source token
    used = row_pair >= 0
    t = row_pair[used] // K
    solo, solo_s = orc.dispatch_fp8(x, np.arange(N, dtype=np.int32).reshape(N, 1), N, round_scale=True)
    assert np.array_equal(c_rows[used], solo[t]) and np.array_equal(s_rows[used], solo_s[t])


@pytest.mark.parametrize("fmt", ["cols", "ue8m0"])
def test_token_scales_then_scatter_is_the_one_call_form(orc, fmt):
    """Per-token scales (SCALE_TOKENS) are the K = 1 row scales of every
    token, dropped or not, with the same codes; placing them by row_pair
    gives the column-major / UE8M0 arrays of the one-call form, leaving
    unused rows as they were."""
    rng = np.random.default_rng(11)
    N, K, E, H, M = 96, 4, 8, 1024, 20            # M < N*K/E: some pairs dropped
    ids = rng.integers(-1, E, size=(N, K)).astype(np.int32)
    ids[5] = -1                                     # a token with no pair at all
    ids[ids == E - 1] = -1
    ids[0, 0] = E - 1                               # expert E-1: one row, M-1 unused
    x = _bits(rng.standard_normal((N, H)) * np.exp(rng.standard_normal((N, 1))))
    counts, pos, row_pair, (_, dropped) = orc.layout_padded(ids, E, M)
    assert dropped > 0
    mode = orc.SCALE_COLS if fmt == "cols" else orc.SCALE_UE8M0
    rows = E * M
    c_tok, s_tok = orc.dispatch_fp8(x, pos, rows, orc.SCALE_TOKENS, M, True, fill=0x5A)
    solo_c, solo_s = orc.dispatch_fp8(x, np.arange(N, dtype=np.int32).reshape(N, 1), N,
                                      round_scale=True)
    assert s_tok.shape == (N, H // 128) and np.array_equal(s_tok, solo_s)
    c_one, s_one = orc.dispatch_fp8(x, pos, rows, mode, M, True, fill=0x5A)
    assert np.array_equal(c_tok, c_one)
    sentinel = np.full_like(s_one, 7)
    s_one2 = orc.dispatch_fp8(x, pos, rows, mode, M, True, codes=np.zeros_like(c_one),
                              scales=sentinel.copy())[1]
    s_sc = orc.scatter_scales(s_tok, K, row_pair, E, M, mode, scales=sentinel.copy())
    assert np.array_equal(s_sc, s_one2)
    unused = (row_pair.reshape(E, M) < 0)
    assert unused.any() and (s_sc.transpose(0, 2, 1)[unused] == 7).all()


def test_scatter_scales_hand_worked(orc):
    # N=2 tokens, K=2, E=2 experts, M=3 rows each, H=512 (4 blocks, one ue8m0 word).
    # row_pair: e0 rows <- pairs 1 (token 0), 2 (token 1), 4 (>= N*K: untouched);
    #           e1 rows <- pairs 3 (token 1), 0 (token 0), -1 (untouched).
    ts = np.array([[1.0, 2.0, 0.5, 0.25], [4.0, 8.0, 0.125, 2.0 ** -126]], np.float32)
    row_pair = np.array([1, 2, 4, 3, 0, -1], np.int32)
    S = -3.0
    cols = orc.scatter_scales(ts, 2, row_pair, 2, 3, orc.SCALE_COLS,
                              scales=np.full((2, 4, 3), S, np.float32))
    assert cols.tolist() == [
        [[1.0, 4.0, S], [2.0, 8.0, S], [0.5, 0.125, S], [0.25, 2.0 ** -126, S]],
        [[4.0, 1.0, S], [8.0, 2.0, S], [0.125, 0.5, S], [2.0 ** -126, 0.25, S]]]
    # ue8m0: byte j of a row's word = biased exponent of its token's block j
    # (1 -> 127, 2 -> 128, 0.5 -> 126, 0.25 -> 125, 4 -> 129, 8 -> 130,
    #  0.125 -> 124, 2^-126 -> 1)
    ue = orc.scatter_scales(ts, 2, row_pair, 2, 3, orc.SCALE_UE8M0,
                            scales=np.full((2, 1, 3), -1, np.int32))
    b = ue.view(np.uint8).reshape(2, 3, 4)
    assert b[0].tolist() == [[127, 128, 126, 125], [129, 130, 124, 1], [255, 255, 255, 255]]
    assert b[1].tolist() == [[129, 130, 124, 1], [127, 128, 126, 125], [255, 255, 255, 255]]


def test_errors(orc):
    x = np.zeros((2, 100), np.uint16)
    with pytest.raises(orc.OracleError):
        orc.dispatch_fp8(x, np.zeros((2, 1), np.int32), 2)              # H % 128
    x = np.zeros((2, 128), np.uint16)
    with pytest.raises(orc.OracleError):
        orc.dispatch_fp8(x, np.zeros((2, 1), np.int32), 2, orc.SCALE_UE8M0, 2, True)   # H % 512
    with pytest.raises(orc.OracleError):
        orc.dispatch_fp8(np.zeros((2, 512), np.uint16), np.zeros((2, 1), np.int32), 2,
                         orc.SCALE_UE8M0, 2, False)                      # ue8m0 needs round_scale
