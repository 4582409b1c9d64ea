"""Pins of the oracle's dispatch (CPU only).

Dispatch is a byte scatter: every received row carries its token's whole
payload, as the recv_x / recv_x_scales / recv_topk_idx / recv_topk_weights
outputs of DeepEP's intranode dispatch (deep_ep.cpp) do. Checked against
numpy fancy indexing, pack/unpack round trips, record-vs-separate equality
and untouched canary rows.
"""
import numpy as np
import pytest

import moe_workloads as mw


def _expected(src, pos, rows, fill):
    out = np.full((rows, src.shape[1]), fill, np.uint8)
    N, K = pos.shape
    t = np.repeat(np.arange(N), K)
    p = pos.reshape(-1)
    ok = p >= 0
    out[p[ok]] = src[t[ok]]
    return out


# The first SAMPLE tokens of each workload (its routing and payload recipe,
# at a size whose receive buffers stay small): the full sizes run in the
# GPU parity tests, and the oracle's code path does not depend on N.
SAMPLE = 512


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed"])
def test_matches_fancy_indexing(orc, name):
    w = mw.make(name)
    n = min(w.N, SAMPLE)
    ids = w.ids[:n]
    _, _, pos, _, _ = orc.layout(ids, w.E)
    srcs = [a[:n] for _, a in w.fields]
    dsts = orc.dispatch(srcs, pos, w.K, fill=0xA5)
    for s, d in zip(srcs, dsts):
        assert np.array_equal(d, _expected(s, pos, n * w.K, 0xA5))


def test_large_records(orc):
    w = mw.make("large")
    n = SAMPLE
    _, _, pos, row_pair, _ = orc.layout(w.ids[:n], w.E)   # ids read in place from the records
    (d,) = orc.dispatch([w.records[:n]], pos, w.K)
    # row r holds the record of token row_pair[r] // K
    assert np.array_equal(d, w.records[:n][row_pair // w.K])


@pytest.mark.parametrize("seed", range(10))
def test_masked_rows_and_canaries(orc, seed):
    rng = np.random.default_rng(seed)
    N, K, E = int(rng.integers(1, 300)), int(rng.integers(1, 9)), int(rng.integers(1, 40))
    w = mw.make_random(seed, N, K, E, row_bytes=(48, 16, 4 * K), mask_frac=0.3, bad_frac=0.05)
    cap = N * K + 7
    _, offsets, pos, _, _ = orc.layout(w.ids, E, cap=cap)
    srcs = [a for _, a in w.fields]
    dsts = orc.dispatch(srcs, pos, K, rows=cap, fill=0xEE)
    for s, d in zip(srcs, dsts):
        assert np.array_equal(d, _expected(s, pos, cap, 0xEE))
        assert (d[offsets[-1]:] == 0xEE).all()          # rows past the used ones untouched


def test_multiset_of_rows(orc):
    w = mw.make("decode")
    _, _, pos, _, _ = orc.layout(w.ids, w.E)
    (d,) = orc.dispatch([w.fields[0][1]], pos, w.K)
    # Every token's hidden row appears exactly K times.
    got = {bytes(r): 0 for r in w.fields[0][1]}
    for r in d:
        got[bytes(r)] += 1
    assert set(got.values()) == {w.K}


def _record_offsets(sizes):
    offs, cur = [], 0
    for s in sizes:
        cur = (cur + 15) & ~15
        offs.append(cur)
        cur += s
    return offs, (cur + 15) & ~15


def test_pack_unpack_roundtrip_and_record_mode(orc):
    w = mw.make("tiny")
    srcs = [a for _, a in w.fields]
    offs, rec_bytes = _record_offsets([a.shape[1] for a in srcs])
    assert offs == [0, 3584, 4032, 4064] and rec_bytes == 4096
    rec = np.zeros((w.N, rec_bytes), np.uint8)
    views = [rec[:, o:o + a.shape[1]] for o, a in zip(offs, srcs)]
    orc.dispatch(srcs, None, 1, dsts=views)                       # pack
    outs = orc.dispatch(views, None, 1)                           # unpack
    for s, o in zip(srcs, outs):
        assert np.array_equal(s, o)
    # record-mode dispatch equals the separate-field dispatch re-packed
    _, _, pos, _, _ = orc.layout(w.ids, w.E)
    (drec,) = orc.dispatch([rec], pos, w.K)
    dsep = orc.dispatch(srcs, pos, w.K)
    for o, d in zip(offs, dsep):
        assert np.array_equal(drec[:, o:o + d.shape[1]], d)


def test_strided_source_rows(orc):
    rng = np.random.default_rng(3)
    base = rng.integers(0, 256, size=(50, 96), dtype=np.uint8)
    src = base[:, 16:64]                                          # row stride 96, row bytes 48
    ids = rng.integers(0, 5, size=(50, 2)).astype(np.int32)
    _, _, pos, _, _ = orc.layout(ids, 5)
    (d,) = orc.dispatch([src], pos, 2)
    assert np.array_equal(d, _expected(np.ascontiguousarray(src), pos, 100, 0))


def test_errors(orc):
    a = np.zeros((3, 16), np.uint8)
    with pytest.raises(orc.OracleError):
        orc.dispatch([a] * 5, np.zeros((3, 1), np.int32), 1)
    with pytest.raises(orc.OracleError):
        orc.dispatch([a], None, 2, rows=6)
