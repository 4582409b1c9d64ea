"""Pins of the oracle's routing layout (CPU only).

The layout's plain definition (DeepEP deep_ep.cpp, Buffer::get_dispatch_layout
counts; an expert-contiguous receive buffer as in Buffer::intranode_dispatch;
ascending (token, k) within an expert, a reading the pages leave open) is a stable
counting sort. The oracle is checked against numpy's bincount / cumsum /
stable argsort, a quadratic brute force, hand-worked fixtures and invariants.
"""
import numpy as np
import pytest

import moe_workloads as mw
from _util import brute_force_layout, ints, read_cases


def _library_layout(ids, E, align=1):
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    padded = -(-counts // align) * align
    offsets = np.concatenate([[0], np.cumsum(padded)])
    # Stable sort of pair indices by expert; masked pairs sort last.
    key = np.where(valid, flat, E)
    order = np.argsort(key, kind="stable")[: int(valid.sum())]
    return counts, offsets, order


def check_layout_invariants(ids, E, align, counts, offsets, pos, row_pair, status):
    N, K = ids.shape
    flat = ids.reshape(-1).astype(np.int64)
    valid = (flat >= 0) & (flat < E)
    p = pos.reshape(-1)
    assert counts.sum() == valid.sum()
    assert status == int((flat >= E).sum())
    assert (p[~valid] == -1).all()
    pv = p[valid]
    # pos is a bijection from valid pairs onto the used rows
    assert len(np.unique(pv)) == len(pv)
    assert offsets[0] == 0 and (np.diff(offsets) >= 0).all()
    assert (np.diff(offsets) % align == 0).all()
    # row_pair inverts pos
    idx = np.nonzero(valid)[0]
    assert (row_pair[pv] == idx).all()
    # every used row is in its expert's segment, and rows fill each segment
    # from its start without gaps
    seg_of_row = np.searchsorted(offsets, pv, side="right") - 1
    assert (seg_of_row == flat[valid]).all()
    for e in range(E):
        rows = row_pair[offsets[e]:offsets[e + 1]]
        used = rows[: counts[e]]
        assert (used >= 0).all() and (np.diff(used) > 0).all()   # ascending (t, k)
        assert (rows[counts[e]:] == -1).all()                    # padding rows
    assert (row_pair[offsets[E]:] == -1).all()
    assert (row_pair >= -1).all() and (row_pair < N * K).all()


@pytest.mark.parametrize("case", read_cases("layout_hand.txt"), ids=lambda c: c["name"][0])
def test_hand_worked_fixture(orc, case):
    N, K, E, align = (int(case[k][0]) for k in ("N", "K", "E", "align"))
    ids = ints(case["ids"]).astype(np.int32).reshape(N, K)
    counts, offsets, pos, row_pair, status = orc.layout(ids, E, align)
    assert counts.tolist() == ints(case["counts"]).tolist()
    assert offsets.tolist() == ints(case["offsets"]).tolist()
    assert pos.reshape(-1).tolist() == ints(case["pos"]).tolist()
    assert row_pair.tolist() == ints(case["row_pair"]).tolist()
    assert status == int(case["status"][0])


@pytest.mark.parametrize("seed", range(40))
def test_brute_force_tiny(orc, seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(0, 17))
    K = int(rng.integers(1, 9))
    E = int(rng.integers(1, 17))
    align = int(rng.choice([1, 1, 2, 3, 4]))
    ids = rng.integers(-2, E + 3, size=(N, K)).astype(np.int32)   # masks, bad ids, duplicates
    counts, offsets, pos, row_pair, status = orc.layout(ids, E, align)
    bc, bo, bp, bbad = brute_force_layout(ids, E, align)
    assert counts.tolist() == bc
    assert offsets.tolist() == bo
    assert (pos == bp).all()
    assert status == bbad
    check_layout_invariants(ids, E, align, counts, offsets, pos, row_pair, status)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed", "large"])
def test_library_equivalence_configs(orc, name):
    w = mw.make(name)
    ids = np.ascontiguousarray(w.ids)
    counts, offsets, pos, row_pair, status = orc.layout(w.ids, w.E)   # strided view for large
    lc, lo, order = _library_layout(ids, w.E)
    assert (counts == lc).all()
    assert (offsets == lo).all()
    assert (row_pair[: len(order)] == order).all()
    assert status == 0 and offsets[-1] == w.N * w.K
    check_layout_invariants(ids, w.E, 1, counts, offsets, pos, row_pair, status)
    if name == "skewed":
        assert (counts == 0).sum() >= 8        # the seeded empty experts


@pytest.mark.parametrize("seed", range(12))
def test_library_equivalence_random_masks(orc, seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.choice([1, 2, 7, 64, 256, 1024]))
    K = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    N = int(rng.integers(0, 3000))
    w = mw.make_random(seed, N, K, E, mask_frac=0.2, bad_frac=0.05, distinct=bool(seed % 2))
    align = int(rng.choice([1, 2, 8, 32]))
    counts, offsets, pos, row_pair, status = orc.layout(w.ids, E, align)
    lc, lo, order = _library_layout(w.ids, E, align)
    assert (counts == lc).all() and (offsets == lo).all()
    check_layout_invariants(w.ids, E, align, counts, offsets, pos, row_pair, status)
    if align == 1:
        assert (row_pair[: len(order)] == order).all()


def test_single_expert_is_identity(orc):
    rng = np.random.default_rng(5)
    ids = np.zeros((37, 5), np.int32)
    counts, offsets, pos, row_pair, _ = orc.layout(ids, 1)
    assert (pos.reshape(-1) == np.arange(37 * 5)).all()
    assert counts.tolist() == [185] and offsets.tolist() == [0, 185]
    del rng


def test_k1_is_stable_argsort(orc):
    rng = np.random.default_rng(6)
    ids = rng.integers(0, 9, size=(500, 1)).astype(np.int32)
    _, _, pos, row_pair, _ = orc.layout(ids, 9)
    order = np.argsort(ids[:, 0], kind="stable")
    assert (row_pair == order).all()
    assert (pos[order, 0] == np.arange(500)).all()


def test_empty_and_all_masked(orc):
    counts, offsets, pos, row_pair, status = orc.layout(np.zeros((0, 8), np.int32), 16)
    assert counts.sum() == 0 and (offsets == 0).all() and pos.shape == (0, 8) and status == 0
    counts, offsets, pos, row_pair, status = orc.layout(np.zeros((0, 8), np.int32), 16, cap=5)
    assert (row_pair == -1).all()
    ids = np.full((10, 4), -1, np.int32)
    counts, offsets, pos, row_pair, status = orc.layout(ids, 16)
    assert (pos == -1).all() and (row_pair == -1).all() and offsets[-1] == 0


def test_larger_capacity_rows_stay_unused(orc):
    ids = np.array([[1, 0], [0, 1]], np.int32)
    _, offsets, _, row_pair, _ = orc.layout(ids, 2, cap=9)
    assert offsets[-1] == 4 and (row_pair[4:] == -1).all() and len(row_pair) == 9


def test_errors(orc):
    ids = np.zeros((4, 2), np.int32)
    with pytest.raises(orc.OracleError) as e:
        orc.layout(ids, 2, cap=7)
    assert e.value.code == orc.ERR_CAPACITY
    with pytest.raises(orc.OracleError) as e:
        orc.layout(np.zeros((4, 33), np.int32), 2)
    assert e.value.code == orc.ERR_LIMIT
    with pytest.raises(orc.OracleError) as e:
        orc.layout(ids, 1025)
    assert e.value.code == orc.ERR_LIMIT
    with pytest.raises(orc.OracleError) as e:
        orc.layout(ids, 0)
    assert e.value.code == orc.ERR_ARG
    with pytest.raises(orc.OracleError) as e:
        orc.layout(ids, 2, align=0)
    assert e.value.code == orc.ERR_ARG
