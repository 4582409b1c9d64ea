"""GPU: the device check of a layout's index arrays (moe_check_layout) and the
debug build (libmoe_get_debug.so, MOE_DEBUG).

- Layouts of every form (one launch for small batches, one pass, two kernels,
  strided ids, the allocation-free call, the padded forms, the fused
  layout + dispatch calls, an empty batch) pass with all four counts zero.
- Corrupted copies of a layout: the four counts equal those of the header's
  definitions evaluated on the host (numpy), for out-of-range rows, rows
  shared by two pairs, row_pair entries that disagree or point outside the
  pairs, and plan entries outside the pairs or naming masked pairs. Every
  read the check makes is guarded by the ranges it checks, so these inputs
  are safe to run.
- The debug build: the same layout calls give bit-identical outputs, every
  call is checked once (the status's fifth word), and no inconsistency is
  found.
"""
import os
import sys

import numpy as np
import pytest
import torch

import moe_workloads as mw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_get_amd as m

    return m


def say(msg):
    print(f"[gpu-check] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_counts(pos, row_pair, cap, order):
    """The four counts as include/moe_get.h defines them, on the host."""
    p = pos.reshape(-1).astype(np.int64)
    nk = p.size
    c0 = int(np.sum((p != -1) & ((p < 0) | (p >= cap))))
    has_row = (p >= 0) & (p < cap)
    c1 = c2 = c3 = 0
    if row_pair is not None:
        rp = row_pair.astype(np.int64)
        named = rp[np.where(has_row, p, 0)]
        c1 = int(np.sum(has_row & (named != np.arange(nk))))
        in_pairs = (rp >= 0) & (rp < nk)
        back = p[np.where(in_pairs, rp, 0)] if nk else np.zeros_like(rp)
        ok = (rp == -1) | (in_pairs & (back == np.arange(cap)))
        c2 = int(np.sum(~ok))
    if order is not None:
        o = order.reshape(-1).astype(np.int64)
        in_pairs = (o >= 0) & (o < nk)
        q = np.where(in_pairs, p[np.where(in_pairs, o, 0)] if nk else -1, -1)
        c3 = int(np.sum((o != -1) & ((q < 0) | (q >= cap))))
    return (c0, c1, c2, c3)


def check(mg, pos, row_pair, order):
    st = torch.zeros(4, dtype=torch.int32, device="cuda")
    mg.moe_check_layout(pos, row_pair, order, st)
    torch.cuda.synchronize()
    return tuple(int(v) for v in st.cpu())


def routed_ids(N, K, E, seed, mask=0.05, bad=0.01):
    rng = np.random.default_rng(seed)
    ids = (mw.uniform_distinct_ids(rng, N, K, E) if K <= E
           else rng.integers(0, E, (N, K))).astype(np.int32)
    ids[rng.random((N, K)) < mask] = -1
    ids[rng.random((N, K)) < bad] = E + 1
    return ids


def make_forms(mg):
    """Every form of layout call, each made once: (name, pos, row_pair, plan)."""
    i32 = lambda *s: torch.full(s, -7, dtype=torch.int32, device="cuda")
    forms = []

    def plain(name, ids_d, E, align):
        lay = mg.layout(ids_d, E, align=align)
        forms.append((name, lay.pos, lay.row_pair, lay.order))

    plain("one launch (1600 pairs)", dev(routed_ids(200, 8, 64, 1)), 64, 4)
    plain("one pass (32768 pairs)", dev(mw.make("prefill").ids), 256, 1)
    plain("two kernels (32776 pairs, align 8)", dev(routed_ids(4097, 8, 256, 2)), 256, 8)
    rec = torch.full((3000, 16), -1, dtype=torch.int32, device="cuda")
    rec[:, :8] = dev(routed_ids(3000, 8, 128, 3))
    plain("strided ids (two kernels)", rec[:, :8], 128, 1)
    plain("empty batch", dev(np.zeros((0, 8), np.int32)), 16, 4)

    # the allocation-free layout
    N, K, E = 1000, 4, 32
    ids = dev(routed_ids(N, K, E, 4))
    cap = mg.moe_required_capacity(N, K, E, 2)
    o = dict(counts=i32(E), offsets=i32(E + 1), pos=i32(N, K), row_pair=i32(cap),
             status=i32(1), order=i32(N * K))
    mg.moe_get_layout_noalloc(ids, E, 2, o["counts"], o["offsets"], o["pos"], o["row_pair"],
                              o["status"], order=o["order"])
    forms.append(("allocation-free", o["pos"], o["row_pair"], o["order"]))

    # padded layouts: one launch, one pass, two kernels (ids 4 bytes off)
    for name, (N, E, M, misalign) in (("padded, one launch", (200, 64, 32, False)),
                                      ("padded, one pass", (4096, 256, 200, False)),
                                      ("padded, two kernels", (3000, 64, 300, True))):
        K = 8
        ids_np = routed_ids(N, K, E, N + E)
        if misalign:
            flat = torch.empty(ids_np.size + 1, dtype=torch.int32, device="cuda")
            ids_d = flat[1:].view(N, K)
            ids_d.copy_(torch.from_numpy(ids_np))
        else:
            ids_d = dev(ids_np)
        pos, rp = i32(N, K), i32(E * M)
        ws = torch.empty(mg.moe_layout_workspace_bytes(N, K, E), dtype=torch.uint8, device="cuda")
        mg.moe_get_layout_padded(ids_d, E, M, i32(E), pos, rp, ws, i32(2))
        forms.append((name, pos, rp, None))

    # layout + dispatch in one launch
    N, K, E = 100, 8, 32
    ids = dev(routed_ids(N, K, E, 5))
    cap = mg.moe_required_capacity(N, K, E, 2)
    pos, rp = i32(N, K), i32(cap)
    src = dev(np.random.default_rng(6).integers(0, 256, (N, 48), dtype=np.uint8))
    dst = torch.zeros((cap, 48), dtype=torch.uint8, device="cuda")
    mg.moe_layout_dispatch(ids, E, 2, i32(E), i32(E + 1), pos, rp, i32(1), [src], [dst])
    forms.append(("layout + dispatch, one launch", pos, rp, None))

    # padded layout + FP8 dispatch in one launch
    N, K, E, M, H = 64, 8, 32, 24, 256
    ids = dev(routed_ids(N, K, E, 7))
    x = mw.bf16_bits_from_f32(np.random.default_rng(8).standard_normal((N, H)).astype(np.float32))
    pos, rp = i32(N, K), i32(E * M)
    mg.moe_dispatch_fp8_padded(ids, E, M, dev(x.view(np.int16)).view(torch.bfloat16), i32(E),
                               pos, rp, i32(2), torch.zeros((E * M, H), dtype=torch.uint8,
                                                            device="cuda"),
                               torch.zeros((E, H // 128, M), dtype=torch.float32, device="cuda"),
                               mg.MOE_SCALE_COLS, False)
    forms.append(("padded layout + FP8 dispatch, one launch", pos, rp, None))
    torch.cuda.synchronize()
    return forms


def test_every_layout_form_passes_the_check(mg):
    for name, pos, rp, order in make_forms(mg):
        say(f"check {name}: N*K={pos.numel()} rows={rp.numel()} plan={order is not None}")
        assert check(mg, pos, rp, order) == (0, 0, 0, 0), name


@pytest.mark.parametrize("seed", range(6))
def test_counts_of_corrupted_layouts(mg, seed):
    """Corrupted copies of a valid layout: each count equals the host's."""
    rng = np.random.default_rng(100 + seed)
    N, K, E, align = [(300, 4, 16, 4), (4096, 8, 256, 1), (257, 8, 64, 1), (1, 1, 1, 1),
                      (3000, 3, 100, 8), (64, 32, 1024, 1)][seed]
    ids = routed_ids(N, K, E, 200 + seed, mask=0.1)
    cap = mg.moe_required_capacity(N, K, E, align) + int(rng.integers(0, 9))
    lay = mg.layout(dev(ids), E, align=align, cap=cap)
    torch.cuda.synchronize()
    pos = lay.pos.cpu().numpy().reshape(-1).copy()
    rp = lay.row_pair.cpu().numpy().copy()
    order = lay.order.cpu().numpy().copy()
    nk = pos.size
    assert check(mg, lay.pos, lay.row_pair, lay.order) == (0, 0, 0, 0)

    def pick(n, k):
        return rng.choice(n, size=min(k, n), replace=False) if n else np.zeros(0, np.int64)

    # rows outside [-1, cap): below -1, at cap, far past it
    for i, v in zip(pick(nk, 5), (-2, -1000, cap, cap + 17, 1 << 30)):
        pos[i] = v
    # two pairs in one row (a copy of another valid pair's row)
    valid = np.flatnonzero((pos >= 0) & (pos < cap))
    if valid.size >= 4:
        a, b = rng.choice(valid, size=2, replace=False)
        pos[a] = pos[b]
    # row_pair entries naming a wrong pair, a pair past N*K, a negative one
    for r, v in zip(pick(cap, 3), (int(rng.integers(0, nk)), nk + 5, -3)):
        rp[r] = v
    # plan entries outside the pairs, or naming masked pairs
    masked = np.flatnonzero(pos == -1)
    bad_plan = [nk, nk + 100, -5] + ([int(masked[0])] if masked.size else [])
    for i, v in zip(pick(nk, len(bad_plan)), bad_plan):
        order[i] = v
    expect = host_counts(pos, rp, cap, order)
    say(f"corrupted N={N} K={K} E={E} cap={cap}: expect {expect}")
    got = check(mg, dev(pos.reshape(N, K)), dev(rp), dev(order))
    assert got == expect
    # without row_pair and plan only the range count remains
    assert check(mg, dev(pos.reshape(N, K)), torch.empty(0, dtype=torch.int32, device="cuda"),
                 None)[1:] == (0, 0, 0)


def test_check_without_rows(mg):
    """cap 0 (no row_pair): every valid row is out of range; -1 is not."""
    pos = dev(np.array([[0, -1, 3], [-1, -1, 7]], np.int32))
    none = torch.empty(0, dtype=torch.int32, device="cuda")
    assert check(mg, pos, none, None) == (3, 0, 0, 0)


def test_debug_build(mg, monkeypatch):
    """libmoe_get_debug.so: every layout call of make_forms checked once, no
    inconsistency found, outputs bit-identical to the release library's."""
    release = make_forms(mg)
    with pytest.raises(mg.MoeError):
        mg.debug_status()          # the release build has no debug status
    path = os.path.join(os.path.dirname(mg.__file__), "libmoe_get_debug.so")
    monkeypatch.setattr(mg, "_lib", mg._load(path))
    before = mg.debug_status(reset=True)
    say(f"debug status at start: {before}")
    assert mg.debug_status() == (0, 0, 0, 0, 0)
    debug = make_forms(mg)
    st = mg.debug_status()
    say(f"debug status after {len(debug)} layout calls: {st}")
    assert st == (0, 0, 0, 0, len(debug))
    for (name, p0, r0, o0), (_, p1, r1, o1) in zip(release, debug):
        assert torch.equal(p0, p1) and torch.equal(r0, r1), name
        assert (o0 is None) == (o1 is None) and (o0 is None or torch.equal(o0, o1)), name
    assert mg.debug_status(reset=True)[4] == len(debug)
    assert mg.debug_status() == (0, 0, 0, 0, 0)
