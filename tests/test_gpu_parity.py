"""GPU parity: the HIP library against the CPU oracle on the same seeded
inputs, through the C ABI (via the ctypes binding).

Bar: layout and dispatch bit-exact; combine within 1 bf16 ulp (ulp distance
on the ordered bf16 encoding, +0 == -0), 0 expected because both sides run
the same fp32 fma chain in k order and round once to nearest even.
"""
import sys

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
from _util import bf16_ulp_diff

pytestmark = pytest.mark.gpu

ULP_TOL = 1


@pytest.fixture(scope="module")
def mg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_get_amd as m

    return m


def say(msg):
    print(f"[gpu-parity] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host_bf16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def check_layout(mg, lay, ids_np, E, align=1, cap=None):
    torch.cuda.synchronize()
    c, o, p, rp, s = oracle.layout(ids_np, E, align, cap)
    assert np.array_equal(host(lay.counts), c)
    assert np.array_equal(host(lay.offsets), o)
    assert np.array_equal(host(lay.pos), p)
    assert np.array_equal(host(lay.row_pair), rp)
    assert int(host(lay.status)[0]) == s
    return p


def check_plan(order_d, pos_np, tile=None):
    """The layout's dispatch plan: every valid pair (pos >= 0) exactly once,
    -1 in the other entries. With `tile` (pairs per tile, where the header
    documents it), also its arrangement: each tile lists pairs of its own
    range, valid ones first and by ascending receive row."""
    o = host(order_d).reshape(-1)
    p = pos_np.reshape(-1)
    valid = o >= 0
    assert (o[~valid] == -1).all()
    assert np.array_equal(np.sort(o[valid]), np.flatnonzero(p >= 0))
    if tile:
        for s in range(0, o.size, tile):
            seg = o[s:s + tile]
            nv = int((p[s:s + tile] >= 0).sum())
            assert (seg[:nv] >= s).all() and (seg[:nv] < s + tile).all()
            assert (seg[nv:] == -1).all()
            assert (np.diff(p[seg[:nv]]) > 0).all()


def dispatch_with_plan(mg, srcs, lay, K, fill, rows=None):
    """Dispatch in the layout's plan order into fresh buffers; host copies."""
    rows = lay.cap if rows is None else rows
    dsts = [torch.full((rows, a.shape[1]), fill, dtype=torch.uint8, device="cuda") for a in srcs]
    mg.moe_dispatch([dev(a) for a in srcs], dsts, lay.pos, K, order=lay.order)
    torch.cuda.synchronize()
    return [host(d) for d in dsts]


def check_combine(out_d, y_bits, w_np, pos_np):
    ref = oracle.combine(y_bits, np.ascontiguousarray(w_np), pos_np)
    got = host_bf16(out_d)
    d = bf16_ulp_diff(got, ref)
    nz = int((d != 0).sum())
    say(f"combine max ulp {int(d.max(initial=0))}, nonzero {nz} of {d.size}")
    assert d.max(initial=0) <= ULP_TOL
    return nz


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skewed"])
def test_named_workload(mg, name):
    wl = mw.make(name)
    say(f"workload={name} seed={wl.seed} N={wl.N} K={wl.K} E={wl.E} Hc={wl.Hc}")
    ids_d = dev(wl.ids)
    lay = mg.layout(ids_d, wl.E)
    pos = check_layout(mg, lay, wl.ids, wl.E)

    srcs = [a for _, a in wl.fields]
    srcs_d = [dev(a) for a in srcs]
    dsts_d = [torch.full((lay.cap, a.shape[1]), 0xA5, dtype=torch.uint8, device="cuda") for a in srcs]
    mg.moe_dispatch(srcs_d, dsts_d, lay.pos, wl.K)
    torch.cuda.synchronize()
    ref = oracle.dispatch(srcs, pos, wl.K, fill=0xA5)
    for f, (r, d) in enumerate(zip(ref, dsts_d)):
        assert np.array_equal(host(d), r), f"field {f}"
    # the same dispatch visiting the pairs in the layout's plan
    check_plan(lay.order, pos, tile=512 if wl.N * wl.K > 2048 else 1)   # N*K/64 or index order
    for f, (r, d) in enumerate(zip(ref, dispatch_with_plan(mg, srcs, lay, wl.K, 0xA5))):
        assert np.array_equal(d, r), f"field {f}, planned"

    y = wl.y()
    out = mg.combine(dev_bf16(y), dev(wl.weights), lay)
    nz = check_combine(out, y, wl.weights, pos)
    assert nz == 0

    if name == "skewed":
        # identity experts: feed the dispatched bf16 hidden rows back as y
        yid = dsts_d[0].view(torch.bfloat16)
        out2 = mg.combine(yid, dev(wl.weights), lay)
        check_combine(out2, host_bf16(yid), wl.weights, pos)


@pytest.mark.timeout(600)
def test_large_packed_records(mg):
    wl = mw.make("large")
    say(f"workload=large seed={wl.seed} N={wl.N} records={wl.records.shape}")
    rec_d = dev(wl.records)
    ids_d = rec_d.view(torch.int32)[:, : wl.K]          # strided view, stride 1024
    w_d = rec_d.view(torch.float32)[:, 8 : 8 + wl.K]
    lay = mg.layout(ids_d, wl.E)
    pos = check_layout(mg, lay, wl.ids, wl.E)
    recv = torch.empty((lay.cap, wl.records.shape[1]), dtype=torch.uint8, device="cuda")
    mg.moe_dispatch([rec_d], [recv], lay.pos, wl.K)
    torch.cuda.synchronize()
    (ref,) = oracle.dispatch([wl.records], pos, wl.K)
    assert np.array_equal(host(recv), ref)
    check_plan(lay.order, pos, tile=4096)       # 262144 pairs / 64 tiles
    mg.moe_dispatch([rec_d], [recv], lay.pos, wl.K, order=lay.order)
    torch.cuda.synchronize()
    assert np.array_equal(host(recv), ref)
    del ref, recv
    say("large: drawing expert outputs")
    y = wl.y()
    out = mg.combine(dev_bf16(y), w_d, lay)
    assert check_combine(out, y, wl.weights, pos) == 0


def _random_case(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.choice([1, 8, 64, 256, 1024]))
    K = int(rng.choice([1, 2, 4, 8, 8, 3, 32]))
    N = int(rng.choice([0, 1, 7, 64, 333, 1000, 4096]))
    if N * K > 40000:
        N = 40000 // K
    row_bytes = tuple(int(b) for b in rng.choice([16, 48, 112, 4, 12, 4 * K], size=int(rng.integers(1, 5))))
    hc = int(rng.choice([8, 64, 200, 2, 6, 7168]))
    if hc == 7168:
        N = min(N, 256)
    align = int(rng.choice([1, 1, 2, 4, 16]))
    mask = float(rng.choice([0.0, 0.1, 0.5, 1.0]))
    bad = float(rng.choice([0.0, 0.0, 0.02]))
    wl = mw.make_random(seed, N, K, E, hc=hc, row_bytes=row_bytes, mask_frac=mask,
                        bad_frac=bad, distinct=bool(rng.integers(0, 2)))
    extra = int(rng.choice([0, 0, 5]))
    return wl, align, extra


def test_random_stress(mg):
    """Seeds 1000..1199: random sizes, masks, out-of-range ids, alignment,
    capacity slack, 4-byte and 16-byte payloads, odd widths."""
    for seed in range(1000, 1200):
        wl, align, extra = _random_case(seed)
        N, K, E = wl.N, wl.K, wl.E
        cap = mg.moe_required_capacity(N, K, E, align) + extra
        say(f"seed={seed} N={N} K={K} E={E} align={align} cap={cap} "
            f"rows={[a.shape[1] for _, a in wl.fields]} Hc={wl.Hc}")
        lay = mg.layout(dev(wl.ids), E, align=align, cap=cap)
        pos = check_layout(mg, lay, wl.ids, E, align, cap)
        srcs = [a for _, a in wl.fields]
        dsts_d = [torch.full((cap, a.shape[1]), 0x5A, dtype=torch.uint8, device="cuda") for a in srcs]
        mg.moe_dispatch([dev(a) for a in srcs], dsts_d, lay.pos, K)
        torch.cuda.synchronize()
        ref = oracle.dispatch(srcs, pos, K, rows=cap, fill=0x5A)
        for r, d in zip(ref, dsts_d):
            assert np.array_equal(host(d), r)
        check_plan(lay.order, pos)
        for r, d in zip(ref, dispatch_with_plan(mg, srcs, lay, K, 0x5A, rows=cap)):
            assert np.array_equal(d, r)
        rng = np.random.default_rng(seed + 1)
        y = mw.bf16_bits_from_f32(rng.standard_normal((max(cap, 1), wl.Hc)).astype(np.float32))
        out = torch.empty((N, wl.Hc), dtype=torch.bfloat16, device="cuda")
        mg.moe_combine(dev_bf16(y), dev(wl.weights), lay.pos, out)
        check_combine(out, y, wl.weights, pos)


def plan_tile(N, K, E):
    """Pairs per tile of the dispatch plan as the header states it: N*K / B
    rounded up to a multiple of 256 (B = 64 tiles for E <= 256, 32 for
    E <= 512, 16 beyond); 1 (the index order) for at most 2048 pairs or for
    tiles above 4096 pairs."""
    nk = N * K
    if nk <= 2048:
        return 1
    B = 64 if E <= 256 else 32 if E <= 512 else 16
    C = -(-(-(-nk // B)) // 256) * 256
    return C if C <= 4096 else 1


@pytest.mark.parametrize("N,K,E", [(4096, 8, 512), (4096, 8, 1024), (3000, 8, 64), (2731, 3, 256),
                                   (40000, 8, 256), (20000, 4, 1024)])
def test_dispatch_plan_arrangement(mg, N, K, E):
    """The plan's tiles at E past 256 (fewer, larger tiles), a short last
    tile, K = 3, and the index order once tiles would pass 4096 pairs; masked
    and out-of-range ids; the dispatch in the plan's order byte for byte."""
    rng = np.random.default_rng(N + K + E)
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < 0.1] = -1
    ids[rng.random((N, K)) < 0.01] = E + 1
    say(f"plan arrangement N={N} K={K} E={E} tile={plan_tile(N, K, E)}")
    lay = mg.layout(dev(ids), E)
    pos = check_layout(mg, lay, ids, E)
    check_plan(lay.order, pos, tile=plan_tile(N, K, E))
    src = rng.integers(0, 256, size=(N, 160), dtype=np.uint8)
    (ref,) = oracle.dispatch([src], pos, K, fill=0x3C)
    (got,) = dispatch_with_plan(mg, [src], lay, K, 0x3C)
    assert np.array_equal(got, ref)


def test_strided_views_and_untouched_padding(mg):
    rng = np.random.default_rng(7)
    N, K, E, Hc = 300, 4, 16, 64
    ids_full = rng.integers(-1, E, size=(N, 12)).astype(np.int32)
    ids = ids_full[:, 2:2 + K]                         # row stride 12
    lay = mg.layout(dev(ids_full)[:, 2:2 + K], E)
    pos = check_layout(mg, lay, ids, E)
    y = mw.bf16_bits_from_f32(rng.standard_normal((N * K, Hc + 8)).astype(np.float32))
    y_d = dev_bf16(y)[:, :Hc]                          # y row stride Hc + 8
    w_full = rng.standard_normal((N, 2 * K)).astype(np.float32)
    w_d = dev(w_full)[:, K:]                           # w row stride 2K
    out_full = torch.full((N, Hc + 16), 1.5, dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(y_d, w_d, lay.pos, out_full[:, :Hc])
    torch.cuda.synchronize()
    check_combine(out_full[:, :Hc], np.ascontiguousarray(y[:, :Hc]), w_full[:, K:], pos)
    assert (out_full[:, Hc:] == 1.5).all()


def test_pack_unpack_and_record_mode(mg):
    wl = mw.make("tiny")
    srcs_d = [dev(a) for _, a in wl.fields]
    rec = mg.pack_records(srcs_d)
    torch.cuda.synchronize()
    offs, rb = mg.record_offsets([a.shape[1] for _, a in wl.fields])
    assert rb == 4096
    ref = np.zeros((wl.N, rb), np.uint8)
    oracle.dispatch([a for _, a in wl.fields], None, 1,
                    dsts=[ref[:, o:o + a.shape[1]] for o, (_, a) in zip(offs, wl.fields)])
    assert np.array_equal(host(rec), ref)
    back = mg.unpack_records(rec, srcs_d)
    for a, b in zip(srcs_d, back):
        assert torch.equal(a, b)
    lay = mg.layout(dev(wl.ids), wl.E)
    (drec,) = mg.dispatch([rec], lay)
    dsep = mg.dispatch(srcs_d, lay)
    for o, d in zip(offs, dsep):
        assert torch.equal(drec[:, o:o + d.shape[1]], d)


def test_edge_cases(mg):
    # N = 0 with spare capacity: empty results, every row marked unused
    lay = mg.layout(torch.zeros((0, 8), dtype=torch.int32, device="cuda"), 16, cap=10)
    torch.cuda.synchronize()
    assert (lay.counts == 0).all() and (lay.offsets == 0).all()
    assert (lay.row_pair == -1).all() and int(lay.status[0]) == 0
    # all masked
    ids = np.full((50, 8), -1, np.int32)
    lay = mg.layout(dev(ids), 32)
    check_layout(mg, lay, ids, 32)
    out = mg.combine(torch.ones((400, 16), dtype=torch.bfloat16, device="cuda"),
                     torch.ones((50, 8), device="cuda"), lay)
    torch.cuda.synchronize()
    assert (host_bf16(out) == 0).all()                 # +0, not -0
    # E = 1, K = 1, K = 32, E = 1024 with hot experts
    rng = np.random.default_rng(8)
    for (N, K, E) in [(100, 1, 1), (100, 8, 1), (1000, 1, 300), (129, 32, 1024), (5000, 8, 1024),
                      # around the one-workgroup layout's limits (32768 pairs, 512 experts)
                      (4096, 8, 512), (4096, 8, 513), (4097, 8, 256), (1024, 32, 64), (1025, 32, 64)]:
        ids = rng.integers(0, min(E, 3) if E > 3 else E, size=(N, K)).astype(np.int32)
        say(f"edge N={N} K={K} E={E}")
        lay = mg.layout(dev(ids), E)
        check_layout(mg, lay, ids, E)


@pytest.mark.parametrize("N", [255, 256, 257])
@pytest.mark.parametrize("align", [1, 16])
def test_layout_around_the_one_launch_limit(mg, N, align):
    """Batches of at most 2048 pairs take the one-launch layout, larger ones
    the two kernels: both sides of the limit, with padding and spare rows."""
    rng = np.random.default_rng(N * 31 + align)
    K, E = 8, 64
    ids = rng.integers(-1, E + 1, size=(N, K)).astype(np.int32)
    cap = oracle.required_cap(N, K, E, align) + 7
    say(f"layout at N*K={N * K} align={align}")
    lay = mg.layout(dev(ids), E, align, cap=cap)
    check_layout(mg, lay, ids, E, align, cap)


@pytest.mark.parametrize("N,E,M,with_status", [(256, 64, 4096, True), (256, 64, 4097, True),
                                               (257, 64, 64, True), (100, 16, 40, False)])
def test_padded_layout_around_the_one_launch_limits(mg, N, E, M, with_status):
    """The padded layout's one-launch form (N*K <= 2048, E*M <= 2^18, status
    given) and its two-kernel form agree with the oracle on both sides."""
    rng = np.random.default_rng(N + E + M)
    K = 8
    ids = rng.integers(-1, E + 1, size=(N, K)).astype(np.int32)
    counts = torch.full((E,), -3, dtype=torch.int32, device="cuda")
    pos = torch.full((N, K), -3, dtype=torch.int32, device="cuda")
    row_pair = torch.full((E * M,), -3, dtype=torch.int32, device="cuda")
    status = torch.full((2,), -3, dtype=torch.int32, device="cuda") if with_status else None
    ws = torch.empty(mg.moe_layout_workspace_bytes(N, K, E), dtype=torch.uint8, device="cuda")
    say(f"padded layout N*K={N * K} E*M={E * M} status={with_status}")
    mg.moe_get_layout_padded(dev(ids), E, M, counts, pos, row_pair, ws, status)
    torch.cuda.synchronize()
    c, p, rp, st = oracle.layout_padded(ids, E, M)
    assert np.array_equal(host(counts), c) and np.array_equal(host(pos), p)
    assert np.array_equal(host(row_pair), rp)
    if with_status:
        assert tuple(host(status).tolist()) == st


@pytest.mark.parametrize("Hc,N", [(131072, 24), (65538, 16), (16392, 64)])
def test_wide_rows(mg, Hc, N):
    """Rows far wider than the workloads': combine over 256 and 129 segments
    (16-byte and 4-byte paths: Hc % 8 != 0 takes the 4-byte one), dispatch of
    256 KiB payload rows, and the FP8 cast over 64 1024-channel segments."""
    rng = np.random.default_rng(Hc)
    K, E = 8, 16
    ids = rng.integers(-1, E, size=(N, K)).astype(np.int32)
    lay = mg.layout(dev(ids), E)
    pos = check_layout(mg, lay, ids, E)
    say(f"wide combine Hc={Hc} N={N}")
    y = mw.bf16_bits_from_f32(rng.standard_normal((lay.cap, Hc)).astype(np.float32))
    w = rng.standard_normal((N, K)).astype(np.float32)
    out = mg.combine(dev_bf16(y), dev(w), lay)
    assert check_combine(out, y, w, pos) == 0
    if Hc % 16 == 0:
        say(f"wide dispatch {2 * Hc} B rows")
        src = rng.integers(0, 256, size=(N, 2 * Hc), dtype=np.uint8)
        (recv,) = mg.dispatch([dev(src)], lay)
        torch.cuda.synchronize()
        valid = pos.reshape(-1) >= 0
        tok = np.repeat(np.arange(N), K)[valid]
        assert np.array_equal(host(recv)[pos.reshape(-1)[valid]], src[tok])
        say("wide fp8 cast, ue8m0")
        H = Hc // 2
        x = mw.bf16_bits_from_f32((rng.standard_normal((N, H)) * 4).astype(np.float32))
        dst = torch.full((lay.cap, H), 0x11, dtype=torch.uint8, device="cuda")
        M = lay.cap
        scales = torch.zeros((1, H // 512, M), dtype=torch.int32, device="cuda")
        # one "expert" of M rows: the column-major forms index rows p directly
        mg.moe_dispatch_fp8(dev_bf16(x), lay.pos, K, dst, scales, mg.MOE_SCALE_UE8M0, M, True)
        torch.cuda.synchronize()
        codes, ref = oracle.dispatch_fp8(x, pos, lay.cap, oracle.SCALE_UE8M0, M, True, fill=0x11)
        assert np.array_equal(host(dst), codes)
        assert np.array_equal(host(scales).view(np.uint32), ref.view(np.uint32))


def misaligned_copy(ids: np.ndarray) -> torch.Tensor:
    """The ids on the GPU at an address 4 bytes past a 16-byte boundary (still
    contiguous), which routes a layout away from its one-pass form."""
    flat = torch.empty(ids.size + 1, dtype=torch.int32, device="cuda")
    view = flat[1:].view(ids.shape)
    view.copy_(torch.from_numpy(np.ascontiguousarray(ids)))
    assert view.data_ptr() % 16 == 4
    return view


@pytest.mark.parametrize("N,K,E,align", [(2049, 1, 64, 1), (1025, 4, 256, 16), (1537, 8, 1024, 1),
                                         (4096, 8, 256, 1), (4096, 8, 256, 8), (4096, 8, 128, 1),
                                         (8192, 4, 512, 4), (32768, 1, 256, 1),
                                         (32769, 1, 256, 1), (4097, 8, 256, 1)])
def test_layout_around_the_one_pass_limits(mg, N, K, E, align):
    """Batches of 2049 .. 32768 contiguous, 16-byte-aligned pairs take the
    one-pass layout (every workgroup counts the whole batch); a ragged last
    round of loads (N*K not a multiple of 1024), E up to 1024 (16 chunks),
    alignment padding, masks, ids >= E and a hot expert. The same ids 4 bytes
    off a 16-byte boundary take the two kernels; both match the oracle, and
    so do the plans' tiles."""
    rng = np.random.default_rng(N * 7 + K + E + align)
    ids = mw.uniform_distinct_ids(rng, N, K, E) if K <= E else rng.integers(0, E, (N, K))
    ids = ids.astype(np.int32)
    ids[rng.random((N, K)) < 0.05] = -1
    ids[rng.random((N, K)) < 0.01] = E + 2
    ids[rng.random((N, K)) < 0.1] = 3                 # hot expert
    cap = oracle.required_cap(N, K, E, align) + 5
    for form, ids_d in (("aligned", dev(ids)), ("misaligned", misaligned_copy(ids))):
        say(f"layout N={N} K={K} E={E} align={align} ids {form}")
        lay = mg.layout(ids_d, E, align=align, cap=cap)
        pos = check_layout(mg, lay, ids, E, align, cap)
        check_plan(lay.order, pos, tile=plan_tile(N, K, E))


@pytest.mark.parametrize("N,E,M", [(4096, 256, 4096), (3000, 64, 200), (1024, 128, 96)])
def test_padded_layout_one_pass(mg, N, E, M):
    """The padded layout on 2049 .. 32768 pairs: the one-pass form marks the
    E*M rows from more workgroups than chunks; pairs past an expert's M rows
    dropped; the ids off a 16-byte boundary take the two kernels."""
    rng = np.random.default_rng(N + E + M)
    K = 8
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < 0.05] = -1
    ids[rng.random((N, K)) < 0.01] = E
    c, p, rp, st = oracle.layout_padded(ids, E, M)
    for form, ids_d in (("aligned", dev(ids)), ("misaligned", misaligned_copy(ids))):
        counts = torch.full((E,), -3, dtype=torch.int32, device="cuda")
        pos = torch.full((N, K), -3, dtype=torch.int32, device="cuda")
        row_pair = torch.full((E * M,), -3, dtype=torch.int32, device="cuda")
        status = torch.full((2,), -3, dtype=torch.int32, device="cuda")
        ws = torch.empty(mg.moe_layout_workspace_bytes(N, K, E), dtype=torch.uint8, device="cuda")
        say(f"padded layout N={N} E={E} M={M} ids {form}")
        mg.moe_get_layout_padded(ids_d, E, M, counts, pos, row_pair, ws, status)
        torch.cuda.synchronize()
        assert np.array_equal(host(counts), c) and np.array_equal(host(pos), p)
        assert np.array_equal(host(row_pair), rp)
        assert tuple(host(status).tolist()) == st


@pytest.mark.parametrize("N,K,E", [(4096, 8, 256), (4097, 8, 256), (4096, 8, 600)])
def test_layout_paths_agree_on_uniform_and_skewed_ids(mg, N, K, E):
    """The layout forms (one pass at 32768 pairs, histogram + assign past it)
    against the oracle on the same kind of routing, with masks and a hot
    expert."""
    rng = np.random.default_rng(N + E)
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < 0.05] = -1
    ids[rng.random((N, K)) < 0.2] = 3                  # hot expert (duplicates within a token)
    for align in (1, 8):
        say(f"layout paths N={N} K={K} E={E} align={align}")
        lay = mg.layout(dev(ids), E, align=align)
        check_layout(mg, lay, ids, E, align)


def test_non_finite_values(mg):
    """inf and NaN propagate as in the oracle (any NaN payload counts as NaN)."""
    N, K, Hc = 4, 2, 16
    ids = np.array([[0, 1], [1, 0], [0, -1], [1, 1]], np.int32)
    lay = mg.layout(dev(ids), 2)
    pos = check_layout(mg, lay, ids, 2)
    y = np.full((N * K, Hc), 0x3F80, np.uint16)        # 1.0
    y[0, 0] = 0x7F80                                   # +inf
    y[1, 1] = 0xFF80                                   # -inf
    y[2, 2] = 0x7FC1                                   # NaN
    y[0, 3], y[1, 3] = 0x7F80, 0xFF80                  # inf - inf -> NaN
    y[3, 4] = 0x7F7F                                   # max finite: overflow in the sum
    w = np.array([[1, 1], [1, 1], [1, 1], [2, 2]], np.float32)
    out = host_bf16(mg.combine(dev_bf16(y), dev(w), lay))
    ref = oracle.combine(y, w, pos)
    nan_o = ((out & 0x7F80) == 0x7F80) & ((out & 0x7F) != 0)
    nan_r = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    assert np.array_equal(nan_o, nan_r) and nan_r.any()
    assert np.array_equal(out[~nan_o], ref[~nan_r])


def test_non_default_stream(mg):
    wl = mw.make("decode")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ids_d = dev(wl.ids)
        lay = mg.layout(ids_d, wl.E)
        srcs_d = [dev(a) for _, a in wl.fields]
        dsts = mg.dispatch(srcs_d, lay)
        y = wl.y()
        out = mg.combine(dev_bf16(y), dev(wl.weights), lay)
    s.synchronize()
    pos = check_layout(mg, lay, wl.ids, wl.E)
    for r, d in zip(oracle.dispatch([a for _, a in wl.fields], pos, wl.K), dsts):
        assert np.array_equal(host(d), r)
    check_combine(out, y, wl.weights, pos)


def test_explicit_stream_argument(mg):
    """The allocating wrappers given stream= (not a stream context) allocate
    on that stream, so blocks they free (the layout's workspace) are not
    handed to the current stream while the kernels on the given stream still
    use them. The current stream meanwhile allocates and fills blocks of the
    workspace's size; every result must still match the oracle."""
    rng = np.random.default_rng(4242)
    N, K, E, Hc = 1500, 8, 64, 512
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < 0.1] = -1
    src = rng.integers(0, 256, size=(N, 272), dtype=np.uint8)
    w = rng.standard_normal((N, K)).astype(np.float32)
    y = mw.bf16_bits_from_f32(rng.standard_normal((N * K, Hc)).astype(np.float32))
    ids_d, src_d, w_d, y_d = dev(ids), dev(src), dev(w), dev_bf16(y)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    nbytes = max(mg.moe_layout_workspace_bytes(N, K, E), 256)
    for rep in range(3):
        say(f"explicit stream argument, pass {rep}")
        lay = mg.layout(ids_d, E, stream=s)
        junk = [torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(8)]
        (recv,) = mg.dispatch([src_d], lay, stream=s)
        out = mg.combine(y_d, w_d, lay, stream=s)
        s.synchronize()
        pos = check_layout(mg, lay, ids, E)
        (ref,) = oracle.dispatch([src], pos, K)
        valid = pos.reshape(-1)[pos.reshape(-1) >= 0]
        assert np.array_equal(host(recv)[valid], ref[valid])
        assert check_combine(out, y, w, pos) == 0
        del junk


@pytest.mark.parametrize("N,fused", [(281, False), (282, False), (1016, True), (1017, True)])
def test_dispatch_on_both_sides_of_the_store_form_switch(mg, N, fused):
    """Receives of at most 16 MiB are written with ordinary stores, larger
    ones with non-temporal stores. moe_dispatch of the prefill fields (7456
    bytes per row, 8 rows per token) at 281 tokens (16 761 088 bytes) and 282
    (16 820 736); moe_layout_dispatch of 2064-byte rows at 1016 tokens
    (16 776 192 bytes) and 1017 (16 792 704). Every byte, untouched rows
    included, against the oracle."""
    K, E = 8, 64
    rng = np.random.default_rng(900 + N)
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < 0.1] = -1
    sizes = [2064] if fused else [7168, 224, 32, 32]
    srcs = [rng.integers(0, 256, (N, b), dtype=np.uint8) for b in sizes]
    _, _, pos, rp, _ = oracle.layout(ids, E)
    ref = oracle.dispatch(srcs, pos, K, rows=N * K, fill=0xEE)
    say(f"store forms: N={N} fused={fused}, {N * K * sum(sizes)} receive bytes")
    if fused:
        i32 = lambda *sh: torch.empty(sh, dtype=torch.int32, device="cuda")
        dsts = [torch.full((N * K, b), 0xEE, dtype=torch.uint8, device="cuda") for b in sizes]
        pos_d, rp_d = i32(N, K), i32(N * K)
        mg.moe_layout_dispatch(dev(ids), E, 1, i32(E), i32(E + 1), pos_d, rp_d, i32(1),
                               [dev(x) for x in srcs], dsts)
        torch.cuda.synchronize()
        assert np.array_equal(host(pos_d), pos) and np.array_equal(host(rp_d), rp)
        got = [host(d) for d in dsts]
    else:
        lay = mg.layout(dev(ids), E)
        check_layout(mg, lay, ids, E)
        got = dispatch_with_plan(mg, srcs, lay, K, 0xEE)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)


@pytest.mark.parametrize("Hc,N,K", [(7168, 2340, 8), (7168, 2341, 8), (6, 32768, 12),
                                     (6, 32769, 12), (7168, 2341, 12)])
def test_combine_on_both_sides_of_the_load_form_switch(mg, Hc, N, K):
    """Jobs of at most 32768 waves (one per token and 64-vector segment)
    issue a lane's row loads together, larger ones one at a time: both forms,
    16-byte (Hc = 7168: 14 segments per token) and 4-byte (Hc = 6) loads,
    one and two batches of 8 pairs, masked pairs, for the combine and the
    dispatch backward (unit weights, weight-gradient sums). Past the switch,
    the combine of 16-byte rows with K <= 8 takes the held form (2341 x 8);
    with K = 12 it loads one row at a time."""
    rng = np.random.default_rng(N * 31 + K)
    E = 64
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < 0.15] = -1
    lay = mg.layout(dev(ids), E)
    pos = check_layout(mg, lay, ids, E)
    say(f"load forms: Hc={Hc} N={N} K={K}")
    y = mw.bf16_bits_from_f32(rng.standard_normal((lay.cap, Hc)).astype(np.float32))
    w = rng.standard_normal((N, K)).astype(np.float32)
    y_d = dev_bf16(y)
    out = mg.combine(y_d, dev(w), lay)
    assert check_combine(out, y, w, pos) == 0
    grw = rng.standard_normal((lay.cap, K)).astype(np.float32)
    gx = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    gw = torch.empty((N, K), dtype=torch.float32, device="cuda")
    mg.moe_dispatch_backward(y_d, lay.pos, gx, dev(grw), gw)
    torch.cuda.synchronize()
    ref_x, ref_w = oracle.dispatch_backward(y, pos, grw)
    assert np.array_equal(host_bf16(gx), ref_x)
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))


@pytest.mark.parametrize("Hc,N,K,mask,strided", [
    (4096, 4096, 8, 0.0, False),      # 32768 waves: the loads issued together
    (4096, 4097, 8, 0.0, False),      # 32776 waves: held, 17 tokens per workgroup
    (7168, 2341, 8, 0.1, True),       # held, a last workgroup of 1 token, strided rows
    (7176, 2400, 5, 0.1, False),      # 15 segments, the last one a single vector
    (8192, 4096, 8, 0.2, False),      # 2 rounds of 8 tokens per workgroup
    (4104, 5000, 1, 0.0, True),       # 9 segments, K = 1
    (4096, 20000, 8, 0.05, False),    # 3 rounds
    (114688, 147, 3, 0.0, False),     # 224 segments: 1 token per workgroup
    (115200, 150, 2, 0.0, False),     # 225 segments: past the held form, one load at a time
    (4096, 4100, 12, 0.1, False),     # K > 8: one load at a time
])
def test_combine_held_form(mg, Hc, N, K, mask, strided):
    """Large batches of 16-byte rows with K <= 8 and 8 to 224 segments per
    row take the held form (each workgroup stores its tokens' sums after its
    last row load): bit-identical to the oracle on both sides of every limit
    of the form, with ragged last workgroups, several rounds of workgroups,
    a one-vector last segment, masked pairs, all-masked tokens and strided
    rows whose padding stays untouched."""
    rng = np.random.default_rng(Hc * 7 + N * 3 + K)
    E = 64
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < mask] = -1
    if mask > 0:
        ids[::97] = -1                       # tokens with every pair masked
    lay = mg.layout(dev(ids), E)
    pos = check_layout(mg, lay, ids, E)
    say(f"held form: Hc={Hc} N={N} K={K} mask={mask} strided={strided}")
    y = mw.bf16_bits_from_f32(rng.standard_normal((lay.cap, Hc)).astype(np.float32))
    w = rng.standard_normal((N, K)).astype(np.float32)
    pad = 24 if strided else 0
    y_d = torch.zeros((lay.cap, Hc + pad), dtype=torch.bfloat16, device="cuda")
    y_d[:, :Hc] = dev_bf16(y)
    out = torch.full((N, Hc + pad), -7.0, dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(y_d[:, :Hc], dev(w), lay.pos, out[:, :Hc])
    torch.cuda.synchronize()
    assert check_combine(out[:, :Hc], y, w, pos) == 0
    if strided:
        assert bool((out[:, Hc:] == -7.0).all())
    # the dispatch backward (unit weights, with the weight-gradient sums) on
    # the same rows takes the same form
    grw = rng.standard_normal((lay.cap, K)).astype(np.float32)
    gx = torch.full((N, Hc + pad), -7.0, dtype=torch.bfloat16, device="cuda")
    gw = torch.empty((N, K), dtype=torch.float32, device="cuda")
    mg.moe_dispatch_backward(y_d[:, :Hc], lay.pos, gx[:, :Hc], dev(grw), gw)
    torch.cuda.synchronize()
    ref_x, ref_w = oracle.dispatch_backward(y, pos, grw)
    assert np.array_equal(host_bf16(gx[:, :Hc]), ref_x)
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))
    if strided:
        assert bool((gx[:, Hc:] == -7.0).all())


def test_concurrent_streams(mg):
    """The library keeps no state between calls: four streams (default
    priority) each run layout -> dispatch -> combine on their own batch and
    buffers, all enqueued before any is waited for, twice over, and every
    result matches the oracle. Batches of both layout forms (one launch and
    histogram + assign) run side by side."""
    cases = []
    for i, N in enumerate([96, 1500, 300, 2600]):
        rng = np.random.default_rng(700 + i)
        K, E = 8, 64
        ids = mw.uniform_distinct_ids(rng, N, K, E)
        ids[rng.random((N, K)) < 0.1] = -1
        src = rng.integers(0, 256, size=(N, 272), dtype=np.uint8)
        w = rng.standard_normal((N, K)).astype(np.float32)
        y = mw.bf16_bits_from_f32(rng.standard_normal((N * K, 512)).astype(np.float32))
        cases.append((ids, src, w, y, E))
    streams = [torch.cuda.Stream() for _ in cases]
    for rep in range(2):
        say(f"concurrent streams, pass {rep}")
        outs = []
        for (ids, src, w, y, E), s in zip(cases, streams):
            with torch.cuda.stream(s):
                lay = mg.layout(dev(ids), E)
                (recv,) = mg.dispatch([dev(src)], lay)
                out = mg.combine(dev_bf16(y), dev(w), lay)
                outs.append((lay, recv, out))
        torch.cuda.synchronize()
        for (ids, src, w, y, E), (lay, recv, out) in zip(cases, outs):
            pos = check_layout(mg, lay, ids, E)
            (ref,) = oracle.dispatch([src], pos, ids.shape[1])
            valid = pos.reshape(-1) >= 0
            assert np.array_equal(host(recv)[pos.reshape(-1)[valid]], ref[pos.reshape(-1)[valid]])
            assert check_combine(out, y, w, pos) == 0


@pytest.mark.parametrize("N,misalign", [(256, False), (1024, False), (1024, True)],
                         ids=["one-launch layout", "one-pass layout", "two-kernel layout"])
def test_graph_capture_replay(mg, N, misalign):
    """layout + dispatch + combine captured once and replayed on new inputs
    (eager work and a sync between replays); every replay checked. 2048
    pairs take the one-launch layout, 8192 contiguous pairs the one-pass
    kernel, and the same 8192 ids 4 bytes off a 16-byte boundary the two
    kernels."""
    K, E, Hc = 8, 64, 512
    if misalign:
        ids_s = torch.zeros(N * K + 1, dtype=torch.int32, device="cuda")[1:].view(N, K)
        assert ids_s.data_ptr() % 16 == 4
    else:
        ids_s = torch.zeros((N, K), dtype=torch.int32, device="cuda")
    x_s = torch.zeros((N, 1024), dtype=torch.uint8, device="cuda")
    w_s = torch.zeros((N, K), dtype=torch.float32, device="cuda")
    y_s = torch.zeros((N * K, Hc), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mg.moe_layout_workspace_bytes(N, K, E), dtype=torch.uint8, device="cuda")
    lay = mg.Layout(torch.empty(E, dtype=torch.int32, device="cuda"),
                    torch.empty(E + 1, dtype=torch.int32, device="cuda"),
                    torch.empty((N, K), dtype=torch.int32, device="cuda"),
                    torch.empty(N * K, dtype=torch.int32, device="cuda"),
                    torch.empty(1, dtype=torch.int32, device="cuda"), E, 1)
    recv = torch.empty((N * K, 1024), dtype=torch.uint8, device="cuda")
    out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")

    def step():
        mg.moe_get_layout(ids_s, E, 1, lay.counts, lay.offsets, lay.pos, lay.row_pair, ws,
                          lay.status)
        mg.moe_dispatch([x_s], [recv], lay.pos, K)
        mg.moe_combine(y_s, w_s, lay.pos, out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                          # warm up outside capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        say(f"graph replay {rep}, N={N} misaligned ids={misalign}")
        rng = np.random.default_rng(50 + rep + N)
        ids = mw.uniform_distinct_ids(rng, N, K, E)
        ids[rng.random((N, K)) < 0.1] = -1
        x = rng.integers(0, 256, size=(N, 1024), dtype=np.uint8)
        w = rng.standard_normal((N, K)).astype(np.float32)
        y = mw.bf16_bits_from_f32(rng.standard_normal((N * K, Hc)).astype(np.float32))
        ids_s.copy_(dev(ids))
        x_s.copy_(dev(x))
        w_s.copy_(dev(w))
        y_s.copy_(dev_bf16(y))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        pos = check_layout(mg, lay, ids, E)
        (ref,) = oracle.dispatch([x], pos, K, rows=N * K)
        got = host(recv)
        used = host(lay.row_pair) >= 0
        assert np.array_equal(got[used], ref[used])
        check_combine(out, y, w, pos)
        _ = (y_s.float() * 2).sum().item()             # unrelated eager work between replays


def test_graph_capture_replay_held_combine(mg):
    """The held form of the combine (2400 tokens of 7168 channels, top-8)
    captured in a HIP graph and replayed on new expert rows and weights, with
    eager work between the replays: every replay equals the oracle."""
    N, K, E, Hc = 2400, 8, 64, 7168
    rng = np.random.default_rng(4242)
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < 0.05] = -1
    lay = mg.layout(dev(ids), E)
    pos = check_layout(mg, lay, ids, E)
    y_s = torch.zeros((lay.cap, Hc), dtype=torch.bfloat16, device="cuda")
    w_s = torch.zeros((N, K), dtype=torch.float32, device="cuda")
    out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mg.moe_combine(y_s, w_s, lay.pos, out)          # warm up outside capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mg.moe_combine(y_s, w_s, lay.pos, out)
    for rep in range(3):
        say(f"held combine graph replay {rep}")
        y = mw.bf16_bits_from_f32(rng.standard_normal((lay.cap, Hc)).astype(np.float32))
        w = rng.standard_normal((N, K)).astype(np.float32)
        y_s.copy_(dev_bf16(y))
        w_s.copy_(dev(w))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert check_combine(out, y, w, pos) == 0
        _ = (y_s.float() * 2).sum().item()             # unrelated eager work between replays


def test_errors_raise(mg):
    ids = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(mg.MoeError) as e:
        mg.layout(ids, 2, cap=7)
    assert e.value.code == mg.MOE_ERR_CAPACITY
    with pytest.raises(mg.MoeError) as e:
        mg.layout(ids, 2000)
    assert e.value.code == mg.MOE_ERR_LIMIT
    lay = mg.layout(ids, 2)
    y = torch.zeros((8, 7), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mg.MoeError) as e:
        mg.combine(y, torch.ones((4, 2), device="cuda"), lay)
    assert e.value.code == mg.MOE_ERR_ALIGN
    x = torch.zeros((4, 6), dtype=torch.uint8, device="cuda")
    with pytest.raises(mg.MoeError) as e:
        mg.dispatch([x], lay)
    assert e.value.code == mg.MOE_ERR_ALIGN
