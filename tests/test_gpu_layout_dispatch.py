"""GPU parity of moe_layout_dispatch (layout and dispatch in one launch for
batches of at most 8192 pairs) against the oracle's layout followed by its
dispatch. Bar: every output bit-exact; rows past the used ones and alignment
padding keep their canary bytes in the receive buffers and -1 in row_pair."""
import sys

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_get_amd as m

    return m


def say(msg):
    print(f"[gpu-layout-dispatch] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check(mg, ids, E, align, srcs, cap=None, ids_view=None, fill=0xC3):
    """ids: int32 [N, K] (the GPU reads ids_view when given: a strided
    device view); srcs: uint8 [N, bytes] fields."""
    N, K = ids.shape
    if cap is None:
        cap = max(oracle.required_cap(N, K, E, align), 0)
    counts = torch.full((E,), -9, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -9, dtype=torch.int32, device="cuda")
    pos = torch.full((N, K), -9, dtype=torch.int32, device="cuda")
    row_pair = torch.full((cap,), -9, dtype=torch.int32, device="cuda")
    status = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    d_srcs = [dev(s) for s in srcs]
    d_dsts = [torch.full((cap, s.shape[1]), fill, dtype=torch.uint8, device="cuda") for s in srcs]
    mg.moe_layout_dispatch(dev(ids) if ids_view is None else ids_view, E, align, counts, offsets,
                           pos, row_pair, status, d_srcs, d_dsts)
    torch.cuda.synchronize()
    c, o, p, rp, st = oracle.layout(ids, E, align, cap=cap)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(pos.cpu().numpy(), p)
    assert np.array_equal(row_pair.cpu().numpy(), rp)
    assert int(status.cpu()[0]) == st
    for r, d in zip(oracle.dispatch(srcs, p, K, rows=cap, fill=fill), d_dsts):
        assert np.array_equal(d.cpu().numpy(), r)


def test_decode_workload(mg):
    wl = mw.make("decode")
    say("decode workload")
    check(mg, wl.ids, wl.E, 1, [a for _, a in wl.fields])


@pytest.mark.parametrize("seed", range(12))
def test_random(mg, seed):
    """Masks, out-of-range and repeated ids, align > 1, spare capacity, the
    4-byte and 16-byte payload paths."""
    rng = np.random.default_rng(600 + seed)
    N = int(rng.choice([1, 9, 64, 200, 1024]))
    K = int(rng.choice([1, 2, 8, 8]))
    E = int(rng.choice([1, 7, 64, 256, 1024]))
    align = int(rng.choice([1, 1, 4, 16]))
    ids = rng.integers(-1, E + 2, size=(N, K)).astype(np.int32)
    sizes = (96, 16, 32) if seed % 3 else (20, 8, 4 * K)        # 16-byte or 4-byte path
    srcs = [rng.integers(0, 256, size=(N, b), dtype=np.uint8) for b in sizes]
    cap = oracle.required_cap(N, K, E, align) + int(rng.integers(0, 40))
    say(f"random seed={seed} N={N} K={K} E={E} align={align} sizes={sizes}")
    check(mg, ids, E, align, srcs, cap=cap)


def test_records_with_ids_read_in_place(mg):
    """Record mode: one 4096-byte field per token, the ids read from inside
    the records (row stride 1024 int32)."""
    wl = mw.make("large")
    n = 1024                                      # N*K = 8192, the limit
    rec = np.ascontiguousarray(wl.records[:n])
    d_rec = dev(rec)
    ids_view = d_rec.view(torch.int32)[:, :wl.K]
    say("records, ids in place")
    check(mg, wl.ids[:n].copy(), wl.E, 1, [rec], ids_view=ids_view)


def test_empty_and_limit(mg):
    say("empty batch")
    check(mg, np.zeros((0, 8), np.int32), 32, 4, [np.zeros((0, 64), np.uint8)], cap=100)
    with pytest.raises(mg.MoeError):
        check(mg, np.zeros((1025, 8), np.int32), 32, 1, [np.zeros((1025, 64), np.uint8)])


def test_graph_capture_of_the_one_launch_forms(mg):
    """moe_layout_dispatch -> combine and moe_dispatch_fp8_padded captured
    once and replayed on new inputs (eager work and a synchronization between
    replays); every replay equals the eager calls on the same inputs."""
    N, K, E, H, M, P = 100, 8, 32, 512, 60, 256
    cap = oracle.required_cap(N, K, E, 4)
    ids_s = torch.zeros((N, K), dtype=torch.int32, device="cuda")
    src_s = torch.zeros((N, P), dtype=torch.uint8, device="cuda")
    x_s = torch.zeros((N, H), dtype=torch.bfloat16, device="cuda")
    w_s = torch.zeros((N, K), dtype=torch.float32, device="cuda")
    y_s = torch.zeros((cap, 64), dtype=torch.bfloat16, device="cuda")

    def buffers():
        i32 = lambda *s: torch.zeros(s, dtype=torch.int32, device="cuda")
        return dict(counts=i32(E), offsets=i32(E + 1), pos=i32(N, K), row_pair=i32(cap),
                    status=i32(1), recv=torch.zeros((cap, P), dtype=torch.uint8, device="cuda"),
                    out=torch.zeros((N, 64), dtype=torch.bfloat16, device="cuda"),
                    pcounts=i32(E), ppos=i32(N, K), prow_pair=i32(E * M), pstatus=i32(2),
                    codes=torch.zeros((E * M, H), dtype=torch.uint8, device="cuda"),
                    scales=torch.zeros((E, H // 512, M), dtype=torch.int32, device="cuda"))

    def step(b):
        mg.moe_layout_dispatch(ids_s, E, 4, b["counts"], b["offsets"], b["pos"], b["row_pair"],
                               b["status"], [src_s], [b["recv"]])
        mg.moe_combine(y_s, w_s, b["pos"], b["out"])
        mg.moe_dispatch_fp8_padded(ids_s, E, M, x_s, b["pcounts"], b["ppos"], b["prow_pair"],
                                   b["pstatus"], b["codes"], b["scales"], mg.MOE_SCALE_UE8M0, True)

    gb = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(gb)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(gb)
    for rep in range(4):
        say(f"graph replay {rep}")
        rng = np.random.default_rng(700 + rep)
        ids = rng.integers(-1, E + 1, size=(N, K)).astype(np.int32)
        ids_s.copy_(dev(ids))
        src_s.copy_(dev(rng.integers(0, 256, size=(N, P), dtype=np.uint8)))
        x_s.copy_(dev(mw.bf16_bits_from_f32(rng.standard_normal((N, H)).astype(np.float32)).view(np.int16)).view(torch.bfloat16))
        w_s.copy_(dev(rng.standard_normal((N, K)).astype(np.float32)))
        y_s.copy_(dev(mw.bf16_bits_from_f32(rng.standard_normal((cap, 64)).astype(np.float32)).view(np.int16)).view(torch.bfloat16))
        for t in gb.values():
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eb = buffers()
        step(eb)
        torch.cuda.synchronize()
        for name in gb:
            a, b = gb[name], eb[name]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (rep, name)


@pytest.mark.parametrize("seed", range(2000, 2060))
def test_stress(mg, seed):
    """Random shapes over the whole parameter space of the one-launch forms:
    N*K up to the 8192 limit, E up to 1024, K up to 32, masks, out-of-range
    and repeated ids, align up to 16, M below the counts."""
    rng = np.random.default_rng(seed)
    K = int(rng.choice([1, 2, 3, 8, 16, 32]))
    N = int(rng.integers(0, 8192 // K + 1))
    E = int(rng.choice([1, 3, 64, 255, 256, 1024]))
    ids = rng.integers(-2, E + 3, size=(N, K)).astype(np.int32)
    if rng.random() < 0.5 and N:
        ids[:, : max(1, K // 2)] = rng.integers(0, min(E, 4), size=(N, max(1, K // 2)))  # hot experts
    align = int(rng.choice([1, 2, 16]))
    srcs = [rng.integers(0, 256, size=(N, b), dtype=np.uint8) for b in (48, 16)]
    say(f"stress seed={seed} N={N} K={K} E={E} align={align}")
    check(mg, ids, E, align, srcs, cap=oracle.required_cap(N, K, E, align) + int(rng.integers(0, 9)))
    # the padded FP8 form on the same ids
    M = int(rng.choice([1, 5, max(1, N * K // max(E, 1)), max(1, N)]))
    if E * M <= 1 << 20:
        H = 512
        x = mw.bf16_bits_from_f32((rng.standard_normal((N, H)) * 8).astype(np.float32))
        fmt = int(rng.integers(0, 3))
        rows = E * M
        counts = torch.empty(E, dtype=torch.int32, device="cuda")
        pos = torch.empty((N, K), dtype=torch.int32, device="cuda")
        row_pair = torch.empty(rows, dtype=torch.int32, device="cuda")
        status = torch.empty(2, dtype=torch.int32, device="cuda")
        dst = torch.full((rows, H), 0x66, dtype=torch.uint8, device="cuda")
        shape = {0: (rows, H // 128), 1: (E, H // 128, M), 2: (E, H // 512, M)}[fmt]
        scales = torch.zeros(shape, dtype=torch.int32 if fmt == 2 else torch.float32, device="cuda")
        mg.moe_dispatch_fp8_padded(dev(ids), E, M, dev(x.view(np.int16)).view(torch.bfloat16),
                                   counts, pos, row_pair, status, dst, scales, fmt, fmt == 2)
        torch.cuda.synchronize()
        c, p, rp, st = oracle.layout_padded(ids, E, M)
        assert np.array_equal(counts.cpu().numpy(), c) and np.array_equal(pos.cpu().numpy(), p)
        assert np.array_equal(row_pair.cpu().numpy(), rp) and tuple(status.cpu().tolist()) == st
        codes, ref_scales = oracle.dispatch_fp8(x, p, rows, fmt, M, fmt == 2, fill=0x66)
        assert np.array_equal(dst.cpu().numpy(), codes)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))
