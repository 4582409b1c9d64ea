"""GPU parity of the low-latency forms: the padded per-expert layout and the
FP8 (e4m3) cast on dispatch, against the oracle. Bar: bit-exact (layout,
codes and scales; the cast decides integer codes, and both sides take that
decision in fp32: amax, one fp32 division by the scale, round to nearest
even)."""
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
    print(f"[gpu-lowlatency] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_recv_meta(layout_range, recv_stats, stats0, counts_np):
    """The receive metadata against the oracle's (layout_range from counts;
    recv_stats = stats0 + counts)."""
    rng, stats = oracle.padded_recv_meta(counts_np, stats0)
    assert np.array_equal(layout_range.cpu().numpy(), rng)
    assert np.array_equal(recv_stats.cpu().numpy(), stats)


def padded(mg, ids_np, E, M):
    """The padded layout with its receive metadata (the stats starting from
    arbitrary values), every output against the oracle."""
    N, K = ids_np.shape
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, K), dtype=torch.int32, device="cuda")
    row_pair = torch.empty(E * M, dtype=torch.int32, device="cuda")
    status = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    layout_range = torch.full((E,), -7, dtype=torch.int64, device="cuda")
    stats0 = np.random.default_rng(N + E + M).integers(0, 1 << 20, size=E).astype(np.int32)
    recv_stats = dev(stats0)
    ws = torch.empty(max(mg.moe_layout_workspace_bytes(N, K, E), 256), dtype=torch.uint8, device="cuda")
    mg.moe_get_layout_padded(dev(ids_np), E, M, counts, pos, row_pair, ws, status,
                             layout_range=layout_range, recv_stats=recv_stats)
    torch.cuda.synchronize()
    c, p, rp, st = oracle.layout_padded(ids_np, E, M)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(pos.cpu().numpy(), p)
    assert np.array_equal(row_pair.cpu().numpy(), rp)
    assert tuple(status.cpu().tolist()) == st
    check_recv_meta(layout_range, recv_stats, stats0, c)
    return pos, p


@pytest.mark.parametrize("seed", range(8))
def test_padded_layout_random(mg, seed):
    rng = np.random.default_rng(200 + seed)
    E = int(rng.choice([1, 8, 64, 256, 1024]))
    K = int(rng.choice([1, 2, 4, 8]))
    N = int(rng.choice([1, 50, 128, 1000, 4096]))
    M = int(rng.choice([N, max(1, N // 8), 1, 3]))
    ids = rng.integers(-1, E + 1, size=(N, K)).astype(np.int32)
    say(f"padded seed={seed} N={N} K={K} E={E} M={M}")
    padded(mg, ids, E, M)


def test_padded_layout_decode_and_prefill_shapes(mg):
    for name, M in (("decode", 128), ("prefill", 4096)):
        wl = mw.make(name)
        say(f"padded {name} M={M}")
        _, p = padded(mg, wl.ids, wl.E, M)
        assert (p >= 0).all()                        # nothing dropped with M >= N


def _x(rng, N, H):
    x = rng.standard_normal((N, H)) * np.exp(rng.standard_normal((N, 1)) * 2)
    x[0, :128] = 0.0                                  # an all-zero block
    if N > 1:
        x[1, -128:] = 1e30                            # a block of huge values
        x[1, H // 2 + 3] = -2.0 ** -130               # a bf16 subnormal
    return mw.bf16_bits_from_f32(x.astype(np.float32))


@pytest.mark.parametrize("fmt,round_scale", [(0, False), (0, True), (1, False), (1, True), (2, True)])
def test_fp8_dispatch_decode_padded(mg, fmt, round_scale):
    """The decode setting of the low-latency kernels: 128 tokens, hidden 7168,
    top-8 of 256 experts, padded receive buffer M = 128."""
    rng = np.random.default_rng(7 + fmt)
    N, K, E, H, M = 128, 8, 256, 7168, 128
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    x = _x(rng, N, H)
    pos_d, pos = padded(mg, ids, E, M)
    rows = E * M
    say(f"fp8 decode format={fmt} round_scale={round_scale}")
    dst = torch.full((rows, H), 0xA5, dtype=torch.uint8, device="cuda")
    if fmt == 0:
        scales = torch.zeros((rows, H // 128), dtype=torch.float32, device="cuda")
    elif fmt == 1:
        scales = torch.zeros((E, H // 128, M), dtype=torch.float32, device="cuda")
    else:
        scales = torch.zeros((E, H // 512, M), dtype=torch.int32, device="cuda")
    x_d = dev(x.view(np.int16)).view(torch.bfloat16)
    mg.moe_dispatch_fp8(x_d, pos_d, K, dst, scales, fmt, M, round_scale)
    torch.cuda.synchronize()
    codes, ref_scales = oracle.dispatch_fp8(x, pos, rows, fmt, M, round_scale, fill=0xA5)
    assert np.array_equal(dst.cpu().numpy(), codes)
    got = scales.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref_scales.view(np.uint32))


def test_fp8_dispatch_prefill_rows(mg):
    wl = mw.make("prefill")
    rng = np.random.default_rng(11)
    N, H = wl.N, 7168
    x = _x(rng, N, H)
    lay = mg.layout(dev(wl.ids), wl.E)
    torch.cuda.synchronize()
    pos = lay.pos.cpu().numpy()
    say("fp8 prefill rows")
    dst = torch.empty((lay.cap, H), dtype=torch.uint8, device="cuda")
    scales = torch.empty((lay.cap, H // 128), dtype=torch.float32, device="cuda")
    mg.moe_dispatch_fp8(dev(x.view(np.int16)).view(torch.bfloat16), lay.pos, wl.K, dst, scales)
    torch.cuda.synchronize()
    codes, ref_scales = oracle.dispatch_fp8(x, pos, lay.cap)
    assert np.array_equal(dst.cpu().numpy(), codes)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("fmt", [1, 2], ids=["cols", "ue8m0"])
def test_fp8_dispatch_prefill_padded_as_benchmarked(mg, fmt):
    """The low-latency prefill step's dispatch as the benchmark runs it: the
    prefill routing, x from the benchmark's recipe, the padded layout with
    M = N = 4096 rows per expert (2^20 rows, 7.5 GB of codes, no drops) and
    column-major fp32 or UE8M0 scales. Every used row's codes, every scale
    word (unused ones keep their sentinel) and the layout against the
    oracle; the codes are compared on the host, row by row."""
    wl = mw.make("prefill")
    N, K, E, H = wl.N, wl.K, wl.E, 7168
    M = N
    rows = E * M
    round_scale = fmt == 2
    x = mw.make_x(N, H, wl.seed + 104729)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    pos_d = torch.empty((N, K), dtype=torch.int32, device="cuda")
    row_pair = torch.empty(rows, dtype=torch.int32, device="cuda")
    status = torch.empty(2, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(mg.moe_layout_workspace_bytes(N, K, E), 256), dtype=torch.uint8,
                     device="cuda")
    mg.moe_get_layout_padded(dev(wl.ids), E, M, counts, pos_d, row_pair, ws, status)
    c, pos, rp, st = oracle.layout_padded(wl.ids, E, M)
    shape = (E, H // 128, M) if fmt == 1 else (E, H // 512, M)
    sentinel = 3 if fmt == 1 else 0x0B0B0B0B
    say(f"fp8 prefill padded M={M} format={fmt}")
    dst = torch.empty((rows, H), dtype=torch.uint8, device="cuda")
    scales = torch.full(shape, sentinel, dtype=torch.float32 if fmt == 1 else torch.int32,
                        device="cuda")
    mg.moe_dispatch_fp8(dev(x.view(np.int16)).view(torch.bfloat16), pos_d, K, dst, scales, fmt,
                        M, round_scale)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), c) and tuple(status.tolist()) == st
    assert np.array_equal(pos_d.cpu().numpy(), pos)
    assert np.array_equal(row_pair.cpu().numpy(), rp)
    used = np.flatnonzero(rp >= 0)
    # np.zeros leaves the pages of rows the oracle never writes unallocated
    ref_codes, ref_scales = oracle.dispatch_fp8(
        x, pos, rows, fmt, M, round_scale, codes=np.zeros((rows, H), np.uint8),
        scales=np.full(shape, sentinel, np.float32 if fmt == 1 else np.int32))
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))
    assert np.array_equal(dst.cpu().numpy()[used], ref_codes[used])


@pytest.mark.parametrize("H", [128, 384, 640])
def test_fp8_identity_partial_segments(mg, H):
    """pos = None quantises N tokens in place order; H not a multiple of 512
    leaves part of the last wave idle."""
    rng = np.random.default_rng(H)
    N = 33
    x = _x(rng, N, H)
    dst = torch.full((N, H), 0x11, dtype=torch.uint8, device="cuda")
    scales = torch.zeros((N, H // 128 + 3), dtype=torch.float32, device="cuda")   # padded stride
    mg.moe_dispatch_fp8(dev(x.view(np.int16)).view(torch.bfloat16), None, 1, dst, scales)
    torch.cuda.synchronize()
    codes, ref_scales = oracle.dispatch_fp8(x, np.arange(N, dtype=np.int32).reshape(N, 1), N)
    assert np.array_equal(dst.cpu().numpy(), codes)
    s = scales.cpu().numpy()
    assert np.array_equal(s[:, :H // 128].view(np.uint32), ref_scales.view(np.uint32))
    assert (s[:, H // 128:] == 0).all()


def test_fp8_codes_decode_to_torch_float8(mg):
    """The codes are OCP e4m3fn: torch reads them back as float8_e4m3fn."""
    rng = np.random.default_rng(5)
    N, H = 8, 512
    x = _x(rng, N, H)
    dst = torch.empty((N, H), dtype=torch.uint8, device="cuda")
    scales = torch.empty((N, H // 128), dtype=torch.float32, device="cuda")
    mg.moe_dispatch_fp8(dev(x.view(np.int16)).view(torch.bfloat16), None, 1, dst, scales)
    deq = dst.view(torch.float8_e4m3fn).float() * scales.repeat_interleave(128, dim=1)
    xf = dev(x.view(np.int16)).view(torch.bfloat16).float()
    ok = (deq - xf).abs() <= xf.abs() * 2.0 ** -4 + scales.repeat_interleave(128, dim=1) * 2.0 ** -10
    assert bool(ok.all())


@pytest.mark.parametrize("H,fmt", [(512, 2), (1536, 2), (640, 1), (1152, 0)])
def test_fp8_partial_waves_all_formats(mg, H, fmt):
    """One wave covers 1024 channels: H below or between multiples of 1024
    leaves the upper lanes (or the upper UE8M0 word) of the last wave idle."""
    rng = np.random.default_rng(H + fmt)
    N, K, E, M = 300, 4, 16, 128
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[::7, 1] = -1                                  # masked pairs
    x = _x(rng, N, H)
    pos_d, pos = padded(mg, ids, E, M)               # some pairs dropped (M < counts)
    say(f"fp8 partial waves H={H} format={fmt}")
    rows = E * M
    dst = torch.full((rows, H), 0x5A, dtype=torch.uint8, device="cuda")
    shape = {0: (rows, H // 128), 1: (E, H // 128, M), 2: (E, H // 512, M)}[fmt]
    scales = torch.zeros(shape, dtype=torch.int32 if fmt == 2 else torch.float32, device="cuda")
    mg.moe_dispatch_fp8(dev(x.view(np.int16)).view(torch.bfloat16), pos_d, K, dst, scales, fmt, M,
                        fmt == 2)
    torch.cuda.synchronize()
    codes, ref_scales = oracle.dispatch_fp8(x, pos, rows, fmt, M, fmt == 2, fill=0x5A)
    assert np.array_equal(dst.cpu().numpy(), codes)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))


def test_padded_layout_empty_batch(mg):
    E, M = 64, 40
    counts = torch.full((E,), 9, dtype=torch.int32, device="cuda")
    row_pair = torch.zeros(E * M, dtype=torch.int32, device="cuda")
    status = torch.full((2,), 9, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(mg.moe_layout_workspace_bytes(0, 8, E), 256), dtype=torch.uint8, device="cuda")
    ids = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    pos = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    layout_range = torch.full((E,), 9, dtype=torch.int64, device="cuda")
    recv_stats = torch.full((E,), 5, dtype=torch.int32, device="cuda")
    mg.moe_get_layout_padded(ids, E, M, counts, pos, row_pair, ws, status,
                             layout_range=layout_range, recv_stats=recv_stats)
    torch.cuda.synchronize()
    assert (counts.cpu() == 0).all() and (row_pair.cpu() == -1).all()
    assert status.cpu().tolist() == [0, 0]
    assert (layout_range.cpu() == 0).all() and (recv_stats.cpu() == 5).all()


def _fused_case(mg, ids, E, M, x_bits, fmt, round_scale, fill=0x3C):
    """moe_dispatch_fp8_padded against the oracle's padded layout followed by
    its FP8 dispatch: every output bit-exact, untouched rows keep `fill`."""
    N, K = ids.shape
    H = x_bits.shape[1]
    rows = E * M
    counts = torch.full((E,), -9, dtype=torch.int32, device="cuda")
    pos = torch.full((N, K), -9, dtype=torch.int32, device="cuda")
    row_pair = torch.full((rows,), -9, dtype=torch.int32, device="cuda")
    status = torch.full((2,), -9, dtype=torch.int32, device="cuda")
    dst = torch.full((rows, H), fill, dtype=torch.uint8, device="cuda")
    shape = {0: (rows, H // 128), 1: (E, H // 128, M), 2: (E, H // 512, M), 3: (N, H // 128)}[fmt]
    scales = torch.zeros(shape, dtype=torch.int32 if fmt == 2 else torch.float32, device="cuda")
    layout_range = torch.full((E,), -9, dtype=torch.int64, device="cuda")
    stats0 = np.arange(E, dtype=np.int32) * 3
    recv_stats = dev(stats0)
    mg.moe_dispatch_fp8_padded(dev(ids), E, M, dev(x_bits.view(np.int16)).view(torch.bfloat16),
                               counts, pos, row_pair, status, dst, scales, fmt, round_scale,
                               layout_range=layout_range, recv_stats=recv_stats)
    torch.cuda.synchronize()
    c, p, rp, st = oracle.layout_padded(ids, E, M)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(pos.cpu().numpy(), p)
    assert np.array_equal(row_pair.cpu().numpy(), rp)
    assert tuple(status.cpu().tolist()) == st
    check_recv_meta(layout_range, recv_stats, stats0, c)
    codes, ref_scales = oracle.dispatch_fp8(x_bits, p, rows, fmt, M, round_scale, fill=fill)
    assert np.array_equal(dst.cpu().numpy(), codes)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))


@pytest.mark.parametrize("fmt,round_scale", [(0, False), (1, False), (1, True), (2, True), (3, False)])
def test_fused_padded_fp8_decode(mg, fmt, round_scale):
    rng = np.random.default_rng(60 + fmt)
    N, K, E, H, M = 128, 8, 256, 7168, 128
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    say(f"fused decode format={fmt} round_scale={round_scale}")
    _fused_case(mg, ids, E, M, _x(rng, N, H), fmt, round_scale)


@pytest.mark.parametrize("seed", range(6))
def test_fused_padded_fp8_random(mg, seed):
    """Drops (M below the counts), masked and out-of-range ids, duplicate
    experts within a token, H not a multiple of 1024."""
    rng = np.random.default_rng(400 + seed)
    N = int(rng.choice([1, 7, 60, 300]))
    K = int(rng.choice([1, 3, 8, 32]))
    E = int(rng.choice([1, 5, 16, 64]))
    M = int(rng.choice([1, 3, max(1, N * K // max(E, 1))]))
    H = int(rng.choice([128, 640, 1536]))
    ids = rng.integers(-1, E + 2, size=(N, K)).astype(np.int32)
    fmt = int(rng.integers(0, 3)) if H % 512 == 0 else int(rng.integers(0, 2))
    say(f"fused random seed={seed} N={N} K={K} E={E} M={M} H={H} format={fmt}")
    _fused_case(mg, ids, E, M, _x(rng, N, H), fmt, fmt == 2)


def test_fused_padded_fp8_largest_and_empty(mg):
    rng = np.random.default_rng(77)
    N, K, E, H, M = 1024, 8, 64, 512, 100          # N*K = 8192, the limit; drops
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    say("fused largest batch")
    _fused_case(mg, ids, E, M, _x(rng, N, H), 1, False)
    say("fused empty batch")
    _fused_case(mg, np.zeros((0, 8), np.int32), 16, 4, np.zeros((0, 256), np.uint16), 0, False)
    with pytest.raises(mg.MoeError):
        _fused_case(mg, np.zeros((1025, 8), np.int32), 16, 4, np.zeros((1025, 256), np.uint16), 0, False)


# ------------------------------------------- token-major scales + scatter ---

STAGED_CASES = [
    # name, N, K, E, H, M, ids recipe
    ("decode", 128, 8, 256, 7168, 128, "uniform"),
    ("prefill", 4096, 8, 256, 7168, 256, "uniform"),
    ("prefill, N % 8 != 0", 4093, 8, 256, 7168, 256, "uniform"),
    ("drops, M % 64 != 0", 300, 3, 5, 1536, 50, "random"),
    ("E = 1000, tiny M", 500, 8, 1000, 512, 3, "random"),
    ("one token", 1, 4, 16, 1024, 1, "random"),
    ("two gather passes, H = 16384", 64, 4, 16, 16384, 40, "random"),
    ("nb % 4 != 0, H = 1152", 70, 3, 12, 1152, 30, "random"),
]


# UE8M0 words need H % 512 == 0
STAGED_RUNS = [(fmt, c) for fmt in (1, 2) for c in STAGED_CASES if fmt == 1 or c[4] % 512 == 0]


@pytest.mark.parametrize("fmt,case", STAGED_RUNS,
                         ids=[("cols-" if f == 1 else "ue8m0-") + c[0] for f, c in STAGED_RUNS])
def test_fp8_cols_direct_and_staged(mg, case, fmt):
    """Column-major and UE8M0 scales of the padded layout, both ways: the
    one-call dispatch, and per-token scales (MOE_SCALE_TOKENS) placed by
    moe_scatter_scales. Both bit-exact against the oracle's one-call form;
    rows without a pair keep their sentinel."""
    name, N, K, E, H, M, recipe = case
    rng = np.random.default_rng(900 + N + fmt)
    if recipe == "uniform":
        ids = mw.uniform_distinct_ids(rng, N, K, E)
    else:
        ids = rng.integers(-1, E + 2, size=(N, K)).astype(np.int32)
    x = _x(rng, N, H)
    round_scale = fmt == 2
    rows = E * M
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    pos_d = torch.empty((N, K), dtype=torch.int32, device="cuda")
    row_pair = torch.empty(rows, dtype=torch.int32, device="cuda")
    status = torch.empty(2, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(mg.moe_layout_workspace_bytes(N, K, E), 256), dtype=torch.uint8,
                     device="cuda")
    mg.moe_get_layout_padded(dev(ids), E, M, counts, pos_d, row_pair, ws, status)
    _, pos, rp, _ = oracle.layout_padded(ids, E, M)
    shape = (E, H // 128, M) if fmt == 1 else (E, H // 512, M)
    sdt = torch.float32 if fmt == 1 else torch.int32
    sentinel = 3 if fmt == 1 else 0x0B0B0B0B
    x_d = dev(x.view(np.int16)).view(torch.bfloat16)
    ref_codes, ref_scales = oracle.dispatch_fp8(
        x, pos, rows, fmt, M, round_scale, fill=0xA5,
        scales=np.full(shape, sentinel, np.float32 if fmt == 1 else np.int32))
    _, ref_tok = oracle.dispatch_fp8(x, pos, rows, oracle.SCALE_TOKENS, M, round_scale,
                                     codes=np.zeros((rows, H), np.uint8))
    used = rp >= 0

    say(f"fp8 {name} format={fmt} direct")
    dst = torch.full((rows, H), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full(shape, sentinel, dtype=sdt, device="cuda")
    mg.moe_dispatch_fp8(x_d, pos_d, K, dst, scales, fmt, M, round_scale)
    torch.cuda.synchronize()
    assert np.array_equal(dst.cpu().numpy()[used], ref_codes[used])
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))

    # token scales with a padded row stride (one block per gather) and
    # contiguous (four blocks per 16-byte gather when H % 512 == 0)
    for pad in (3, 0):
        say(f"fp8 {name} format={fmt} staged, token-scale row padding {pad}")
        dst.fill_(0xA5)
        scales.fill_(sentinel)
        tok = torch.full((N, H // 128 + pad), -1.0, dtype=torch.float32,
                         device="cuda")[:, : H // 128]
        mg.moe_dispatch_fp8(x_d, pos_d, K, dst, tok, mg.MOE_SCALE_TOKENS, 0, round_scale)
        mg.moe_scatter_scales(tok, K, H, row_pair, E, M, scales, fmt)
        torch.cuda.synchronize()
        assert np.array_equal(dst.cpu().numpy(), ref_codes)
        assert np.array_equal(tok.cpu().numpy().view(np.uint32), ref_tok.view(np.uint32))
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref_scales.view(np.uint32))


def test_scatter_scales_ignores_out_of_range_pairs(mg):
    """row_pair entries outside [0, N*K) leave their rows untouched, so a
    stale or foreign row_pair cannot make the gathers leave token_scales."""
    N, K, E, M, H = 3, 2, 2, 70, 512
    ts = np.arange(N * 4, dtype=np.float32).reshape(N, 4) + 1
    rp = np.full(E * M, -1, np.int32)
    rp[[0, 1, 5, 69, 70, 71, 139]] = [0, 5, 6, 1 << 30, 2, -5, 3]
    ref = oracle.scatter_scales(ts, K, rp, E, M, oracle.SCALE_COLS,
                                scales=np.full((E, 4, M), 9, np.float32))
    got = torch.full((E, 4, M), 9.0, dtype=torch.float32, device="cuda")
    mg.moe_scatter_scales(dev(ts), K, H, dev(rp), E, M, got, mg.MOE_SCALE_COLS)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)
    # rows 0, 1 of expert 0 <- tokens 0, 2; rows 0, 69 of expert 1 <- token 1;
    # entries 6 (= N*K), 2^30 and -5 leave rows 5, 69 of expert 0 and row 1 of expert 1
    assert ref[0, :, 0].tolist() == ts[0].tolist() and ref[0, :, 1].tolist() == ts[2].tolist()
    assert ref[1, :, 0].tolist() == ts[1].tolist() and ref[1, :, 69].tolist() == ts[1].tolist()
    assert (ref[0, :, [5, 69]] == 9).all() and (ref[1, :, 1] == 9).all()
    with pytest.raises(mg.MoeError):
        mg.moe_scatter_scales(dev(ts), K, H, dev(rp), E, M, got, mg.MOE_SCALE_ROWS)
    with pytest.raises(mg.MoeError):
        mg.moe_scatter_scales(dev(ts), K, 500, dev(rp), E, M, got, mg.MOE_SCALE_COLS)


@pytest.mark.parametrize("fmt", [0, 2])
def test_fp8_every_bf16_value(mg, fmt):
    """Every finite bf16 value of magnitude <= 448 (and the infinities and a
    NaN) through the FP8 dispatch with a scale of exactly 1: each 128-channel
    block holds 448 (so amax / 448 = 1, a power of two) and 127 test values,
    so every code is the e4m3 rounding of the bf16 value itself, ties
    included. Bit-exact against the oracle, row-major and UE8M0 scales."""
    vals = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = (vals.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) <= 448.0)
    vals = vals[keep]
    per = 127
    nblk = -(-vals.size // per)
    blocks = np.zeros((nblk, 128), np.uint16)
    blocks[:, 0] = 0x43E0                                 # 448.0 in bf16
    flat = np.concatenate([vals, np.zeros(nblk * per - vals.size, np.uint16)])
    blocks[:, 1:] = flat.reshape(nblk, per)
    H = 7168
    bpt = H // 128
    N = -(-nblk // bpt)
    x = np.zeros((N * bpt, 128), np.uint16)
    x[:nblk] = blocks
    x[nblk:, 0] = 0x43E0
    x = x.reshape(N, H)
    x[N - 1, H - 3] = 0x7FC1                              # NaN
    x[N - 1, H - 2], x[N - 1, H - 1] = 0x7F80, 0xFF80     # +-inf (their block's s becomes inf)
    pos = np.arange(N, dtype=np.int32).reshape(N, 1)
    say(f"fp8 every bf16 value: {vals.size} values in {N} tokens, format {fmt}")
    dst = torch.full((N, H), 0x33, dtype=torch.uint8, device="cuda")
    if fmt == 0:
        scales = torch.zeros((N, bpt), dtype=torch.float32, device="cuda")
    else:
        scales = torch.zeros((1, H // 512, N), dtype=torch.int32, device="cuda")
    mg.moe_dispatch_fp8(dev(x.view(np.int16)).view(torch.bfloat16), dev(pos), 1, dst, scales,
                        fmt, N, True)
    torch.cuda.synchronize()
    codes, ref = oracle.dispatch_fp8(x, pos, N, fmt, N, True, fill=0x33)
    assert np.array_equal(dst.cpu().numpy(), codes)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    # the blocks built from test values really had a scale of 1
    if fmt == 0:
        assert (scales.cpu().numpy().reshape(-1)[:nblk] == 1.0).all()
