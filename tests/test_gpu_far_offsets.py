"""Byte offsets past 4 GiB.

Every kernel forms a row's address as a 64-bit product of a row index and a
row stride. Here each strided operand is a view whose rows are spread over
about 4.5 GiB, so its last rows start more than 4 GiB past the base (an
address computed in 32 bits would wrap). The results are checked against the
oracle on compact host copies of the same inputs, to the usual bar: layout,
dispatch, the FP8 cast and the unit-weight sums bit-exact, combine within
1 bf16 ulp, weight-gradient dot products within the bound of their sum tree.
"""
import sys

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
from _util import bf16_ulp_diff, bf16_bits_to_float

pytestmark = pytest.mark.gpu

GiB = 1 << 30
SPAN = 4 * GiB + GiB // 2


@pytest.fixture(scope="module")
def mg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_get_amd as m

    return m


@pytest.fixture(autouse=True)
def _release():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(msg):
    print(f"[far-offsets] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits(a):
    return mw.bf16_bits_from_f32(np.asarray(a, np.float32))


def far(rows, cols, dtype, src=None, fill=None):
    """A [rows, cols] device view with contiguous rows spread over SPAN bytes
    (row stride a multiple of 16 B), so rows past 4 GiB / stride start more
    than 4 GiB after the first. Filled from the device tensor `src` or with
    `fill`; the bytes between rows are never read or written."""
    es = torch.tensor([], dtype=dtype).element_size()
    row_bytes = max(SPAN // rows // 16 * 16, -(-cols * es // 16) * 16)
    assert (rows - 1) * row_bytes > 4 * GiB, "too few rows to reach past 4 GiB"
    stride = row_bytes // es
    buf = torch.empty((rows - 1) * stride + cols, dtype=dtype, device="cuda")
    v = buf.as_strided((rows, cols), (stride, 1))
    if src is not None:
        v.copy_(src)
    elif fill is not None:
        v.fill_(fill)
    return v


def routing(seed, N, K, E, mask=0.1, bad=0.0):
    rng = np.random.default_rng(seed)
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < mask] = -1
    ids[rng.random((N, K)) < bad] = E + 3
    return rng, ids


# -------------------------------------------------------------- layout ---

@pytest.mark.parametrize("N", [4096, 128])
def test_layout_far_ids(mg, N):
    """ids read through a row stride past 4 GiB: the histogram + assign pair
    (4096 tokens) and the one-launch form (128 tokens), plain and padded."""
    K, E = 8, 256
    _, ids = routing(N, N, K, E, mask=0.05, bad=0.01)
    ids_d = far(N, K, torch.int32, src=dev(ids))
    say(f"layout N={N} ids row stride {ids_d.stride(0) * 4} B")
    lay = mg.layout(ids_d, E)
    torch.cuda.synchronize()
    c, o, p, rp, s = oracle.layout(ids, E)
    assert np.array_equal(lay.counts.cpu().numpy(), c)
    assert np.array_equal(lay.offsets.cpu().numpy(), o)
    assert np.array_equal(lay.pos.cpu().numpy(), p)
    assert np.array_equal(lay.row_pair.cpu().numpy(), rp)
    assert int(lay.status.cpu()[0]) == s > 0

    M = 64 if N > 1000 else 8      # some experts overflow their M rows
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, K), dtype=torch.int32, device="cuda")
    row_pair = torch.empty(E * M, dtype=torch.int32, device="cuda")
    status = torch.empty(2, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(mg.moe_layout_workspace_bytes(N, K, E), 256), dtype=torch.uint8,
                     device="cuda")
    mg.moe_get_layout_padded(ids_d, E, M, counts, pos, row_pair, ws, status)
    torch.cuda.synchronize()
    c, p, rp, st = oracle.layout_padded(ids, E, M)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(pos.cpu().numpy(), p)
    assert np.array_equal(row_pair.cpu().numpy(), rp)
    assert tuple(status.cpu().tolist()) == st and st[1] > 0


# ------------------------------------------------------------ dispatch ---

def test_dispatch_far_rows(mg):
    """Sources and receive rows both spread past 4 GiB: 16-byte fields, a
    12-byte field (4-byte vectors), and the one-launch layout + dispatch."""
    N, K, E = 64, 8, 16
    rng, ids = routing(5, N, K, E)
    lay = mg.layout(dev(ids), E)
    torch.cuda.synchronize()
    pos = lay.pos.cpu().numpy()
    cap = lay.cap
    for row_bytes in ((1024, 32), (12,)):
        srcs = [rng.integers(0, 256, size=(N, b), dtype=np.uint8) for b in row_bytes]
        src_d = [far(N, b, torch.uint8, src=dev(s)) for s, b in zip(srcs, row_bytes)]
        dst_d = [far(cap, b, torch.uint8, fill=0xA5) for b in row_bytes]
        say(f"dispatch fields {row_bytes}: dst row stride {dst_d[0].stride(0)} B")
        mg.moe_dispatch(src_d, dst_d, lay.pos, K)
        torch.cuda.synchronize()
        ref = oracle.dispatch(srcs, pos, K, rows=cap, fill=0xA5)
        for got, want in zip(dst_d, ref):
            assert np.array_equal(got.cpu().numpy(), want)
        del src_d, dst_d

    say("layout + dispatch in one launch, far ids, sources and rows")
    src = rng.integers(0, 256, size=(N, 2048), dtype=np.uint8)
    ids_d = far(N, K, torch.int32, src=dev(ids))
    src_d = far(N, 2048, torch.uint8, src=dev(src))
    dst_d = far(cap, 2048, torch.uint8, fill=0x5A)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    pos_d = torch.empty((N, K), dtype=torch.int32, device="cuda")
    row_pair = torch.empty(cap, dtype=torch.int32, device="cuda")
    status = torch.empty(1, dtype=torch.int32, device="cuda")
    mg.moe_layout_dispatch(ids_d, E, 1, counts, offsets, pos_d, row_pair, status, [src_d], [dst_d])
    torch.cuda.synchronize()
    assert np.array_equal(pos_d.cpu().numpy(), pos)
    (ref,) = oracle.dispatch([src], pos, K, rows=cap, fill=0x5A)
    assert np.array_equal(dst_d.cpu().numpy(), ref)


# ------------------------------------------------------------- combine ---

@pytest.mark.parametrize("Hc", [1024, 1030])
def test_combine_far_rows(mg, Hc):
    """Expert rows, weights and output rows spread past 4 GiB (16-byte
    vectors at Hc = 1024, 4-byte words at Hc = 1030)."""
    N, K, E = 64, 8, 16
    rng, ids = routing(Hc, N, K, E)
    lay = mg.layout(dev(ids), E)
    torch.cuda.synchronize()
    pos = lay.pos.cpu().numpy()
    y = bits(rng.standard_normal((lay.cap, Hc)))
    w = rng.standard_normal((N, K)).astype(np.float32)
    y_d = far(lay.cap, Hc, torch.bfloat16, src=dev_bf16(y))
    w_d = far(N, K, torch.float32, src=dev(w))
    out = far(N, Hc, torch.bfloat16, fill=3.0)
    say(f"combine Hc={Hc}: y row stride {y_d.stride(0) * 2} B")
    mg.moe_combine(y_d, w_d, lay.pos, out)
    torch.cuda.synchronize()
    d = bf16_ulp_diff(host_bf16(out), oracle.combine(y, w, pos))
    say(f"  max ulp {int(d.max())}, nonzero {int((d != 0).sum())} of {d.size}")
    assert d.max() <= 1
    if Hc % 8:
        return

    say("combine epilogue with far biases, residual and outputs")
    res = bits(rng.standard_normal((N, Hc)) * 2)
    b0 = bits(rng.standard_normal((N, Hc)) * 0.5)
    gamma = bits(np.abs(rng.standard_normal(Hc)) + 0.5)
    res_d = far(N, Hc, torch.bfloat16, src=dev_bf16(res))
    b0_d = far(N, Hc, torch.bfloat16, src=dev_bf16(b0))
    res_out = far(N, Hc, torch.bfloat16, fill=5.0)
    mg.moe_combine_epilogue(y_d, w_d, lay.pos, out, bias0=b0_d, residual=res_d,
                            gamma=dev_bf16(gamma), eps=1e-6, residual_out=res_out)
    torch.cuda.synchronize()
    ref_out, ref_res = oracle.combine_epilogue(y, w, pos, b0, None, res, gamma, 1e-6)
    assert np.array_equal(host_bf16(res_out), ref_res)
    assert bf16_ulp_diff(host_bf16(out), ref_out).max() <= 1


# ------------------------------------------------------------ FP8 cast ---

def test_fp8_dispatch_far_rows(mg):
    """bf16 rows, e4m3 receive rows and row-major scales spread past 4 GiB;
    per-token scales through a far row stride; the one-launch padded form
    with far ids, rows and codes."""
    N, K, E, H = 64, 8, 16, 1024
    rng, ids = routing(9, N, K, E)
    lay = mg.layout(dev(ids), E)
    torch.cuda.synchronize()
    pos = lay.pos.cpu().numpy()
    cap = lay.cap
    x = bits(rng.standard_normal((N, H)) * np.exp(rng.standard_normal((N, 1)) * 2))
    x_d = far(N, H, torch.bfloat16, src=dev_bf16(x))
    dst = far(cap, H, torch.uint8, fill=0x11)
    sc = far(cap, H // 128, torch.float32, fill=0.0)
    say(f"fp8 rows: dst row stride {dst.stride(0)} B, scale row stride {sc.stride(0) * 4} B")
    mg.moe_dispatch_fp8(x_d, lay.pos, K, dst, sc, mg.MOE_SCALE_ROWS)
    torch.cuda.synchronize()
    codes, ref = oracle.dispatch_fp8(x, pos, cap, oracle.SCALE_ROWS, fill=0x11)
    assert np.array_equal(dst.cpu().numpy(), codes)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    del sc

    say("fp8 per-token scales")
    ts = far(N, H // 128, torch.float32, fill=0.0)
    mg.moe_dispatch_fp8(x_d, lay.pos, K, dst, ts, mg.MOE_SCALE_TOKENS)
    torch.cuda.synchronize()
    _, ref_t = oracle.dispatch_fp8(x, pos, cap, oracle.SCALE_TOKENS)
    assert np.array_equal(ts.cpu().numpy().view(np.uint32), ref_t.view(np.uint32))
    assert np.array_equal(dst.cpu().numpy(), codes)
    del dst, ts

    say("padded layout + FP8 dispatch in one launch")
    M = 48
    ids_d = far(N, K, torch.int32, src=dev(ids))
    dst = far(E * M, H, torch.uint8, fill=0x22)
    scales = torch.zeros((E, H // 128, M), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    pos_d = torch.empty((N, K), dtype=torch.int32, device="cuda")
    row_pair = torch.empty(E * M, dtype=torch.int32, device="cuda")
    status = torch.empty(2, dtype=torch.int32, device="cuda")
    mg.moe_dispatch_fp8_padded(ids_d, E, M, x_d, counts, pos_d, row_pair, status, dst, scales,
                               mg.MOE_SCALE_COLS)
    torch.cuda.synchronize()
    c, p, rp, st = oracle.layout_padded(ids, E, M)
    assert np.array_equal(pos_d.cpu().numpy(), p)
    assert np.array_equal(row_pair.cpu().numpy(), rp)
    assert tuple(status.cpu().tolist()) == st
    codes, ref = oracle.dispatch_fp8(x, p, E * M, oracle.SCALE_COLS, M, fill=0x22)
    assert np.array_equal(dst.cpu().numpy(), codes)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------ backward ---

def test_backward_far_rows(mg):
    """Both backward entry points with every row operand spread past 4 GiB."""
    N, K, E, H = 64, 8, 16, 1024
    rng, ids = routing(13, N, K, E)
    lay = mg.layout(dev(ids), E)
    torch.cuda.synchronize()
    pos = lay.pos.cpu().numpy()
    rows = lay.cap

    say("dispatch backward")
    gr = bits(rng.standard_normal((rows, H)))
    grw = rng.standard_normal((rows, K)).astype(np.float32)
    gr_d = far(rows, H, torch.bfloat16, src=dev_bf16(gr))
    grw_d = far(rows, K, torch.float32, src=dev(grw))
    gx = far(N, H, torch.bfloat16, fill=7.0)
    gw = far(N, K, torch.float32, fill=7.0)
    mg.moe_dispatch_backward(gr_d, lay.pos, gx, grw_d, gw)
    torch.cuda.synchronize()
    ref_x, ref_w = oracle.dispatch_backward(gr, pos, grw)
    assert np.array_equal(host_bf16(gx), ref_x)
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))
    del gr_d, grw_d, gx, gw

    say("combine backward")
    g = bits(rng.standard_normal((N, H)))
    w = rng.standard_normal((N, K)).astype(np.float32)
    y = bits(rng.standard_normal((rows, H)))
    g_d = far(N, H, torch.bfloat16, src=dev_bf16(g))
    w_d = far(N, K, torch.float32, src=dev(w))
    y_d = far(rows, H, torch.bfloat16, src=dev_bf16(y))
    gy = far(rows, H, torch.int16, fill=0x5555).view(torch.bfloat16)
    gw = far(N, K, torch.float32, fill=7.0)
    mg.moe_combine_backward(g_d, w_d, lay.pos, gy, y=y_d, grad_w=gw)
    torch.cuda.synchronize()
    ref_gy, ref_gw = oracle.combine_backward(g, w, pos, rows, y=y, fill=0x5555)
    assert np.array_equal(host_bf16(gy), ref_gy)
    got = gw.cpu().numpy().astype(np.float64)
    gf = np.abs(bf16_bits_to_float(g)).astype(np.float64)
    yf = np.abs(bf16_bits_to_float(y)).astype(np.float64)
    S = np.zeros((N, K))
    for k in range(K):
        ok = pos[:, k] >= 0
        S[ok, k] = (gf[ok] * yf[pos[ok, k]]).sum(1)
    tol = (8 + 22 + 1) * 2.0 ** -24 * S + 2.0 ** -24 * np.abs(ref_gw)
    assert (np.abs(got - ref_gw) <= tol).all()
    assert (got[pos < 0] == 0).all()
