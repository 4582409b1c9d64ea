"""GPU parity of the backward entry points against the oracle.

Bar: dispatch backward (grad_x and the weight-gradient sums) and the combine
backward's grad_y bit-exact (the same fp32 operations in the same order);
the combine backward's grad_w, a length-Hc dot product whose order the
pages do not fix, within the bound its header states, derived from the
kernel's arithmetic: (8*ceil(Hc/8192) + 22) fp32 roundings along any path,
times sum_h |grad_out * y|, plus the oracle's own final rounding.
"""
import sys

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
from _util import bf16_bits_to_float

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_get_amd as m

    return m


def say(msg):
    print(f"[gpu-backward] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bits(a):
    return mw.bf16_bits_from_f32(np.asarray(a, np.float32))


def _pos(seed, N, K, E, mask):
    """Layout of random ids (the oracle's), so pairs land on distinct rows."""
    rng = np.random.default_rng(seed)
    ids = mw.uniform_distinct_ids(rng, N, K, E) if K <= E else rng.integers(0, E, (N, K)).astype(np.int32)
    ids[rng.random((N, K)) < mask] = -1
    _, _, pos, _, _ = oracle.layout(ids, E)
    return rng, pos


def grad_w_bound(g, y, pos):
    """sum_h |g[t,h] * y[pos[t,k],h]| per pair (float64), 0 for masked pairs."""
    gf = np.abs(bf16_bits_to_float(g)).astype(np.float64)
    yf = np.abs(bf16_bits_to_float(y)).astype(np.float64)
    N, K = pos.shape
    out = np.zeros((N, K))
    for k in range(K):
        ok = pos[:, k] >= 0
        out[ok, k] = (gf[ok] * yf[pos[ok, k]]).sum(1)
    return out


def check_grad_w(got, ref, S, Hc):
    depth = 8 * -(-Hc // 8192) + 22 + 1
    tol = depth * 2.0 ** -24 * S + 2.0 ** -24 * np.abs(ref)
    bad = np.abs(got.astype(np.float64) - ref) > tol
    assert not bad.any(), (got[bad][:5], ref[bad][:5], tol[bad][:5])


# ------------------------------------------------------------ dispatch ---

@pytest.mark.parametrize("seed,N,K,E,H,mask", [
    (1, 300, 8, 64, 7168, 0.1), (2, 64, 3, 16, 2, 0.3), (3, 129, 12, 40, 6, 0.2),
    (4, 50, 32, 32, 512, 0.0), (5, 17, 1, 4, 64, 0.5), (6, 40, 8, 8, 200, 1.0)])
def test_dispatch_backward_parity(mg, seed, N, K, E, H, mask):
    say(f"dispatch backward seed={seed} N={N} K={K} H={H}")
    rng, pos = _pos(seed, N, K, E, mask)
    rows = max(N * K, 1)
    gr = bits(rng.standard_normal((rows, H)) * np.exp(rng.standard_normal((rows, 1)) * 3))
    grw = (rng.standard_normal((rows, K)) * 10).astype(np.float32)
    ref_x, ref_w = oracle.dispatch_backward(gr, pos, grw)
    gx = torch.full((N, H), 7.0, dtype=torch.bfloat16, device="cuda")
    gw = torch.full((N, K), 7.0, dtype=torch.float32, device="cuda")
    mg.moe_dispatch_backward(dev_bf16(gr), dev(pos), gx, dev(grw), gw)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(gx), ref_x)
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))
    # without weight gradients
    gx2 = torch.empty((N, H), dtype=torch.bfloat16, device="cuda")
    mg.moe_dispatch_backward(dev_bf16(gr), dev(pos), gx2)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(gx2), ref_x)


def test_dispatch_backward_prefill_full(mg):
    wl = mw.make("prefill")
    say("dispatch backward prefill")
    _, _, pos, _, _ = oracle.layout(wl.ids, wl.E)
    rng = np.random.default_rng(77)
    rows = wl.N * wl.K
    gr = mw.make_y(rows, 7168, 78)
    grw = rng.standard_normal((rows, wl.K)).astype(np.float32)
    ref_x, ref_w = oracle.dispatch_backward(gr, pos, grw)
    gx = torch.empty((wl.N, 7168), dtype=torch.bfloat16, device="cuda")
    gw = torch.empty((wl.N, wl.K), dtype=torch.float32, device="cuda")
    mg.moe_dispatch_backward(dev_bf16(gr), dev(pos), gx, dev(grw), gw)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(gx), ref_x)
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))


def test_dispatch_backward_weights_only_and_strided(mg):
    rng, pos = _pos(8, 33, 4, 16, 0.2)
    rows = 33 * 4
    grw = (rng.standard_normal((rows, 6))).astype(np.float32)       # row stride 6 > K
    _, ref_w = oracle.dispatch_backward(np.zeros((rows, 0), np.uint16), pos, grw)
    gw = torch.zeros((33, 4), dtype=torch.float32, device="cuda")
    mg.moe_dispatch_backward(torch.empty((rows, 0), dtype=torch.bfloat16, device="cuda"), dev(pos),
                             torch.empty((33, 0), dtype=torch.bfloat16, device="cuda"), dev(grw), gw)
    torch.cuda.synchronize()
    assert np.array_equal(gw.cpu().numpy(), ref_w)
    # strided rows with untouched padding columns
    H = 64
    big = bits(rng.standard_normal((rows, H + 16)))
    ref_x, _ = oracle.dispatch_backward(big[:, :H], pos)
    out = torch.full((33, H + 8), 3.0, dtype=torch.bfloat16, device="cuda")
    mg.moe_dispatch_backward(dev_bf16(big)[:, :H], dev(pos), out[:, :H])
    torch.cuda.synchronize()
    o = host_bf16(out)
    assert np.array_equal(o[:, :H], ref_x) and (o[:, H:] == 0x4040).all()


# ------------------------------------------------------------- combine ---

@pytest.mark.parametrize("seed,N,K,E,Hc,mask", [
    (11, 300, 8, 64, 7168, 0.1), (12, 64, 3, 16, 8, 0.3), (13, 70, 12, 40, 8200, 0.2),
    (14, 20, 32, 32, 16384, 0.0), (15, 9, 1, 4, 32768, 0.5), (16, 40, 8, 8, 256, 1.0),
    (17, 33, 5, 9, 24, 0.1), (18, 50, 4, 12, 8192, 0.25), (19, 7, 16, 64, 64, 0.5)])
def test_combine_backward_parity(mg, seed, N, K, E, Hc, mask):
    say(f"combine backward seed={seed} N={N} K={K} Hc={Hc}")
    rng, pos = _pos(seed, N, K, E, mask)
    rows = N * K
    g = bits(rng.standard_normal((N, Hc)) * np.exp(rng.standard_normal((N, 1)) * 3))
    w = rng.standard_normal((N, K)).astype(np.float32)
    y = bits(rng.standard_normal((rows, Hc)))
    ref_gy, ref_gw = oracle.combine_backward(g, w, pos, rows, y=y, fill=0x5555)
    gy = torch.full((rows, Hc), 0, dtype=torch.int16, device="cuda")
    gy.fill_(0x5555)
    gy = gy.view(torch.bfloat16)
    gw = torch.full((N, K), 7.0, dtype=torch.float32, device="cuda")
    mg.moe_combine_backward(dev_bf16(g), dev(w), dev(pos), gy, y=dev_bf16(y), grad_w=gw)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(gy), ref_gy)
    got_w = gw.cpu().numpy()
    check_grad_w(got_w, ref_gw.astype(np.float64), grad_w_bound(g, y, pos), Hc)
    assert (got_w[pos < 0] == 0).all()
    # the same result on a second run, and grad_y alone without y
    gw2 = torch.empty((N, K), dtype=torch.float32, device="cuda")
    gy2 = torch.zeros((rows, Hc), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine_backward(dev_bf16(g), dev(w), dev(pos), gy2, y=dev_bf16(y), grad_w=gw2)
    gy3 = torch.zeros((rows, Hc), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine_backward(dev_bf16(g), dev(w), dev(pos), gy3)
    torch.cuda.synchronize()
    assert np.array_equal(gw2.cpu().numpy().view(np.uint32), got_w.view(np.uint32))
    landed = np.zeros(rows, bool)
    landed[pos[pos >= 0]] = True
    assert np.array_equal(host_bf16(gy3)[landed], ref_gy[landed])


def test_combine_backward_prefill_full(mg):
    wl = mw.make("prefill")
    say("combine backward prefill")
    _, _, pos, _, _ = oracle.layout(wl.ids, wl.E)
    rows = wl.N * wl.K
    g = mw.make_y(wl.N, 7168, 91)
    y = wl.y()
    w = np.ascontiguousarray(wl.weights)
    ref_gy, ref_gw = oracle.combine_backward(g, w, pos, rows, y=y)
    gy = torch.empty((rows, 7168), dtype=torch.bfloat16, device="cuda")
    gw = torch.empty((wl.N, wl.K), dtype=torch.float32, device="cuda")
    mg.moe_combine_backward(dev_bf16(g), dev(w), dev(pos), gy, y=dev_bf16(y), grad_w=gw)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(gy), ref_gy)                 # every row lands (no masks)
    check_grad_w(gw.cpu().numpy(), ref_gw.astype(np.float64), grad_w_bound(g, y, pos), 7168)


def test_combine_backward_zero_width(mg):
    """Hc = 0: no rows to write; every weight gradient is an empty sum."""
    rng, pos = _pos(21, 10, 4, 8, 0.2)
    gw = torch.full((10, 4), 3.0, dtype=torch.float32, device="cuda")
    e = lambda r: torch.empty((r, 0), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine_backward(e(10), dev(rng.standard_normal((10, 4)).astype(np.float32)), dev(pos),
                            e(40), y=e(40), grad_w=gw)
    torch.cuda.synchronize()
    assert (gw.cpu().numpy() == 0).all()


def test_backward_errors(mg):
    pos = torch.zeros((4, 2), dtype=torch.int32, device="cuda")
    g = torch.zeros((4, 60), dtype=torch.bfloat16, device="cuda")          # Hc % 8 != 0
    with pytest.raises(mg.MoeError):
        mg.moe_combine_backward(g, torch.zeros((4, 2), device="cuda"), pos,
                                torch.zeros((8, 60), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        mg.moe_dispatch_backward(torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda"), pos,
                                 torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda"),
                                 grad_recv_w=torch.zeros((8, 2), device="cuda"))


def test_graph_capture_lowlatency_and_backward(mg):
    """Padded layout -> FP8 dispatch -> combine -> combine backward ->
    dispatch backward captured once and replayed on new inputs (eager work
    and a synchronization between replays); every replay equals the eager
    calls on the same inputs."""
    N, K, E, H, M = 96, 4, 16, 512, 96
    rows = E * M
    ids_s = torch.zeros((N, K), dtype=torch.int32, device="cuda")
    x_s = torch.zeros((N, H), dtype=torch.bfloat16, device="cuda")
    w_s = torch.zeros((N, K), dtype=torch.float32, device="cuda")
    y_s = torch.zeros((rows, H), dtype=torch.bfloat16, device="cuda")
    g_s = torch.zeros((N, H), dtype=torch.bfloat16, device="cuda")
    gr_s = torch.zeros((rows, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(mg.moe_layout_workspace_bytes(N, K, E), 256), dtype=torch.uint8, device="cuda")

    def buffers():
        return dict(counts=torch.empty(E, dtype=torch.int32, device="cuda"),
                    pos=torch.empty((N, K), dtype=torch.int32, device="cuda"),
                    row_pair=torch.empty(rows, dtype=torch.int32, device="cuda"),
                    status=torch.empty(2, dtype=torch.int32, device="cuda"),
                    codes=torch.zeros((rows, H), dtype=torch.uint8, device="cuda"),
                    scales=torch.zeros((E, H // 128, M), dtype=torch.float32, device="cuda"),
                    out=torch.empty((N, H), dtype=torch.bfloat16, device="cuda"),
                    gy=torch.zeros((rows, H), dtype=torch.bfloat16, device="cuda"),
                    gw=torch.empty((N, K), dtype=torch.float32, device="cuda"),
                    gx=torch.empty((N, H), dtype=torch.bfloat16, device="cuda"))

    def step(b):
        mg.moe_get_layout_padded(ids_s, E, M, b["counts"], b["pos"], b["row_pair"], ws, b["status"])
        mg.moe_dispatch_fp8(x_s, b["pos"], K, b["codes"], b["scales"], mg.MOE_SCALE_COLS, M, False)
        mg.moe_combine(y_s, w_s, b["pos"], b["out"])
        mg.moe_combine_backward(g_s, w_s, b["pos"], b["gy"], y=y_s, grad_w=b["gw"])
        mg.moe_dispatch_backward(gr_s, b["pos"], b["gx"])

    gb = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(gb)                                          # warm up outside capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(gb)
    for rep in range(4):
        say(f"graph replay {rep}")
        rng = np.random.default_rng(300 + rep)
        ids = mw.uniform_distinct_ids(rng, N, K, E)
        ids[rng.random((N, K)) < 0.1] = -1
        ids_s.copy_(dev(ids))
        x_s.copy_(dev_bf16(bits(rng.standard_normal((N, H)) * 4)))
        w_s.copy_(dev(rng.standard_normal((N, K)).astype(np.float32)))
        y_s.copy_(dev_bf16(bits(rng.standard_normal((rows, H)))))
        g_s.copy_(dev_bf16(bits(rng.standard_normal((N, H)))))
        gr_s.copy_(dev_bf16(bits(rng.standard_normal((rows, H)))))
        for t in gb.values():                             # no stale rows or scale slots
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
