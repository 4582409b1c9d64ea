"""Jobs larger than one launch.

A launch holds fewer than 2^32 work-items, so the kernels whose grid grows
with the batch run in pieces of at most 2^31 work-items on the same stream:
2^25 waves for the 256-thread kernels (dispatch, combine, dispatch backward,
FP8 dispatch) and 2^21 tokens for the 1024-thread ones (combine epilogue,
combine backward). Each case here is a few items past one piece, so the last
piece holds the ragged tail, and is compared with the oracle: everything
for the byte and sum kernels, and for the FP8 cast (2^25 tokens, where the
oracle would take minutes) the rows on both sides of the piece boundary and
a random sample of the rest, each of which depends on its own token only.
"""
import math
import sys

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
from _util import bf16_bits_to_float, bf16_ulp_diff

pytestmark = pytest.mark.gpu

WAVES_PER_PIECE = (1 << 31) // 64          # 256-thread kernels: 2^23 workgroups of 4 waves
TOKENS_PER_PIECE = (1 << 31) // 1024       # 1024-thread kernels: one workgroup per token


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
    print(f"[launch-pieces] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def scattered_pos(rng, N, K, mask=0.1):
    """An injective pos [N, K] onto the rows 0 .. N*K-1 (a multiplicative
    permutation, so consecutive pairs land far apart), ~mask of it -1."""
    R = N * K
    A = 2654435761 % R
    while math.gcd(A, R) != 1:
        A += 1
    pos = ((np.arange(R, dtype=np.int64) * A) % R).astype(np.int32).reshape(N, K)
    pos[rng.random((N, K)) < mask] = -1
    return pos


def test_dispatch_in_pieces(mg):
    """16-byte rows, one wave per pair: 2^25 + 24 pairs, two launches."""
    K = 8
    N = WAVES_PER_PIECE // K + 3
    rng = np.random.default_rng(1)
    pos = scattered_pos(rng, N, K)
    src = rng.integers(0, 256, size=(N, 16), dtype=np.uint8)
    say(f"dispatch N={N} K={K}: {N * K} waves")
    dst = torch.full((N * K, 16), 0xC3, dtype=torch.uint8, device="cuda")
    mg.moe_dispatch([dev(src)], [dst], dev(pos), K)
    torch.cuda.synchronize()
    (ref,) = oracle.dispatch([src], pos, K, rows=N * K, fill=0xC3)
    assert np.array_equal(dst.cpu().numpy(), ref)


@pytest.mark.parametrize("backward", [False, True])
def test_combine_in_pieces(mg, backward):
    """One wave per token at Hc = 8: 2^25 + 3 tokens, two launches; the
    dispatch backward runs the same kernel (unit weights, row sums)."""
    K, Hc = 2, 8
    N = WAVES_PER_PIECE + 3
    rng = np.random.default_rng(2)
    pos = scattered_pos(rng, N, K)
    y = mw.bf16_bits_from_f32(rng.standard_normal((N * K, Hc)).astype(np.float32))
    out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    if not backward:
        w = rng.standard_normal((N, K)).astype(np.float32)
        say(f"combine N={N} K={K} Hc={Hc}")
        mg.moe_combine(dev_bf16(y), dev(w), dev(pos), out)
        torch.cuda.synchronize()
        d = bf16_ulp_diff(host_bf16(out), oracle.combine(y, w, pos))
        assert d.max() <= 1
        return
    grw = rng.standard_normal((N * K, K)).astype(np.float32)
    gw = torch.empty((N, K), dtype=torch.float32, device="cuda")
    say(f"dispatch backward N={N} K={K} H={Hc}")
    mg.moe_dispatch_backward(dev_bf16(y), dev(pos), out, dev(grw), gw)
    torch.cuda.synchronize()
    ref_x, ref_w = oracle.dispatch_backward(y, pos, grw)
    assert np.array_equal(host_bf16(out), ref_x)
    assert np.array_equal(gw.cpu().numpy().view(np.uint32), ref_w.view(np.uint32))


def test_epilogue_and_combine_backward_in_pieces(mg):
    """One 1024-thread workgroup per token: 2^21 + 3 tokens, two launches."""
    K, Hc = 2, 8
    N = TOKENS_PER_PIECE + 3
    rng = np.random.default_rng(3)
    pos = scattered_pos(rng, N, K)
    bits = lambda a: mw.bf16_bits_from_f32(a.astype(np.float32))
    y = bits(rng.standard_normal((N * K, Hc)))
    w = rng.standard_normal((N, K)).astype(np.float32)
    res = bits(rng.standard_normal((N, Hc)))
    gamma = bits(np.abs(rng.standard_normal(Hc)) + 0.5)
    say(f"combine epilogue N={N}")
    out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    res_out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine_epilogue(dev_bf16(y), dev(w), dev(pos), out, residual=dev_bf16(res),
                            gamma=dev_bf16(gamma), eps=1e-6, residual_out=res_out)
    torch.cuda.synchronize()
    ref_out, ref_res = oracle.combine_epilogue(y, w, pos, None, None, res, gamma, 1e-6)
    assert np.array_equal(host_bf16(res_out), ref_res)
    assert bf16_ulp_diff(host_bf16(out), ref_out).max() <= 1
    del out, res_out

    say(f"combine backward N={N}")
    g = bits(rng.standard_normal((N, Hc)))
    gy = torch.full((N * K, Hc), 0, dtype=torch.int16, device="cuda")
    gy.fill_(0x5555)
    gy = gy.view(torch.bfloat16)
    gw = torch.empty((N, K), dtype=torch.float32, device="cuda")
    mg.moe_combine_backward(dev_bf16(g), dev(w), dev(pos), gy, y=dev_bf16(y), grad_w=gw)
    torch.cuda.synchronize()
    ref_gy, ref_gw = oracle.combine_backward(g, w, pos, N * K, y=y, fill=0x5555)
    assert np.array_equal(host_bf16(gy), ref_gy)
    # the weight gradients within the bound of the kernel's fp32 sum tree
    got = gw.cpu().numpy().astype(np.float64)
    S = np.zeros((N, K))
    gf = np.abs(bf16_bits_to_float(g)).astype(np.float64)
    yf = np.abs(bf16_bits_to_float(y)).astype(np.float64)
    for k in range(K):
        ok = pos[:, k] >= 0
        S[ok, k] = (gf[ok] * yf[pos[ok, k]]).sum(1)
    tol = (8 + 22 + 1) * 2.0 ** -24 * S + 2.0 ** -24 * np.abs(ref_gw)
    assert (np.abs(got - ref_gw) <= tol).all()


def test_fp8_dispatch_in_pieces(mg):
    """One wave per token at H = 128: 2^25 + 3 tokens, two launches. Every
    row's codes and scale against the oracle, in chunks of 2^22 rows (the
    second launch's 3 rows in the last chunk)."""
    H = 128
    N = WAVES_PER_PIECE + 3
    g = torch.Generator(device="cuda")
    g.manual_seed(4)
    say(f"fp8 dispatch N={N} H={H}")
    x = (torch.randn((N, H), device="cuda", generator=g) *
         torch.exp2(torch.randn((N, 1), device="cuda", generator=g) * 4)).to(torch.bfloat16)
    dst = torch.empty((N, H), dtype=torch.uint8, device="cuda")
    sc = torch.empty((N, 1), dtype=torch.float32, device="cuda")
    mg.moe_dispatch_fp8(x, None, 1, dst, sc, mg.MOE_SCALE_ROWS)
    torch.cuda.synchronize()
    step = 1 << 22
    for s in range(0, N, step):
        e = min(s + step, N)
        say(f"fp8 dispatch: rows {s} .. {e - 1} against the oracle")
        xs = x[s:e].view(torch.int16).cpu().numpy().view(np.uint16)
        ident = np.arange(e - s, dtype=np.int32).reshape(-1, 1)
        codes, scales = oracle.dispatch_fp8(xs, ident, e - s, oracle.SCALE_ROWS)
        assert np.array_equal(dst[s:e].cpu().numpy(), codes), (s, e)
        assert np.array_equal(sc[s:e].cpu().numpy().view(np.uint32), scales.view(np.uint32))
        del xs, codes, scales
