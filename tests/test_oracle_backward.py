"""Pins of the oracle's backward (CPU only).

The pages (DeepEP repository dump, README, "Example use in model training")
define the backward of the dispatch as a combine of the received rows'
gradients, with the gradients of the received top-k weights combined
alongside, and the backward of the combine as a dispatch of the output
gradient. For the forward recv[pos[t,k]] = x[t], out[t] = sum_k w[t,k]
y[pos[t,k]] the oracle computes the chain rule's terms; these tests pin them
against a hand-worked fixture, exact rational arithmetic (the fp32 sums in k
order), torch float64 autograd of the forward, exact adjointness, and
special cases.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import moe_workloads as mw
from _util import (bf16_bits_to_float, f32_fraction, read_cases, round_bf16,
                   round_f32, float_to_bf16_bits_exact)


def _bits(a):
    return mw.bf16_bits_from_f32(np.asarray(a, np.float32))


def _case(N, K, H, rows, seed, mask=0.2):
    """Random pairs landing on distinct rows of a `rows`-row buffer."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(rows)[:N * K].astype(np.int32)
    pos = perm.reshape(N, K)
    pos[rng.random((N, K)) < mask] = -1
    return rng, pos


# ------------------------------------------------------------ fixture ---

def test_hand_worked_fixture(orc):
    (c,) = read_cases("backward_hand.txt")
    N, K, H, rows = (int(c[k][0]) for k in ("N", "K", "H", "rows"))
    pos = np.array([int(v) for v in c["pos"]], np.int32).reshape(N, K)
    grad_recv = _bits([float(v) for v in c["grad_recv"]]).reshape(rows, H)
    grad_recv_w = np.array([float(v) for v in c["grad_recv_w"]], np.float32).reshape(rows, K)
    gx, gw_in = orc.dispatch_backward(grad_recv, pos, grad_recv_w)
    assert gx.reshape(-1).tolist() == [int(v, 16) for v in c["grad_x"]]
    assert gw_in.reshape(-1).tolist() == [float(v) for v in c["grad_w_in"]]
    grad_out = _bits([float(v) for v in c["grad_out"]]).reshape(N, H)
    w = np.array([float(v) for v in c["w"]], np.float32).reshape(N, K)
    y = _bits([float(v) for v in c["y"]]).reshape(rows, H)
    gy, gw = orc.combine_backward(grad_out, w, pos, rows, y=y, fill=0xFFFF)
    assert gy.reshape(-1).tolist() == [int(v, 16) for v in c["grad_y"]]
    assert gw.reshape(-1).tolist() == [float(v) for v in c["grad_w"]]


# ------------------------------------------------- exact fp32 chains ---

@pytest.mark.parametrize("seed", range(4))
def test_sums_over_k_exact_rational(orc, seed):
    """grad_x before rounding and grad_w_in are fp32 sums with k ascending,
    each addition rounded: recomputed in exact rationals, rounded per step."""
    N, K, H, rows = 12, 6, 16, 80
    rng, pos = _case(N, K, H, rows, seed)
    g = _bits(rng.standard_normal((rows, H)) * np.exp(rng.standard_normal((rows, 1)) * 6))
    gw_rows = (rng.standard_normal((rows, K)) * np.exp(rng.standard_normal((rows, 1)) * 6)).astype(np.float32)
    gx, gw_in = orc.dispatch_backward(g, pos, gw_rows)
    gf = bf16_bits_to_float(g)
    for t in range(N):
        for h in range(H):
            a = Fraction(0)
            for k in range(K):
                if pos[t, k] >= 0:
                    a = round_f32(a + Fraction(float(gf[pos[t, k], h])))
            assert gx[t, h] == float_to_bf16_bits_exact(round_bf16(a)) or (a == 0 and gx[t, h] & 0x7FFF == 0)
        for j in range(K):
            a = Fraction(0)
            for k in range(K):
                if pos[t, k] >= 0:
                    a = round_f32(a + f32_fraction(gw_rows[pos[t, k], j]))
            assert Fraction(float(gw_in[t, j])) == a


def test_order_of_the_sum_is_observable(orc):
    """1 + 2^-24 + 2^-24 in k order stays 1 (two ties to even); the reverse
    order gives 1 + 2^-23: the fixture pins the order, not just the set."""
    pos = np.array([[0, 1, 2]], np.int32)
    rows = np.array([[1.0], [2.0 ** -24], [2.0 ** -24]], np.float32)
    _, gw_in = orc.dispatch_backward(np.zeros((3, 8), np.uint16), pos,
                                     np.repeat(rows, 3, axis=1))
    assert gw_in[0, 0] == 1.0
    _, rev = orc.dispatch_backward(np.zeros((3, 8), np.uint16), pos[:, ::-1].copy(),
                                   np.repeat(rows, 3, axis=1))
    assert rev[0, 0] == 1.0 + 2.0 ** -23


@pytest.mark.parametrize("seed", range(3))
def test_grad_y_is_one_fp32_product_rounded(orc, seed):
    N, K, H, rows = 20, 4, 32, 100
    rng, pos = _case(N, K, H, rows, seed)
    g = _bits(rng.standard_normal((N, H)) * 10)
    w = (rng.standard_normal((N, K))).astype(np.float32)
    gy, _ = orc.combine_backward(g, w, pos, rows, fill=0x1234)
    gf = bf16_bits_to_float(g)
    for t in range(N):
        for k in range(K):
            p = pos[t, k]
            if p < 0:
                continue
            for h in range(H):
                q = round_f32(f32_fraction(w[t, k]) * Fraction(float(gf[t, h])))
                assert gy[p, h] == float_to_bf16_bits_exact(round_bf16(q)) or (q == 0 and gy[p, h] & 0x7FFF == 0)
    untouched = np.ones(rows, bool)
    untouched[pos[pos >= 0]] = False
    assert (gy[untouched] == 0x1234).all()


# --------------------------------------------------- float64 autograd ---

@pytest.mark.parametrize("seed", range(3))
def test_against_float64_autograd(orc, seed):
    """The whole forward in torch float64 (gather to rows, weighted sum back),
    differentiated by autograd; the oracle's outputs are its terms rounded as
    the readings say."""
    N, K, H, rows = 24, 8, 64, 256
    rng, pos = _case(N, K, H, rows, seed)
    x = torch.randn(N, H, dtype=torch.float64, requires_grad=True)
    w_in = torch.randn(N, K, dtype=torch.float64, requires_grad=True)
    w = torch.tensor(rng.standard_normal((N, K)), requires_grad=True)
    y = torch.tensor(bf16_bits_to_float(_bits(rng.standard_normal((rows, H)))).astype(np.float64),
                     requires_grad=True)
    grad_recv = _bits(rng.standard_normal((rows, H)))
    grad_recv_w = rng.standard_normal((rows, K)).astype(np.float32)
    grad_out = _bits(rng.standard_normal((N, H)) * 3)
    valid = torch.tensor(pos >= 0)
    p = torch.tensor(np.where(pos >= 0, pos, 0), dtype=torch.long)
    # dispatch forward: rows[p] = x[t], with the token's weights alongside
    recv = torch.zeros(rows, H, dtype=torch.float64).index_put((p[valid],), x.repeat_interleave(K, 0)[valid.reshape(-1)])
    recv_w = torch.zeros(rows, K, dtype=torch.float64).index_put((p[valid],), w_in.repeat_interleave(K, 0)[valid.reshape(-1)])
    # combine forward
    out = (w.unsqueeze(-1) * y[p] * valid.unsqueeze(-1)).sum(1)
    f64 = lambda b: torch.tensor(bf16_bits_to_float(b).astype(np.float64))
    loss = (recv * f64(grad_recv)).sum() + (recv_w * torch.tensor(grad_recv_w, dtype=torch.float64)).sum() \
        + (out * f64(grad_out)).sum()
    loss.backward()

    gx, gw_in = orc.dispatch_backward(grad_recv, pos, grad_recv_w)
    gfl = np.abs(bf16_bits_to_float(grad_recv)).astype(np.float64)
    bound_x = np.array([[sum(gfl[pos[t, k], h] for k in range(K) if pos[t, k] >= 0) for h in range(H)] for t in range(N)])
    err = np.abs(bf16_bits_to_float(gx) - x.grad.numpy())
    assert (err <= K * 2.0 ** -24 * bound_x + np.abs(x.grad.numpy()) * 2.0 ** -8 + 1e-300).all()
    bound_w = np.array([[sum(abs(float(grad_recv_w[pos[t, k], j])) for k in range(K) if pos[t, k] >= 0) for j in range(K)] for t in range(N)])
    assert (np.abs(gw_in - w_in.grad.numpy()) <= K * 2.0 ** -24 * bound_w).all()

    yb = _bits(y.detach().numpy())
    gy, gw = orc.combine_backward(grad_out, w.detach().numpy().astype(np.float32), pos, rows, y=yb)
    # autograd used float64 w; the oracle's fp32 w differs by <= 2^-24 relative
    ref_gy = y.grad.numpy()
    landed = np.zeros(rows, bool)
    landed[pos[pos >= 0]] = True
    got = bf16_bits_to_float(gy[landed]).astype(np.float64)
    assert (np.abs(got - ref_gy[landed]) <= np.abs(ref_gy[landed]) * (2.0 ** -8 + 2.0 ** -23)).all()
    ref_gw = w.grad.numpy()
    gdot = np.abs(bf16_bits_to_float(grad_out)).astype(np.float64)
    mag = np.array([[float(gdot[t] @ np.abs(bf16_bits_to_float(yb[pos[t, k]]))) if pos[t, k] >= 0 else 0.0
                     for k in range(K)] for t in range(N)])
    assert (np.abs(gw - ref_gw) <= np.abs(ref_gw) * 2.0 ** -24 + mag * 2.0 ** -40).all()
    assert (gw[pos < 0] == 0).all()


# ------------------------------------------------------- adjointness ---

def test_adjointness_exact(orc):
    """<combine(y), g> = <y, combine_backward(g)> and <dispatch(x), r> =
    <x, dispatch_backward(r)>, exactly, on small integers and power-of-two
    weights (every sum and product exact in fp32 and bf16)."""
    rng = np.random.default_rng(9)
    N, K, H, rows = 30, 4, 24, 150
    _, pos = _case(N, K, H, rows, 9)
    # |sum of K=4 terms| <= 8 in steps of 1/2: at most 5 significant bits
    y = _bits(rng.integers(-2, 3, (rows, H)))
    g = _bits(rng.integers(-8, 9, (N, H)))
    w = (2.0 ** rng.integers(-1, 1, (N, K)) * rng.choice([-1, 1], (N, K))).astype(np.float32)
    out = orc.combine(y, w, pos)
    gy, _ = orc.combine_backward(g, w, pos, rows)
    lhs = float((bf16_bits_to_float(out).astype(np.float64) * bf16_bits_to_float(g)).sum())
    landed = np.zeros(rows, bool)
    landed[pos[pos >= 0]] = True
    rhs = float((bf16_bits_to_float(y[landed]).astype(np.float64) * bf16_bits_to_float(gy[landed])).sum())
    assert lhs == rhs
    x = rng.integers(0, 256, (N, 2 * H), dtype=np.uint8)
    xb = x.view(np.uint16) & 0x80FF | 0x4000            # small-magnitude bf16 codes
    (recv,) = orc.dispatch([xb.view(np.uint8)], pos, K, rows=rows)
    r = _bits(rng.integers(-4, 5, (rows, H)))
    gx, _ = orc.dispatch_backward(r, pos)
    recv_f = bf16_bits_to_float(recv.view(np.uint16))
    lhs = float((recv_f[landed].astype(np.float64) * bf16_bits_to_float(r[landed])).sum())
    rhs = float((bf16_bits_to_float(xb).astype(np.float64) * bf16_bits_to_float(gx)).sum())
    assert lhs == rhs


# ----------------------------------------------------- special cases ---

def test_k1_identity_and_all_masked(orc):
    rng = np.random.default_rng(4)
    N, H = 10, 40
    r = _bits(rng.standard_normal((N, H)))
    pos = np.arange(N, dtype=np.int32).reshape(N, 1)
    gx, _ = orc.dispatch_backward(r, pos)
    assert np.array_equal(gx, r)                        # one copy: the row itself
    gy, gw = orc.combine_backward(r, np.ones((N, 1), np.float32), pos, N, y=r)
    assert np.array_equal(gy, r)                        # unit weight: the gradient itself
    ref = (bf16_bits_to_float(r).astype(np.float64) ** 2).sum(1)
    assert np.allclose(gw[:, 0], ref, rtol=2.0 ** -23, atol=0)
    masked = np.full((N, 3), -1, np.int32)
    gx, gw_in = orc.dispatch_backward(r, masked, np.ones((N, 3), np.float32))
    assert (gx == 0).all() and (gw_in == 0).all()
    gy, gw = orc.combine_backward(r, np.ones((N, 3), np.float32), masked, 5, y=r, fill=7)
    assert (gy == 7).all() and (gw == 0).all()


def test_strided_rows(orc):
    rng = np.random.default_rng(5)
    N, K, H, rows = 8, 2, 16, 20
    _, pos = _case(N, K, H, rows, 5, mask=0)
    big = _bits(rng.standard_normal((rows, H + 8)))
    gx_s, _ = orc.dispatch_backward(big[:, :H], pos)
    gx_c, _ = orc.dispatch_backward(np.ascontiguousarray(big[:, :H]), pos)
    assert np.array_equal(gx_s, gx_c)
