"""Pins of the oracle's combine epilogue (CPU only).

Definition: biases added in fp32 after the top-k sum (DeepEP deep_ep.cpp,
Buffer::intranode_combine takes bias_0 / bias_1 [num_recv_tokens, hidden];
their position is a reading of ours); with a residual, the fp32 sum plus
residual is stored (bf16) as the new residual and RMS-normalised with gamma
(vLLM branch compare ds-exp-2...ds-exp-ag, moe_rs_fused.cu, fused
POLL + REDUCE + RESIDUAL + RMSNORM phase).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import moe_workloads as mw
from _util import bf16_bits_to_float, bf16_ulp_diff, float_to_bf16_bits_exact, round_bf16


def _bits(x):
    return mw.bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def _case(seed, N=8, K=4, Hc=64, mask=0.2):
    rng = np.random.default_rng(seed)
    y = _bits(rng.standard_normal((N * K, Hc)))
    w = rng.standard_normal((N, K)).astype(np.float32)
    pos = rng.permutation(N * K).reshape(N, K).astype(np.int32)
    pos[rng.random((N, K)) < mask] = -1
    b0 = _bits(rng.standard_normal((N, Hc)))
    b1 = _bits(rng.standard_normal((N, Hc)))
    res = _bits(rng.standard_normal((N, Hc)) * 2)
    gamma = _bits(np.abs(rng.standard_normal(Hc)) + 0.5)
    return y, w, pos, b0, b1, res, gamma


def test_bf16_from_f64_exact_rational(orc):
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000))
    # exact ties between bf16 neighbours, both parities, and edge magnitudes
    for b in rng.integers(0, 0x7F7F, 300):
        lo = float(bf16_bits_to_float(np.array([b], np.uint16))[0])
        hi = float(bf16_bits_to_float(np.array([b + 1], np.uint16))[0])
        vals += [(lo + hi) / 2, -(lo + hi) / 2, np.nextafter((lo + hi) / 2, 0.0)]
    vals += [0.0, -0.0, 1e-45, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -134, 3.3895e38, 3.4e38, 1e300]
    for v in vals:
        r = round_bf16(Fraction(v))
        expect = (0x7F80 | (0x8000 if v < 0 else 0)) if r is None else (
            float_to_bf16_bits_exact(r) | (0x8000 if (v < 0 or (v == 0 and np.signbit(v))) else 0))
        got = orc.bf16_from_f64(float(v))
        if r is not None and r == 0:
            assert got & 0x7FFF == 0
        else:
            assert got == expect, (v, hex(got), hex(expect))


def test_biases_only_match_fp32_adds(orc):
    y, w, pos, b0, b1, _, _ = _case(1)
    out, res_out = orc.combine_epilogue(y, w, pos, bias0=b0, bias1=b1)
    assert res_out is None
    acc = orc.combine_acc(y, w, pos)
    ref = (acc + bf16_bits_to_float(b0)).astype(np.float32) + bf16_bits_to_float(b1)
    ref_bits = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref_bits)
    # without any epilogue term it is the plain combine
    out0, _ = orc.combine_epilogue(y, w, pos)
    assert np.array_equal(out0, orc.combine(y, w, pos))


def test_small_integer_sums_exact(orc):
    rng = np.random.default_rng(2)
    N, K, Hc = 6, 4, 32
    yv = rng.integers(-8, 9, size=(N * K, Hc)).astype(np.float32)
    w = (2.0 ** rng.integers(-2, 3, size=(N, K))).astype(np.float32)
    pos = rng.permutation(N * K).reshape(N, K).astype(np.int32)
    b0v = rng.integers(-8, 9, size=(N, Hc)).astype(np.float32)
    b1v = rng.integers(-8, 9, size=(N, Hc)).astype(np.float32)
    out, _ = orc.combine_epilogue(_bits(yv), w, pos, bias0=_bits(b0v), bias1=_bits(b1v))
    exact = (w[:, :, None].astype(np.float64) * yv[pos]).sum(axis=1) + b0v + b1v
    assert np.array_equal(out, _bits(exact))


@pytest.mark.parametrize("seed", range(4))
def test_rmsnorm_against_torch_float64(orc, seed):
    y, w, pos, b0, b1, res, gamma = _case(10 + seed, N=16, K=8, Hc=256)
    eps = 1e-6
    out, res_out = orc.combine_epilogue(y, w, pos, b0, b1, res, gamma, eps)
    acc = orc.combine_acc(y, w, pos)
    x = ((acc + bf16_bits_to_float(b0)).astype(np.float32) + bf16_bits_to_float(b1)).astype(np.float32)
    x = (x + bf16_bits_to_float(res)).astype(np.float32)
    # residual_out is the fp32 pre-norm value rounded once
    assert np.array_equal(res_out, _bits(x))
    g = torch.from_numpy(bf16_bits_to_float(gamma).astype(np.float64))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (x.shape[1],), g, eps)
    ref_bits = np.array([orc.bf16_from_f64(float(v)) for v in ref.numpy().reshape(-1)],
                        np.uint16).reshape(ref.shape)
    d = bf16_ulp_diff(out, ref_bits)
    # both sides are float64 up to the last rounding: exact but for the
    # rare element within a double's rounding of a bf16 tie
    assert d.max() <= 1 and (d == 0).mean() > 0.999


def test_rmsnorm_closed_forms(orc):
    N, K, Hc = 4, 2, 64
    y = np.zeros((N * K, Hc), np.uint16)
    w = np.zeros((N, K), np.float32)
    pos = np.full((N, K), -1, np.int32)                      # nothing routed: acc = residual
    a = np.array([3.0, 0.5, 96.0, 2.0 ** -20], np.float32)
    sign = np.where(np.arange(Hc) % 2 == 0, 1.0, -1.0).astype(np.float32)
    res = _bits(a[:, None] * sign[None, :])
    gamma = _bits(np.ones(Hc))
    out, res_out = orc.combine_epilogue(y, w, pos, residual=res, gamma=gamma, eps=0.0)
    assert np.array_equal(res_out, res)                      # masked pairs leave the residual
    assert np.array_equal(out, np.broadcast_to(_bits(sign), out.shape))   # +-a / |a| = +-1
    # scale invariance by a power of two (eps = 0)
    out4, _ = orc.combine_epilogue(y, w, pos, residual=_bits(4 * bf16_bits_to_float(res)), gamma=gamma, eps=0.0)
    assert np.array_equal(out4, out)
    # gamma multiplies elementwise
    g2 = _bits(np.full(Hc, 2.0))
    out2, _ = orc.combine_epilogue(y, w, pos, residual=res, gamma=g2, eps=0.0)
    assert np.array_equal(out2, _bits(2 * sign[None, :] * np.ones((N, 1))))
    # eps dominates a tiny residual: out ~ x / sqrt(eps)
    outs, _ = orc.combine_epilogue(y, w, pos, residual=res, gamma=gamma, eps=1.0)
    xs = bf16_bits_to_float(res).astype(np.float64)
    ref = xs / np.sqrt((xs ** 2).mean(axis=1, keepdims=True) + 1.0)
    assert bf16_ulp_diff(outs, np.array([orc.bf16_from_f64(v) for v in ref.reshape(-1)],
                                         np.uint16).reshape(ref.shape)).max() == 0


def test_errors(orc):
    y, w, pos, b0, b1, res, gamma = _case(3)
    with pytest.raises(orc.OracleError) as e:
        orc.combine_epilogue(y, w, pos, residual=res)         # a residual needs gamma
    assert e.value.code == orc.ERR_ARG
