"""Pins of the oracle's combine (CPU only).

Definition (vLLM branch compare ds-exp-2...ds-exp-ag, moe_reduce_scatter.cu,
POLL + REDUCE: fp32 accumulation in a fixed order, one bf16 rounding at the
end; DeepEP deep_ep.cpp low_latency_combine: fp32 topk_weights weight the
expert outputs): acc = +0; for k ascending with pos >= 0,
acc = fmaf(w[t,k], y[pos[t,k], h], acc); out = bf16_rne(acc).

Pins: the bf16 conversions against torch's CPU conversion; the fp32 chain
against exact rational arithmetic rounded per step; exact special cases
(gathers, one-hot and power-of-two weights); a float64 reference within the
fp32 chain's a-priori error bound; identity experts; a hand-worked fixture.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import moe_workloads as mw
from _util import (bf16_bits_to_float, bf16_ulp_diff, f32_fraction, ints, read_cases,
                   round_bf16, round_f32, float_to_bf16_bits_exact)


def _torch_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _special_f32_values():
    rng = np.random.default_rng(0)
    bits = [rng.integers(0, 2**32, size=20000, dtype=np.uint64).astype(np.uint32)]
    # exact ties and near-ties around bf16 boundaries, both parities
    hi = rng.integers(0, 2**16, size=4000, dtype=np.uint32) << 16
    for low in (0x7FFF, 0x8000, 0x8001, 0x0000, 0x0001, 0xFFFF):
        bits.append(hi | low)
    # subnormals, zeros, max finite, infinities
    bits.append(np.array([0, 0x80000000, 1, 0x80000001, 0x007FFFFF, 0x00008000, 0x00018000,
                          0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x7F800000, 0xFF800000],
                         dtype=np.uint32))
    return np.concatenate(bits).view(np.float32)


def test_f32_to_bf16_matches_torch(orc):
    x = _special_f32_values()
    x = x[~np.isnan(x)]
    ours = np.array([orc.f32_to_bf16(float(v)) for v in x], np.uint16)
    assert np.array_equal(ours, _torch_bf16_bits(x))


def test_f32_to_bf16_nan_is_canonical(orc):
    for b in (0x7FC00000, 0x7F800001, 0xFFC00000, 0x7FFFFFFF):
        v = np.array([b], np.uint32).view(np.float32)[0]
        assert orc.f32_to_bf16(float(v)) == 0x7FC0


def test_bf16_to_f32_matches_torch(orc):
    bits = np.arange(0, 2**16, 7, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    ours = np.array([orc.bf16_to_f32(int(b)) for b in bits], np.float32)
    same = (ours.view(np.uint32) == ref.view(np.uint32)) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def _small_case(seed, N=6, K=8, Hc=24, R=None, mask_frac=0.2):
    rng = np.random.default_rng(seed)
    R = N * K if R is None else R
    y = mw.bf16_bits_from_f32(rng.standard_normal((R, Hc)).astype(np.float32) * 3)
    w = rng.standard_normal((N, K)).astype(np.float32)
    pos = rng.permutation(R)[: N * K].reshape(N, K).astype(np.int32)
    pos[rng.random((N, K)) < mask_frac] = -1
    return y, w, pos


@pytest.mark.parametrize("seed", range(6))
def test_fp32_chain_exact_rational(orc, seed):
    """The accumulator equals the rational chain rounded to fp32 after every
    fused step (k ascending) -- pins the order and the fusion."""
    y, w, pos = _small_case(seed)
    acc = orc.combine_acc(y, w, pos)
    yf = bf16_bits_to_float(y)
    N, K = pos.shape
    for t in range(N):
        for h in range(y.shape[1]):
            a = Fraction(0)
            for k in range(K):
                p = pos[t, k]
                if p < 0:
                    continue
                a = round_f32(f32_fraction(w[t, k]) * Fraction(float(yf[p, h])) + a)
            assert Fraction(float(acc[t, h])) == a, (t, h)


def test_fused_and_ordered_chain_is_observable(orc):
    """On these inputs both a mul-then-add chain and a descending-k chain give
    different fp32 accumulators, so the exact-rational pin above can tell
    them apart."""
    y, w, pos = _small_case(11, N=8, K=8, Hc=64, mask_frac=0.0)
    yf = bf16_bits_to_float(y).astype(np.float32)
    acc = orc.combine_acc(y, w, pos)
    unfused = np.zeros_like(acc)
    backwards = np.zeros_like(acc)
    for t in range(8):
        a = np.zeros(64, np.float32)
        b = np.zeros(64, np.float32)
        for k in range(8):
            a = (w[t, k] * yf[pos[t, k]]).astype(np.float32) + a
        for k in reversed(range(8)):
            b = np.float32(w[t, k]) * yf[pos[t, k]] + b
        unfused[t], backwards[t] = a, b
    assert (unfused != acc).any() and (backwards != acc).any()


@pytest.mark.parametrize("seed", range(4))
def test_final_rounding_exact_rational(orc, seed):
    y, w, pos = _small_case(20 + seed)
    acc = orc.combine_acc(y, w, pos)
    out = orc.combine(y, w, pos)
    for t in range(acc.shape[0]):
        for h in range(acc.shape[1]):
            r = round_bf16(Fraction(float(acc[t, h])))
            assert out[t, h] == float_to_bf16_bits_exact(r)


def test_hand_worked_fixture(orc):
    (c,) = read_cases("combine_hand.txt")
    N, K, Hc = int(c["N"][0]), int(c["K"][0]), int(c["Hc"][0])
    pos = ints(c["pos"]).astype(np.int32).reshape(N, K)
    w = np.array([float(v) for v in c["w"]], np.float32).reshape(N, K)
    y = _torch_bf16_bits(np.array([float(v) for v in c["y"]], np.float32)).reshape(-1, Hc)
    out = orc.combine(y, w, pos)
    assert out.reshape(-1).tolist() == ints(c["out"]).tolist()


def test_k1_unit_weight_is_gather(orc):
    rng = np.random.default_rng(1)
    y = rng.integers(0, 2**16, size=(40, 32), dtype=np.uint16)
    y = np.where(((y >> 7) & 0xFF) == 0xFF, y & 0x807F, y).astype(np.uint16)   # no inf/NaN
    pos = rng.permutation(40)[:25].reshape(25, 1).astype(np.int32)
    w = np.ones((25, 1), np.float32)
    out = orc.combine(y, w, pos)
    ref = y[pos[:, 0]]
    # -0 times +1 plus +0 is +0; everything else is reproduced bit for bit
    ref = np.where(ref == 0x8000, 0, ref)
    assert np.array_equal(out, ref)


def test_one_hot_weights_are_exact_gathers(orc):
    y, _, pos = _small_case(2, N=10, K=8, Hc=40, mask_frac=0.0)
    rng = np.random.default_rng(2)
    hot = rng.integers(0, 8, size=10)
    w = np.zeros((10, 8), np.float32)
    w[np.arange(10), hot] = 1.0
    out = orc.combine(y, w, pos)
    ref = y[pos[np.arange(10), hot]]
    assert np.array_equal(out, np.where(ref == 0x8000, 0, ref))


def test_power_of_two_weights_small_integers_exact(orc):
    """Small-integer y and power-of-two weights keep every partial sum exact,
    so the result is the exact sum rounded once to bf16."""
    rng = np.random.default_rng(3)
    N, K, Hc = 16, 8, 32
    yv = rng.integers(-16, 17, size=(N * K, Hc)).astype(np.float32)
    y = _torch_bf16_bits(yv)
    w = (2.0 ** rng.integers(-3, 4, size=(N, K))).astype(np.float32) * rng.choice([-1, 1], size=(N, K))
    w = w.astype(np.float32)
    pos = rng.permutation(N * K).reshape(N, K).astype(np.int32)
    out = orc.combine(y, w, pos)
    exact = (w[:, :, None].astype(np.float64) * yv[pos].astype(np.float64)).sum(axis=1)
    assert np.array_equal(out, _torch_bf16_bits(exact.astype(np.float32)))
    assert (np.abs(exact) < 2**23).all()


def _f64_reference(y, w, pos):
    """Exact-ish reference: each bf16 x fp32 product is exact in float64; the
    float64 sum of K of them is off by far less than the bounds used below.
    Also returns sum_k |w y|, the scale of the fp32 chain's error bound."""
    yf = bf16_bits_to_float(y).astype(np.float64)
    N, K = pos.shape
    acc = np.zeros((N, y.shape[1]), np.float64)
    mag = np.zeros_like(acc)
    for k in range(K):
        p = pos[:, k]
        ok = p >= 0
        term = w[ok, k].astype(np.float64)[:, None] * yf[p[ok]]
        acc[ok] += term
        mag[ok] += np.abs(term)
    return acc, mag


def assert_within_error_bound(orc, y, w, pos):
    """The fp32 chain of K fused steps is within K * 2^-24 * sum|w y| of the
    exact sum (each step rounds once, by at most 2^-24 of a partial sum that
    is at most sum|w y|). The bf16 result is then within one bf16 ulp of the
    exact sum rounded to bf16 wherever that bound is below a quarter of the
    bf16 spacing, and within bound + one bf16 spacing everywhere."""
    K = pos.shape[1]
    acc = orc.combine_acc(y, w, pos).astype(np.float64)
    out = orc.combine(y, w, pos)
    exact, mag = _f64_reference(y, w, pos)
    bound = K * 2.0**-24 * mag + 1e-300
    assert (np.abs(acc - exact) <= bound).all()
    outf = bf16_bits_to_float(out).astype(np.float64)
    spacing = np.abs(exact) * 2.0**-7 + 2.0**-133
    assert (np.abs(outf - exact) <= bound + spacing).all()
    tight = bound < spacing / 4
    d = bf16_ulp_diff(out, _torch_bf16_bits(exact.astype(np.float32)))
    assert d[tight].max(initial=0) <= 1
    return d


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_float64_reference_within_bound(orc, name):
    wl = mw.make(name)
    _, _, pos, _, _ = orc.layout(wl.ids, wl.E)
    d = assert_within_error_bound(orc, wl.y(), np.ascontiguousarray(wl.weights), pos)
    assert (d == 0).mean() > 0.99


def test_float64_reference_prefill_sampled_tokens(orc):
    """Prefill routing and softmax weights on 64 sampled tokens; only the
    expert-output rows those tokens use are drawn (renumbered compactly)."""
    wl = mw.make("prefill")
    _, _, pos, _, _ = orc.layout(wl.ids, wl.E)
    sample = np.random.default_rng(9).choice(wl.N, 64, replace=False)
    rows = pos[sample]
    y = mw.make_y(rows.size, wl.Hc, 91)
    compact = np.arange(rows.size, dtype=np.int32).reshape(rows.shape)
    assert_within_error_bound(orc, y, np.ascontiguousarray(wl.weights[sample]), compact)


@pytest.mark.parametrize("seed", range(4))
def test_float64_reference_signed_weights_masks(orc, seed):
    y, w, pos = _small_case(40 + seed, N=32, K=8, Hc=128, mask_frac=0.25)
    assert_within_error_bound(orc, y, w, pos)


def test_identity_experts(orc):
    """With y = dispatch(x) (bf16 payload), combine gives x * sum_k w within
    one ulp (the skewed workload's payload is bf16 hidden states)."""
    rng = np.random.default_rng(4)
    N, K, E, H = 64, 8, 16, 256
    x = mw.bf16_bits_from_f32(rng.standard_normal((N, H)).astype(np.float32))
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    w = np.abs(rng.standard_normal((N, K))).astype(np.float32)
    _, _, pos, _, _ = orc.layout(ids, E)
    (yb,) = orc.dispatch([x.view(np.uint8).reshape(N, -1)], pos, K)
    y = yb.view(np.uint16).reshape(N * K, H)
    out = orc.combine(y, w, pos)
    ref = bf16_bits_to_float(x).astype(np.float64) * w.astype(np.float64).sum(axis=1, keepdims=True)
    assert bf16_ulp_diff(out, _torch_bf16_bits(ref.astype(np.float32))).max() <= 1


def test_masked_and_all_masked_tokens(orc):
    y, w, pos = _small_case(5, N=4, K=4, Hc=16, mask_frac=0.0)
    pos[1, :] = -1
    pos[2, 1] = -1
    out = orc.combine(y, w, pos)
    assert (out[1] == 0).all()                       # +0.0, not -0.0
    keep = pos[2] >= 0
    assert_within_error_bound(orc, y, w, pos)
    assert keep.sum() == 3


def test_strided_weights_and_records(orc):
    wl = mw.make("large")
    sample = np.arange(0, wl.N, 997)
    ids = wl.ids[sample]
    _, _, pos, _, _ = orc.layout(np.ascontiguousarray(ids), wl.E)
    rng = np.random.default_rng(0)
    y = mw.bf16_bits_from_f32(rng.standard_normal((len(sample) * wl.K, 64)).astype(np.float32))
    a = orc.combine(y, wl.weights[sample], pos)                          # strided view
    b = orc.combine(y, np.ascontiguousarray(wl.weights[sample]), pos)
    assert np.array_equal(a, b)
