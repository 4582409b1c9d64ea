"""GPU parity of moe_combine_epilogue against the oracle.

Bar: out without a residual (biases only) and residual_out bit-exact (the
same fp32 operations in the same order); the RMS-normalised out within one
bf16 ulp (the kernel's sum of squares is an fp32 tree sum and its scale a
hardware reciprocal square root; both sit far below a bf16 ulp, so only
elements next to a rounding boundary can move, by one).
"""
import sys

import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
from _util import bf16_ulp_diff

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_get_amd as m

    return m


def say(msg):
    print(f"[gpu-epilogue] {msg}", flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _inputs(seed, N, K, E, Hc, mask=0.1):
    rng = np.random.default_rng(seed)
    ids = mw.uniform_distinct_ids(rng, N, K, E) if K <= E else rng.integers(0, E, (N, K)).astype(np.int32)
    ids[rng.random((N, K)) < mask] = -1
    w = rng.standard_normal((N, K)).astype(np.float32)
    bits = lambda a: mw.bf16_bits_from_f32(a.astype(np.float32))
    y = bits(rng.standard_normal((N * K, Hc)))
    b0 = bits(rng.standard_normal((N, Hc)) * 0.5)
    b1 = bits(rng.standard_normal((N, Hc)) * 0.5)
    res = bits(rng.standard_normal((N, Hc)) * 2)
    gamma = bits(np.abs(rng.standard_normal(Hc)) + 0.5)
    return ids, w, y, b0, b1, res, gamma


@pytest.mark.parametrize("N,K,E,Hc", [(4096, 8, 256, 7168), (64, 8, 32, 8), (37, 3, 16, 64),
                                      (100, 8, 64, 2048), (100, 8, 64, 2056), (50, 4, 16, 4096),
                                      (30, 8, 64, 8192), (9, 2, 4, 16384), (0, 8, 16, 64),
                                      (40, 32, 64, 256), (33, 12, 40, 1024), (20, 32, 8, 64)])
def test_epilogue_parity(mg, N, K, E, Hc):
    say(f"N={N} K={K} E={E} Hc={Hc}")
    ids, w, y, b0, b1, res, gamma = _inputs(N * 7 + Hc, N, K, E, Hc)
    lay = mg.layout(dev(ids), E)
    torch.cuda.synchronize()
    pos = lay.pos.cpu().numpy()
    y_d, w_d = dev_bf16(y), dev(w)
    # biases only: bit-exact
    out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine_epilogue(y_d, w_d, lay.pos, out, bias0=dev_bf16(b0), bias1=dev_bf16(b1))
    ref, _ = oracle.combine_epilogue(y, w, pos, bias0=b0, bias1=b1)
    assert np.array_equal(host_bf16(out), ref)
    # one bias
    mg.moe_combine_epilogue(y_d, w_d, lay.pos, out, bias1=dev_bf16(b1))
    ref, _ = oracle.combine_epilogue(y, w, pos, bias1=b1)
    assert np.array_equal(host_bf16(out), ref)
    # residual + RMSNorm, with and without biases
    for with_bias in (False, True):
        res_out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
        kw = dict(bias0=dev_bf16(b0), bias1=dev_bf16(b1)) if with_bias else {}
        mg.moe_combine_epilogue(y_d, w_d, lay.pos, out, residual=dev_bf16(res), gamma=dev_bf16(gamma),
                                eps=1e-6, residual_out=res_out, **kw)
        ref_out, ref_res = oracle.combine_epilogue(y, w, pos, b0 if with_bias else None,
                                                   b1 if with_bias else None, res, gamma, 1e-6)
        assert np.array_equal(host_bf16(res_out), ref_res)
        d = bf16_ulp_diff(host_bf16(out), ref_out)
        say(f"  norm (bias={with_bias}): max ulp {int(d.max(initial=0))}, nonzero {int((d != 0).sum())} of {d.size}")
        assert d.max(initial=0) <= 1


def test_epilogue_strided_rows_and_untouched_padding(mg):
    N, K, E, Hc = 200, 4, 32, 512
    ids, w, y, b0, b1, res, gamma = _inputs(5, N, K, E, Hc)
    lay = mg.layout(dev(ids), E)
    torch.cuda.synchronize()
    pos = lay.pos.cpu().numpy()
    pad = lambda a: np.concatenate([a, np.zeros((a.shape[0], 16), np.uint16)], axis=1)
    res_d = dev_bf16(pad(res))[:, :Hc]
    b0_d = dev_bf16(pad(b0))[:, :Hc]
    out_full = torch.full((N, Hc + 8), 3.0, dtype=torch.bfloat16, device="cuda")
    ro_full = torch.full((N, Hc + 24), 5.0, dtype=torch.bfloat16, device="cuda")
    mg.moe_combine_epilogue(dev_bf16(y), dev(w), lay.pos, out_full[:, :Hc], bias0=b0_d, residual=res_d,
                            gamma=dev_bf16(gamma), eps=1e-5, residual_out=ro_full[:, :Hc])
    torch.cuda.synchronize()
    ref_out, ref_res = oracle.combine_epilogue(y, w, pos, b0, None, res, gamma, 1e-5)
    assert np.array_equal(host_bf16(ro_full[:, :Hc]), ref_res)
    assert bf16_ulp_diff(host_bf16(out_full[:, :Hc]), ref_out).max() <= 1
    assert (out_full[:, Hc:] == 3.0).all() and (ro_full[:, Hc:] == 5.0).all()


def test_epilogue_all_masked_is_rmsnorm_of_residual(mg):
    N, K, E, Hc = 16, 4, 8, 256
    ids = np.full((N, K), -1, np.int32)
    _, w, y, _, _, res, gamma = _inputs(6, N, K, E, Hc)
    lay = mg.layout(dev(ids), E)
    out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    ro = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine_epilogue(dev_bf16(y), dev(w), lay.pos, out, residual=dev_bf16(res),
                            gamma=dev_bf16(gamma), eps=1e-6, residual_out=ro)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16(ro), res)
    ref, _ = oracle.combine_epilogue(y, w, lay.pos.cpu().numpy(), None, None, res, gamma, 1e-6)
    assert bf16_ulp_diff(host_bf16(out), ref).max() <= 1


def test_epilogue_errors(mg):
    N, K, E, Hc = 8, 2, 4, 64
    ids, w, y, b0, b1, res, gamma = _inputs(7, N, K, E, Hc)
    lay = mg.layout(dev(ids), E)
    out = torch.empty((N, Hc), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mg.MoeError) as e:
        mg.moe_combine_epilogue(dev_bf16(y), dev(w), lay.pos, out, residual=dev_bf16(res))
    assert e.value.code == mg.MOE_ERR_ARG
