"""The oracle's OpenMP loops run over tokens, and each token's work is
independent, so every output must be bit-identical whatever the thread count
(the CPU baseline times the oracle on all host cores). Each parallel oracle
function runs on 1 and on 4 threads on the same seeded inputs (CPU only)."""
import numpy as np
import pytest

import moe_workloads as mw


@pytest.fixture
def inputs(orc):
    rng = np.random.default_rng(77)
    N, K, E, H, Hc = 300, 8, 32, 1024, 512
    ids = rng.integers(-1, E + 1, size=(N, K)).astype(np.int32)
    _, _, pos, _, _ = orc.layout(ids, E)
    rows = N * K
    f32 = lambda *s: rng.standard_normal(s).astype(np.float32)
    return dict(
        N=N, K=K, E=E, H=H, Hc=Hc, ids=ids, pos=pos, rows=rows,
        src=rng.integers(0, 256, size=(N, 48), dtype=np.uint8),
        x=mw.bf16_bits_from_f32(f32(N, H) * np.exp(f32(N, 1))),
        y=mw.bf16_bits_from_f32(f32(rows, Hc)),
        w=f32(N, K),
        go=mw.bf16_bits_from_f32(f32(N, Hc)),
        gr=mw.bf16_bits_from_f32(f32(rows, H)),
        grw=f32(rows, K),
        res=mw.bf16_bits_from_f32(f32(N, Hc)),
        gamma=mw.bf16_bits_from_f32(f32(Hc)),
    )


def _runs(orc, fn):
    prev = orc.set_threads(1)
    try:
        one = fn()
        orc.set_threads(4)
        four = fn()
    finally:
        orc.set_threads(prev)
    return one, four


def _same(a, b):
    if isinstance(a, (tuple, list)):
        assert len(a) == len(b)
        for x, y in zip(a, b):
            _same(x, y)
    elif a is None:
        assert b is None
    else:
        assert a.dtype == b.dtype and a.shape == b.shape
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_dispatch(orc, inputs):
    d = inputs
    _same(*_runs(orc, lambda: orc.dispatch([d["src"]], d["pos"], d["K"])))


def test_combine_and_epilogue(orc, inputs):
    d = inputs
    _same(*_runs(orc, lambda: orc.combine(d["y"], d["w"], d["pos"])))
    _same(*_runs(orc, lambda: orc.combine_epilogue(d["y"], d["w"], d["pos"], residual=d["res"],
                                                   gamma=d["gamma"])))


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_dispatch_fp8(orc, inputs, mode):
    d = inputs
    E, M = d["E"], 90
    _, pos, _, _ = orc.layout_padded(d["ids"], E, M)
    _same(*_runs(orc, lambda: orc.dispatch_fp8(d["x"], pos, E * M, mode, M, mode == 2)))


def test_backward(orc, inputs):
    d = inputs
    _same(*_runs(orc, lambda: orc.dispatch_backward(d["gr"], d["pos"], d["grw"])))
    _same(*_runs(orc, lambda: orc.combine_backward(d["go"], d["w"], d["pos"], d["rows"],
                                                   y=d["y"][:, :d["Hc"]])))
