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


# --- every parallel oracle function at the prefill shape -------------------
# N = 4096 tokens, K = 8, E = 256, hidden 7168: the shape the GPU parity tests
# and the CPU baseline run the oracle on. Each function runs on one thread and
# on four and must give the same bytes. It runs in a child process started with
# OMP_NUM_THREADS=1, so that a crash in the oracle (a stack that grows per
# token, say) fails this test instead of ending the test run.

def _prefill_cases():
    import oracle

    rng = np.random.default_rng(2024)
    N, K, E, H = mw.CONFIGS["prefill"][0], 8, 256, 7168
    ids = mw.make("prefill").ids
    _, _, pos, _, _ = oracle.layout(ids, E)
    rows = N * K
    f32 = lambda *s: rng.standard_normal(s, dtype=np.float32)
    y = mw.bf16_bits_from_f32(f32(rows, H))
    w = f32(N, K)
    res = mw.bf16_bits_from_f32(f32(N, H))
    b0 = mw.bf16_bits_from_f32(f32(N, H))
    gamma = mw.bf16_bits_from_f32(f32(H))
    src = rng.integers(0, 256, size=(N, 7456), dtype=np.uint8)
    x = mw.bf16_bits_from_f32(f32(N, H) * np.exp(f32(N, 1)))
    grw = f32(rows, K)
    return [
        ("dispatch", lambda: oracle.dispatch([src], pos, K)),
        ("combine", lambda: oracle.combine(y, w, pos)),
        ("combine_epilogue", lambda: oracle.combine_epilogue(y, w, pos, bias0=b0, residual=res,
                                                             gamma=gamma)),
        ("dispatch_fp8", lambda: oracle.dispatch_fp8(x, pos, rows, 0, 1, False)),
        ("dispatch_backward", lambda: oracle.dispatch_backward(y, pos, grw)),
        ("combine_backward", lambda: oracle.combine_backward(res, w, pos, rows, y=y)),
    ]


def _prefill_main():
    import oracle

    for name, fn in _prefill_cases():
        one, four = _runs(oracle, fn)
        _same(one, four)
        print(name, "same on 1 and 4 threads", flush=True)


@pytest.mark.slow
def test_prefill_shape_one_thread():
    import os
    import subprocess
    import sys

    env = dict(os.environ, OMP_NUM_THREADS="1")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env["PYTHONPATH"] = root + os.pathsep + env.get("PYTHONPATH", "")
    p = subprocess.run([sys.executable, os.path.abspath(__file__)], env=env, cwd=root,
                       capture_output=True, text=True, timeout=600)
    assert p.returncode == 0, f"rc {p.returncode}\n{p.stdout}\n{p.stderr[-4000:]}"
    for name in ("dispatch", "combine", "combine_epilogue", "dispatch_fp8", "dispatch_backward",
                 "combine_backward"):
        assert f"{name} same on 1 and 4 threads" in p.stdout


if __name__ == "__main__":
    _prefill_main()
