"""moe_get_layout_noalloc, the layout entry point that allocates nothing (its
workspace is the library's static scratch on the GPU), against
moe_get_layout with a caller workspace: every output bit for bit, on calls in
a row where each later one is smaller than the one before, so a call that
read anything a previous call left in the scratch would show. Both batches
are above the one-launch size, so both run the two-kernel layout that uses
the scratch. Through the C ABI (ctypes binding)."""
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
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


def _outputs(N, K, E, cap):
    i32 = dict(dtype=torch.int32, device="cuda")
    return (torch.full((E,), -7, **i32), torch.full((E + 1,), -7, **i32),
            torch.full((N, K), -7, **i32), torch.full((cap,), -7, **i32),
            torch.full((1,), -7, **i32), torch.full((N * K,), -7, **i32))


def _cases():
    prefill = mw.make("prefill")
    rng = np.random.default_rng(99)
    N, K, E = 700, 8, 1000
    ids = mw.uniform_distinct_ids(rng, N, K, E)
    ids[rng.random((N, K)) < 0.1] = -1
    ids[rng.random((N, K)) < 0.02] = E + 3          # out of range: counted in status
    rng2 = np.random.default_rng(7)
    ids3 = rng2.integers(0, 16, size=(400, 6)).astype(np.int32)
    return [("prefill", prefill.ids, prefill.E, 1), ("N=700 E=1000 align 4", ids, E, 4),
            ("N=400 K=6 E=16", ids3, 16, 1)]


def test_noalloc_matches_workspace_layout(mg):
    for name, ids, E, align in _cases():
        N, K = ids.shape
        assert N * K > 2048   # the two-kernel layout, which uses the scratch
        cap = mg.moe_required_capacity(N, K, E, align) + 5
        say(f"{name}: N={N} K={K} E={E} align={align} cap={cap}")
        ids_d = torch.from_numpy(np.ascontiguousarray(ids)).cuda()
        a = _outputs(N, K, E, cap)
        b = _outputs(N, K, E, cap)
        mg.moe_get_layout_noalloc(ids_d, E, align, *a[:4], status=a[4], order=a[5])
        ws = torch.empty(mg.moe_layout_workspace_bytes(N, K, E), dtype=torch.uint8, device="cuda")
        mg.moe_get_layout(ids_d, E, align, *b[:4], ws, status=b[4], order=b[5])
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        c, o, p, rp, st = oracle.layout(ids, E, align, cap)
        got = [t.cpu().numpy() for t in a]
        for g, r in zip(got, (c, o, p, rp)):
            assert np.array_equal(g.reshape(r.shape), r)
        assert int(got[4][0]) == st
