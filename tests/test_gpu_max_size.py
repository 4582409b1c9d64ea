"""The largest batch the ABI accepts: N*K = 2^31 - 8 pairs (N = 2^28 - 1,
K = 8, E = 256), one pair short of the N*K < 2^31 limit.

At this size the oracle would take minutes, so the layouts are checked
against properties that determine them completely, computed with torch on
the GPU in chunks:
  * counts = the histogram of the valid ids, offsets its exclusive scan,
    status the number of ids >= E;
  * every valid pair's row lies in its expert's segment and row_pair maps
    it back (so pos is a bijection onto the used rows), masked pairs get -1,
    unused rows -1;
  * inside a segment row_pair increases (the stable order), and in the
    padded form every dropped pair comes after its expert's last kept one.
A stable counting sort is the only layout with all of these. The layout's
dispatch plan must list every valid pair once (each used row hit once). The
dispatch (in the plan's order) and the combine then run on that layout with
16-byte rows: every received
row equals its token's row (compared on the host), and with small-integer
payloads and power-of-two weights every step of the combine is exact, so its
output equals bf16(x * sum of the token's valid weights).
"""
import sys
import time

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

N, K, E = (1 << 28) - 1, 8, 256
NK = N * K
CHUNK = 1 << 27


@pytest.fixture(scope="module")
def mg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_get_amd as m

    return m


_T0 = time.monotonic()


def say(msg):
    print(f"[max-size {time.monotonic() - _T0:6.1f}s] {msg}", flush=True)
    sys.stdout.flush()


def chunks(n):
    for s in range(0, n, CHUNK):
        yield s, min(s + CHUNK, n)


def histogram(flat, E):
    """(valid pairs per expert, ids >= E) of the flat ids."""
    hist = torch.zeros(E, dtype=torch.int64, device=flat.device)
    nbad = 0
    for s, e in chunks(flat.numel()):
        x = flat[s:e]
        v = (x >= 0) & (x < E)
        hist += torch.bincount(x[v].long(), minlength=E)
        nbad += int((x >= E).sum())
    return hist, nbad


def check_layout(flat, E, hist, nbad, counts, offsets, pos, rp, status):
    """The stable layout's defining properties (any index is range-checked
    before it is used to gather)."""
    nk, dev = flat.numel(), flat.device
    assert int(status) == nbad
    assert torch.equal(counts.long(), hist)
    off = offsets.long()
    assert int(off[0]) == 0 and torch.equal(off[1:], torch.cumsum(hist, 0))
    R = int(off[E])
    for s, e in chunks(nk):
        x = flat[s:e].long()
        p = pos[s:e].long()
        v = (x >= 0) & (x < E)
        assert (p[~v] == -1).all()
        xv, pv = x[v], p[v]
        assert ((pv >= off[xv]) & (pv < off[xv + 1])).all()       # inside its segment
        assert torch.equal(rp[pv].long(), torch.arange(s, e, device=dev)[v])   # inverse
    assert (rp[R:] == -1).all()
    for s, e in chunks(R - 1):
        a, b = rp[s:e].long(), rp[s + 1:e + 1].long()
        assert ((a >= 0) & (a < nk) & (b >= 0) & (b < nk)).all()
        same = flat[a] == flat[b]
        assert (a[same] < b[same]).all()                           # stable inside a segment
    return R


def check_plan(order, pos, R):
    """The dispatch plan: every valid pair once (each of the R used rows is
    hit by exactly one entry), -1 in the other NK - R entries."""
    hits = torch.zeros(R, dtype=torch.int32, device=order.device)
    nskip = 0
    for s, e in chunks(order.numel()):
        o = order[s:e].long()
        v = o >= 0
        assert (o[~v] == -1).all()
        ov = o[v]
        assert ((ov >= 0) & (ov < NK)).all()
        rows = pos[ov].long()
        assert ((rows >= 0) & (rows < R)).all()
        hits.index_add_(0, rows, torch.ones_like(rows, dtype=torch.int32))
        nskip += int((~v).sum())
    assert bool((hits == 1).all()) and nskip == order.numel() - R


def check_padded(flat, E, M, hist, nbad, counts, pos, rp, status):
    """The padded layout's defining properties; every expert must overflow
    its M rows (so each has a last kept pair to compare the dropped with)."""
    nk, dev = flat.numel(), flat.device
    kept = torch.clamp(hist, max=M)
    assert torch.equal(counts.long(), kept)
    assert int(status[0]) == nbad
    assert int(status[1]) == int((hist - kept).sum()) > 0
    assert bool((hist >= M).all())
    last = rp.view(E, M)[:, M - 1].long()                          # last kept pair
    assert ((last >= 0) & (last < nk)).all()
    nkept = 0
    for s, e in chunks(nk):
        x = flat[s:e].long()
        p = pos[s:e].long()
        v = (x >= 0) & (x < E)
        assert (p[~v] == -1).all()
        i = torch.arange(s, e, device=dev)
        k = v & (p >= 0)
        xk, pk = x[k], p[k]
        assert ((pk >= xk * M) & (pk < xk * M + kept[xk])).all()
        assert torch.equal(rp[pk].long(), i[k])
        d = v & (p < 0)
        assert (i[d] > last[x[d]]).all()                           # dropped after the kept
        nkept += int(k.sum())
    assert nkept == int(kept.sum())
    r = torch.arange(E * M, device=dev)
    used = (r % M) < kept[r // M]
    assert (rp[~used] == -1).all()
    a, b = rp[:-1].long(), rp[1:].long()
    inner = used[:-1] & used[1:] & ((r[:-1] % M) != M - 1)        # same expert's rows
    assert (a[inner] < b[inner]).all()                             # stable inside a segment


@pytest.fixture(scope="module")
def routed(mg):
    say(f"drawing {NK} ids (N={N}, K={K}, E={E}; -1 masked, {E} out of range)")
    g = torch.Generator(device="cuda")
    g.manual_seed(20261202)
    ids = torch.randint(-1, E + 1, (N, K), dtype=torch.int32, device="cuda", generator=g)
    hist, nbad = histogram(ids.view(-1), E)
    assert nbad > 0
    yield ids, hist, nbad
    del ids
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_layout_dispatch_combine_at_the_pair_limit(mg, routed):
    ids, hist, nbad = routed
    say("layout")
    lay = mg.layout(ids, E)
    torch.cuda.synchronize()
    assert lay.cap == NK
    say("layout: checking")
    check_layout(ids.view(-1), E, hist, nbad, lay.counts, lay.offsets, lay.pos.view(-1),
                 lay.row_pair, lay.status[0])

    say("layout: checking the dispatch plan")
    check_plan(lay.order, lay.pos.view(-1), int(lay.offsets[E]))
    torch.cuda.empty_cache()

    say("dispatch of 16-byte rows in the plan's order")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x = torch.randint(-16, 17, (N, 8), dtype=torch.int16, device="cuda",
                      generator=g).to(torch.bfloat16)
    y = torch.empty((NK, 8), dtype=torch.bfloat16, device="cuda")
    mg.moe_dispatch([x], [y], lay.pos, K, order=lay.order)
    torch.cuda.synchronize()
    # Used row r holds the row of token row_pair[r] / K (row_pair inverts
    # pos, checked above). Compared on the host for the first, a middle and
    # the last 2^27 rows (their pairs come from every launch piece): torch's
    # row gather (y[index] on a [2^31, 8] int16 tensor) returned wrong rows
    # at this size. Then every used row, on the GPU (below). The combine
    # reads every received row too.
    say("dispatch: checking on the host")
    R = int(lay.offsets[E])
    x_h = x.view(torch.int16).cpu().numpy()
    for s in (0, (R // 2) // CHUNK * CHUNK, max(R - CHUNK, 0)):
        e = min(s + CHUNK, R)
        t = lay.row_pair[s:e].cpu().numpy() // K
        assert np.array_equal(y[s:e].view(torch.int16).cpu().numpy(), x_h[t])
    del x_h
    # Every used row, on the GPU, 2^22 rows at a time: the 16-byte rows as
    # pairs of int64 gathered from the [2^28, 2] source (and the gather agrees
    # with the host on the three ranges above).
    say("dispatch: checking every used row on the GPU")
    x64 = x.view(torch.int64)
    y64 = y.view(torch.int64)
    step = 1 << 22
    for s in range(0, R, step):
        e = min(s + step, R)
        t = lay.row_pair[s:e].long() // K
        assert torch.equal(y64[s:e], x64.index_select(0, t)), (s, e)
        if s % CHUNK == 0:
            say(f"dispatch: rows below {e} agree")
    del x64, y64, t

    say("combine of the received rows")
    w = torch.randint(-2, 2, (N, K), dtype=torch.int32, device="cuda", generator=g)
    sign = torch.randint(0, 2, (N, K), dtype=torch.int32, device="cuda", generator=g) * 2 - 1
    w = torch.exp2(w.float()) * sign.float()         # +-1/4 .. +-2
    out = torch.empty((N, 8), dtype=torch.bfloat16, device="cuda")
    mg.moe_combine(y, w, lay.pos, out)
    torch.cuda.synchronize()
    del y
    wsum = (w * (lay.pos >= 0)).sum(1)               # exact: quarters, |sum| <= 16
    ref = (x.float() * wsum[:, None]).to(torch.bfloat16)
    assert torch.equal(out.float(), ref.float())     # +0 == -0


@pytest.mark.timeout(600)
def test_padded_layout_at_the_pair_limit(mg, routed):
    ids, hist, nbad = routed
    M = 1 << 21                       # far below the ~8.3M pairs per expert: most drop
    say(f"padded layout, M={M}")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    pos = torch.empty((N, K), dtype=torch.int32, device="cuda")
    rp = torch.empty(E * M, dtype=torch.int32, device="cuda")
    status = torch.empty(2, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(mg.moe_layout_workspace_bytes(N, K, E), 256), dtype=torch.uint8,
                     device="cuda")
    mg.moe_get_layout_padded(ids, E, M, counts, pos, rp, ws, status)
    torch.cuda.synchronize()
    say("padded layout: checking")
    check_padded(ids.view(-1), E, M, hist, nbad, counts, pos.view(-1), rp, status)


def check_sparse_padded(ids, E, M, counts, pos, rp, status, nbad):
    """A padded layout over E*M rows of which only a few are used (no
    drops), checked row by row over all E*M rows in chunks with elementwise
    operations and gathers from the small per-pair tensors only: every used
    row r (r % M < counts[r / M]) names a valid pair i = rp[r] with
    pos[i] = r and expert r / M, the rows of an expert keep (t, k) order,
    and every other row holds -1."""
    flat = ids.view(-1).long()
    pos = pos.view(-1).long()
    nk, dev = flat.numel(), flat.device
    v = (flat >= 0) & (flat < E)
    hist = torch.bincount(flat[v], minlength=E)
    assert torch.equal(counts.long(), hist) and int(hist.max()) <= M
    assert tuple(status.tolist()) == (nbad, 0)
    assert (pos[~v] == -1).all()
    c = counts.long()
    used_total = 0
    for s, e in chunks(E * M):
        e1 = min(e + 1, E * M)              # one row more, for the order across chunks
        r = torch.arange(s, e1, device=dev)
        ex = r // M
        used = (r % M) < c[ex]
        i = rp[s:e1].long()
        assert (i[~used] == -1).all()
        iu, ru, eu = i[used], r[used], ex[used]
        assert ((iu >= 0) & (iu < nk)).all()
        assert torch.equal(pos[iu], ru) and torch.equal(flat[iu], eu)
        nxt = used[:-1] & used[1:] & (ex[:-1] == ex[1:])
        assert (i[:-1][nxt] < i[1:][nxt]).all()
        used_total += int(used[:e - s].sum())
    assert used_total == int(v.sum())


@pytest.mark.timeout(600)
def test_padded_layout_and_scale_scatter_at_the_row_limit(mg):
    """E*M = 2^31 - 1024 padded rows (E = 1024, M = 2^21 - 1) for a 4096-token
    batch: the layout marks every unused row, and moe_scatter_scales places
    per-token scales into the column-major fp32 [E, 1, M] and UE8M0 int32
    [E, 1, M] arrays (8 GB each) at the used rows only."""
    Np, Ep, Mp = 4096, 1024, (1 << 21) - 1
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    ids = torch.randint(-1, Ep + 1, (Np, K), dtype=torch.int32, device="cuda", generator=g)
    nbad = int((ids >= Ep).sum())
    say(f"padded layout E={Ep} M={Mp}: {Ep * Mp} rows")
    counts = torch.empty(Ep, dtype=torch.int32, device="cuda")
    pos = torch.empty((Np, K), dtype=torch.int32, device="cuda")
    rp = torch.empty(Ep * Mp, dtype=torch.int32, device="cuda")
    status = torch.empty(2, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(mg.moe_layout_workspace_bytes(Np, K, Ep), 256), dtype=torch.uint8,
                     device="cuda")
    mg.moe_get_layout_padded(ids, Ep, Mp, counts, pos, rp, ws, status)
    torch.cuda.synchronize()
    say("padded layout: checking")
    check_sparse_padded(ids, Ep, Mp, counts, pos, rp, status, nbad)

    for fmt, H in ((mg.MOE_SCALE_COLS, 128), (mg.MOE_SCALE_UE8M0, 512)):
        say(f"scale scatter, format {fmt}, H={H}")
        ts = torch.exp2(torch.randint(-20, 20, (Np, H // 128), device="cuda",
                                      generator=g).float())
        canary = -7
        out = torch.full((Ep, 1, Mp), canary, dtype=torch.int32, device="cuda")
        if fmt == mg.MOE_SCALE_COLS:
            out = out.view(torch.float32)
        mg.moe_scatter_scales(ts, K, H, rp, Ep, Mp, out, fmt)
        torch.cuda.synchronize()
        words = out.view(torch.int32).view(-1)
        tsb = ts.view(torch.int32)
        if fmt == mg.MOE_SCALE_COLS:
            want_of = lambda t: tsb[t, 0]
        else:
            ex = ((tsb >> 23) & 0xFF).long()
            packed = ex[:, 0] | (ex[:, 1] << 8) | (ex[:, 2] << 16) | (ex[:, 3] << 24)
            packed = (packed - (packed >= 1 << 31).long() * (1 << 32)).int()   # as int32 bits
            want_of = lambda t: packed[t]
        for s, e in chunks(Ep * Mp):
            i = rp[s:e].long()
            used = i >= 0                   # the layout marks every unused row -1 (checked)
            got = words[s:e]
            assert (got[~used] == canary).all()
            assert torch.equal(got[used], want_of(i[used] // K))
