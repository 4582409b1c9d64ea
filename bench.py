#!/usr/bin/env python3
"""Throughput of the MoE layout -> dispatch -> combine path on one MI355X.

One step = moe_get_layout + moe_dispatch + moe_combine over one batch of the
workload (default: prefill, N=4096 tokens, hidden 7168, top-8 of 256
experts, fp8 e4m3 hidden + fp32 scales dispatched, bf16 expert outputs
combined with fp32 accumulation). Inputs are seeded synthetic data already
resident in HBM when timing starts; buffer sets rotate so one step's data is
not left in the 256 MB last-level cache for the next.

Prints one JSON line: effective GB/s (algorithmic bytes / step time),
tokens/s, per-op times, the combine kernel against the 8 TB/s HBM roofline,
and the CPU oracle timed on the host as a baseline.

    python bench.py [--steps K] [--warmup W] [--config prefill]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine effective HBM GB/s and tokens/s, 4096×7168 top-8, 1 GPU"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_bytes(N, K, E, P, Hc, R, cap, epilogue=False):
    """Bytes each op must move at minimum: every input read once, every
    output written once. With the epilogue, combine also reads the residual
    and gamma and writes residual_out."""
    layout = 4 * N * K + 8 * E + 4 + 4 * N * K + 4 * cap
    dispatch = N * P + 4 * N * K + R * P
    combine = R * Hc * 2 + 8 * N * K + N * Hc * 2
    if epilogue:
        combine += N * Hc * 2 + Hc * 2 + N * Hc * 2
    return layout, dispatch, combine


def source_hash(paths):
    """Hash of a kernel's source files (one path or several) with comments and
    whitespace removed, so that counters stay attached to a kernel until its
    code changes."""
    import re

    if isinstance(paths, str):
        paths = [paths]
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(re.sub(r"\s+", " ", text).strip().encode() + b"\0")
    return h.hexdigest()[:16]


def traffic_entry(kernel, workload):
    """Measured HBM bytes per launch for `kernel` on `workload`, if the
    counters were taken on the current kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(f"{kernel}/{workload}")
    if not e or e.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return e


_CSRC = os.path.join(ROOT, "combine_moe_get_amd", "csrc")
# Each kernel's source file and the library headers it is built with.
_HDRS = (os.path.join(_CSRC, "internal.hpp"), os.path.join(_CSRC, "fp8.hpp"))
KERNEL_SOURCES = {k: (os.path.join(_CSRC, f),) + _HDRS for k, f in (
    ("combine_epilogue_kernel", "combine.hip"),
    ("combine_kernel", "combine.hip"),
    ("combine_held_kernel", "combine.hip"),
    ("dispatch_kernel", "dispatch.hip"),
    ("layout_hist", "layout.hip"),
    ("layout_assign", "layout.hip"),
    ("layout_onepass", "layout.hip"),
    ("dispatch_fp8_kernel", "quant.hip"),
    ("combine_backward_kernel", "combine.hip"),
    ("combine_backward_group_kernel", "combine.hip"),
    ("dispatch_fp8_padded_kernel", "quant.hip"),
    ("layout_dispatch_kernel", "dispatch.hip"),
    ("scatter_scales_kernel", "quant.hip"),
)}
def combine_kernel_name(N, K, Hc):
    """The kernel moe_combine (and moe_dispatch_backward, with H for Hc) runs
    for N tokens, top-K and Hc channels of 16-byte-aligned rows (every
    workload here): the held form past 32768
    waves (one per token and 64-vector segment) for K <= 8 and 8 to 224
    segments per row, else combine_kernel. The same rule as the library's
    (combine.hip), which also needs the device's compute-unit count (always
    known on these GPUs) and a grid of at most 2^22 workgroups."""
    segs = -(-(Hc // 8) // 64)
    if N * segs > 32768 and K <= 8 and 8 <= segs <= 224:
        return "combine_held_kernel"
    return "combine_kernel"


COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 2 << 30     # bytes read (and written) per launch by copy_bandwidth()


def _counter_rows(directory):
    import csv
    import glob

    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {directory}")
    for f in files:
        with open(f) as fh:
            yield from csv.DictReader(fh)


def kernel_key(name):
    """The function name of a profiled kernel ("void moe::(anonymous
    namespace)::combine_kernel<4, false>(...)" -> "combine_kernel")."""
    import re

    m = re.match(r"(?:void\s+)?(?:[\w:]*\(anonymous namespace\)::|moe::)*([A-Za-z_]\w*)", name)
    return m.group(1) if m else name


def _per_kernel(directory, counter):
    """{short kernel name: [value per dispatch]} for one counter."""
    out = {}
    for r in _counter_rows(directory):
        if r.get("Counter_Name") != counter:
            continue
        key = kernel_key(r["Kernel_Name"])
        if key in KERNEL_SOURCES or key == COPY_KERNEL:
            out.setdefault(key, []).append(float(r["Counter_Value"]))
    return out


def kernel_name_with_args(name):
    """A profiled kernel's name with its template arguments but without
    namespaces and parameters ("void (anonymous namespace)::read_kernel<true,
    1>(...)" -> "read_kernel<true, 1>")."""
    import re

    base = re.sub(r"^void\s+", "", name)
    base = re.sub(r"(?:[\w]*\(anonymous namespace\)::|moe::)", "", base)
    depth, out = 0, []
    for ch in base:
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out).strip()


def summarize_ceiling_traffic(fetch_dir, write_dir):
    """HBM bytes per launch of every kernel `bench.py --ceilings` runs, from
    two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE), calibrated by the
    2 GiB device copy that run also makes. Printed as a table."""
    def rows(counter):
        out = {}
        for r in _counter_rows(fetch_dir if counter == "FETCH_SIZE" else write_dir):
            if r.get("Counter_Name") == counter:
                out.setdefault(kernel_name_with_args(r["Kernel_Name"]), []).append(
                    float(r["Counter_Value"]))
        return out

    fetch, write = rows("FETCH_SIZE"), rows("WRITE_SIZE")
    known_kib = COPY_BYTES / 1024

    def calib(vals):
        big = sorted(v for v in vals if v > 0.5 * max(vals, default=0.0))
        if len(big) < 3:
            raise SystemExit(f"need the {COPY_KERNEL} launches of copy_bandwidth(), got {vals}")
        return known_kib / big[len(big) // 2]

    fscale, wscale = calib(fetch.get(COPY_KERNEL, [])), calib(write.get(COPY_KERNEL, []))
    print(f"copy calibration: FETCH x{fscale:.4f}, WRITE x{wscale:.4f}")
    print("| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |")
    print("|---|---|---|---|---|---|")
    for k in sorted(set(fetch) & set(write)):
        if k == COPY_KERNEL:
            continue
        f, w = float(np.median(fetch[k])), float(np.median(write[k]))
        print(f"| {k} | {len(fetch[k])} | {f:.0f} | {w:.0f} | {f * fscale * 1024 / 1e6:.2f} | "
              f"{w * wscale * 1024 / 1e6:.2f} |")


def summarize_write_requests(directory):
    """Write requests that leave the L2 (TCC) for memory, per kernel, from a
    rocprofv3 --pmc run of TCC_EA0_WRREQ, TCC_EA0_WRREQ_64B and
    TCC_EA0_WRREQ_DRAM_CREDIT_STALL in its default (SQLite) output: requests
    per launch, the share that are whole 64-byte requests (the rest are 32
    bytes), the bytes they carry, and how evenly the requests and the stalls
    for want of memory credits spread over the 16 x 8 L2 channels (per-channel
    values, median over launches)."""
    import glob
    import sqlite3

    dbs = glob.glob(os.path.join(directory, "**", "*.db"), recursive=True)
    if not dbs:
        raise SystemExit(f"no rocprofv3 database under {directory}")
    per = {}   # kernel -> counter -> dispatch -> [per-channel values]
    for db in dbs:
        con = sqlite3.connect(db)
        for disp, name, counter, value in con.execute(
                "select dispatch_id, name, counter_name, counter_value from pmc_events order by id"):
            k = kernel_name_with_args(name)
            per.setdefault(k, {}).setdefault(counter, {}).setdefault(disp, []).append(value)
        con.close()
    print("| kernel | launches | write requests / launch | 64-B share | bytes / launch (MB) | "
          "requests per channel min / median / max | credit-stall cycles per channel "
          "min / median / max |")
    print("|---|---|---|---|---|---|---|")
    for k in sorted(per):
        c = per[k]
        if "TCC_EA0_WRREQ" not in c or "TCC_EA0_WRREQ_64B" not in c:
            continue
        tot = [sum(v) for v in c["TCC_EA0_WRREQ"].values()]
        b64 = [sum(v) for v in c["TCC_EA0_WRREQ_64B"].values()]
        if np.median(tot) < 1000:
            continue
        req, r64 = float(np.median(tot)), float(np.median(b64))
        nbytes = 64 * r64 + 32 * (req - r64)
        ch = np.median(np.array(list(c["TCC_EA0_WRREQ"].values()), dtype=float), axis=0)
        st = c.get("TCC_EA0_WRREQ_DRAM_CREDIT_STALL")
        stall = (np.median(np.array(list(st.values()), dtype=float), axis=0) if st
                 else np.zeros(1))
        print(f"| {k} | {len(tot)} | {req:.0f} | {r64 / req:.3f} | {nbytes / 1e6:.2f} | "
              f"{ch.min():.0f} / {np.median(ch):.0f} / {ch.max():.0f} | "
              f"{stall.min():.0f} / {np.median(stall):.0f} / {stall.max():.0f} |")


def summarize_traffic(fetch_dir, write_dir, workload, command):
    """HBM traffic per launch from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, both in KiB per dispatch), each scaled by what the same
    counter reads for the 2 GiB device copy of copy_bandwidth()."""
    fetch, write = _per_kernel(fetch_dir, "FETCH_SIZE"), _per_kernel(write_dir, "WRITE_SIZE")
    known_kib = COPY_BYTES / 1024

    def copy_median(vals):
        # The 2 GiB copies of copy_bandwidth() are the largest launches of
        # that kernel (the runtime also uses it for small uploads); they must
        # read alike, whatever scale the counter has.
        big = [v for v in vals if v > 0.5 * max(vals, default=0.0)]
        if len(big) < 3:
            raise SystemExit(f"need the {COPY_KERNEL} launches of copy_bandwidth(), got {vals}")
        m = float(np.median(big))
        if max(abs(v - m) for v in big) > 0.1 * m:
            raise SystemExit(f"{COPY_KERNEL} launches disagree: {big}")
        return m

    fscale = known_kib / copy_median(fetch.get(COPY_KERNEL, []))
    wscale = known_kib / copy_median(write.get(COPY_KERNEL, []))
    result = {}
    lines = ["| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated HBM bytes / launch |",
             "|---|---|---|---|---|"]
    for k, src in KERNEL_SOURCES.items():
        if k not in fetch or k not in write:
            continue
        f, w = float(np.mean(fetch[k])), float(np.mean(write[k]))
        b = (f * fscale + w * wscale) * 1024
        result[f"{k}/{workload}"] = {
            "fetch_kib_per_launch": round(f, 1), "write_kib_per_launch": round(w, 1),
            "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5),
            "bytes_per_launch": int(round(b)), "launches": len(fetch[k]),
            "source_sha256_16": source_hash(src), "command": command,
        }
        lines.append(f"| {k} | {len(fetch[k])} | {f:.1f} | {w:.1f} | {b:.0f} |")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    old = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            old = json.load(fh)
    old.update(result)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(old, fh, indent=1, sort_keys=True)
    print(f"copy calibration: FETCH x{fscale:.4f}, WRITE x{wscale:.4f} "
          f"({COPY_KERNEL}, {COPY_BYTES} B read and written per launch)")
    print("\n".join(lines))


class HipEvents:
    """Timing-only HIP events, created through the HIP runtime torch loaded,
    with hipEventDisableSystemFence: recording one skips the system-scope
    cache write-back and invalidate an ordinary event record performs, so
    per-op timestamps inside the timed loop barely perturb it."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self, torch):
        import ctypes

        self.ct = ctypes
        lib = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
        self.L = ctypes.CDLL(lib)
        self.L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def create(self):
        ev = self.ct.c_void_p()
        rc = self.L.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        self.events.append(ev)
        return ev

    def record(self, ev, stream):
        rc = self.L.hipEventRecord(ev, stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, a, b):
        ms = self.ct.c_float()
        self.L.hipEventSynchronize(b)
        rc = self.L.hipEventElapsedTime(self.ct.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def close(self):
        for ev in self.events:
            self.L.hipEventDestroy(ev)
        self.events = []


class BufferSet:
    """Device inputs and outputs of one step."""

    def __init__(self, torch, mg, wl, y_bits, fused=False):
        d = "cuda"
        self.fused = fused
        if wl.records is not None:
            # record mode: one 16-B-aligned record per token moves whole; the
            # ids and weights are read in place from inside the records
            rec = torch.from_numpy(wl.records).to(d)
            self.srcs = [rec]
            self.ids = rec.view(torch.int32)[:, :wl.K]
            self.w = rec.view(torch.float32)[:, 8:8 + wl.K]
            self.ids_stride = self.w_stride = rec.shape[1] // 4
        else:
            self.ids = torch.from_numpy(np.ascontiguousarray(wl.ids)).to(d)
            self.w = torch.from_numpy(np.ascontiguousarray(wl.weights)).to(d)
            self.srcs = [torch.from_numpy(a).to(d) for _, a in wl.fields]
            self.ids_stride = self.w_stride = wl.K
        self.y = torch.from_numpy(y_bits.view(np.int16)).to(d).view(torch.bfloat16)
        N, K, E = wl.N, wl.K, wl.E
        self.cap = cap = mg.moe_required_capacity(N, K, E, 1)
        self.counts = torch.empty(E, dtype=torch.int32, device=d)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=d)
        self.pos = torch.empty((N, K), dtype=torch.int32, device=d)
        self.row_pair = torch.empty(cap, dtype=torch.int32, device=d)
        self.order = torch.empty(N * K, dtype=torch.int32, device=d)   # the dispatch plan
        self.status = torch.empty(1, dtype=torch.int32, device=d)
        self.ws = torch.empty(mg.moe_layout_workspace_bytes(N, K, E), dtype=torch.uint8, device=d)
        self.dsts = [torch.empty((cap, a.shape[1]), dtype=torch.uint8, device=d) for a in self.srcs]
        self.out = torch.empty((N, wl.Hc), dtype=torch.bfloat16, device=d)
        g = torch.Generator().manual_seed(wl.seed + 31)
        self.residual = (torch.randn((N, wl.Hc), generator=g) * 2).to(torch.bfloat16).to(d)
        self.gamma = (torch.rand(wl.Hc, generator=g) + 0.5).to(torch.bfloat16).to(d)
        self.residual_out = torch.empty((N, wl.Hc), dtype=torch.bfloat16, device=d)

    def calls(self, mg, wl, stream, epilogue=False):
        """Argument tuples of the three C-ABI calls, marshalled once."""
        L = mg._lib
        N, K, E = wl.N, wl.K, wl.E
        fields = (mg.moe_field * len(self.srcs))()
        for i, (s, t) in enumerate(zip(self.srcs, self.dsts)):
            fields[i] = mg.moe_field(s.data_ptr(), s.stride(0), t.data_ptr(), t.stride(0), s.shape[1])
        self._fields = fields
        lay = (self.ids.data_ptr(), self.ids_stride, N, K, E, 1, self.counts.data_ptr(), self.offsets.data_ptr(),
               self.pos.data_ptr(), self.row_pair.data_ptr(), self.cap, self.order.data_ptr(),
               self.ws.data_ptr(), self.ws.numel(), self.status.data_ptr(), stream)
        dis = (fields, len(self.srcs), N, K, self.pos.data_ptr(), self.order.data_ptr(), stream)
        if self.fused:
            ld = (self.ids.data_ptr(), self.ids_stride, N, K, E, 1, self.counts.data_ptr(),
                  self.offsets.data_ptr(), self.pos.data_ptr(), self.row_pair.data_ptr(), self.cap,
                  self.status.data_ptr(), fields, len(self.srcs), stream)
            com = (self.y.data_ptr(), wl.Hc, self.w.data_ptr(), self.w_stride, self.pos.data_ptr(),
                   N, K, wl.Hc, self.out.data_ptr(), wl.Hc, stream)
            return (L.moe_layout_dispatch, ld), (L.moe_combine, com)
        if not epilogue:
            com = (self.y.data_ptr(), wl.Hc, self.w.data_ptr(), self.w_stride, self.pos.data_ptr(),
                   N, K, wl.Hc, self.out.data_ptr(), wl.Hc, stream)
            return (L.moe_get_layout, lay), (L.moe_dispatch, dis), (L.moe_combine, com)
        import ctypes

        ep = mg.moe_epilogue()
        ep.residual, ep.residual_row_stride = self.residual.data_ptr(), wl.Hc
        ep.gamma, ep.eps = self.gamma.data_ptr(), 1e-6
        ep.residual_out, ep.residual_out_row_stride = self.residual_out.data_ptr(), wl.Hc
        self._ep = ep
        com = (self.y.data_ptr(), wl.Hc, self.w.data_ptr(), self.w_stride, self.pos.data_ptr(), N,
               K, wl.Hc, ctypes.byref(ep), self.out.data_ptr(), wl.Hc, stream)
        return (L.moe_get_layout, lay), (L.moe_dispatch, dis), (L.moe_combine_epilogue, com)


SCALE_FORMATS = {"rows": 0, "cols": 1, "ue8m0": 2}


def ll_algorithmic_bytes(N, K, E, M, H, Hc, R, scale_format):
    """Minimum bytes of the low-latency step. Layout: ids in, counts, pos
    and the whole padded row_pair table (E*M entries, unused rows -1) out.
    Dispatch: each token's bf16 row read once, pos, and per landed pair H
    e4m3 codes plus its scales (4 B per 128 channels, or 1 B per 128 as
    packed UE8M0 exponents). Combine as in the plain step."""
    layout = 4 * N * K + 4 * E + 4 * N * K + 4 * E * M + 8
    sb = H // 128 if scale_format == "ue8m0" else 4 * (H // 128)
    dispatch = 2 * N * H + 4 * N * K + R * (H + sb)
    combine = R * Hc * 2 + 8 * N * K + N * Hc * 2
    return layout, dispatch, combine


class LowLatencySet:
    """Device inputs and outputs of one low-latency step: padded layout (M
    rows per expert), bf16 -> e4m3 cast on dispatch with per-128-channel
    scales, combine reading the expert outputs from the padded buffer."""

    def __init__(self, torch, mg, wl, x_bits, y_bits, M, scale_format, round_scale, fused=False,
                 staged=False):
        d = "cuda"
        self.fused = fused
        N, K, E, Hc = wl.N, wl.K, wl.E, wl.Hc
        H = x_bits.shape[1]
        self.M, self.H, self.fmt = M, H, SCALE_FORMATS[scale_format]
        # staged: per-token scales (MOE_SCALE_TOKENS) placed by moe_scatter_scales
        self.staged = staged
        if staged:
            self.tok = torch.empty((N, H // 128), dtype=torch.float32, device=d)
        self.round_scale = int(round_scale)
        self.ids = torch.from_numpy(np.ascontiguousarray(wl.ids)).to(d)
        self.w = torch.from_numpy(np.ascontiguousarray(wl.weights)).to(d)
        self.x = torch.from_numpy(x_bits.view(np.int16)).to(d).view(torch.bfloat16)
        self.counts = torch.empty(E, dtype=torch.int32, device=d)
        self.pos = torch.empty((N, K), dtype=torch.int32, device=d)
        self.row_pair = torch.empty(E * M, dtype=torch.int32, device=d)
        self.status = torch.empty(2, dtype=torch.int32, device=d)
        self.ws = torch.empty(mg.moe_layout_workspace_bytes(N, K, E), dtype=torch.uint8, device=d)
        self.codes = torch.empty((E * M, H), dtype=torch.uint8, device=d)
        if self.fmt == 0:
            self.scales = torch.empty((E * M, H // 128), dtype=torch.float32, device=d)
        elif self.fmt == 1:
            self.scales = torch.empty((E, H // 128, M), dtype=torch.float32, device=d)
        else:
            self.scales = torch.empty((E, H // 512, M), dtype=torch.int32, device=d)
        self.out = torch.empty((N, Hc), dtype=torch.bfloat16, device=d)
        # Expert outputs in the padded layout: pair (t, k) finds the
        # workload's y row t*K + k at its padded row; other rows are unused.
        # the receive metadata of the pages' low-latency dispatch: each
        # expert's row range and its running count of received rows
        self.layout_range = torch.empty(E, dtype=torch.int64, device=d)
        self.recv_stats = torch.zeros(E, dtype=torch.int32, device=d)
        mg.moe_get_layout_padded(self.ids, E, M, self.counts, self.pos, self.row_pair,
                                 self.ws, self.status)
        torch.cuda.synchronize()
        st = self.status.cpu().tolist()
        if st != [0, 0]:
            raise SystemExit(f"low-latency bench needs no bad ids and no drops (status {st}); "
                             f"raise --rows-per-expert above {M}")
        y = torch.from_numpy(y_bits.view(np.int16)).to(d).view(torch.bfloat16)
        self.y = torch.empty((E * M, Hc), dtype=torch.bfloat16, device=d)
        self.y[self.pos.flatten().long()] = y
        del y

    def calls(self, mg, wl, stream, epilogue=False):
        L = mg._lib
        N, K, E, Hc, H, M = wl.N, wl.K, wl.E, wl.Hc, self.H, self.M
        srs = H // 128 if self.fmt == 0 else 0
        lay = (self.ids.data_ptr(), K, N, K, E, M, self.counts.data_ptr(), self.pos.data_ptr(),
               self.row_pair.data_ptr(), self.layout_range.data_ptr(), self.recv_stats.data_ptr(),
               self.ws.data_ptr(), self.ws.numel(), self.status.data_ptr(), stream)
        dis = (self.x.data_ptr(), H, N, K, H, self.pos.data_ptr(), self.codes.data_ptr(), H,
               self.scales.data_ptr(), self.fmt, srs, M, self.round_scale, stream)
        com = (self.y.data_ptr(), Hc, self.w.data_ptr(), K, self.pos.data_ptr(), N, K, Hc,
               self.out.data_ptr(), Hc, stream)
        if self.staged:
            dis = (self.x.data_ptr(), H, N, K, H, self.pos.data_ptr(), self.codes.data_ptr(), H,
                   self.tok.data_ptr(), mg.MOE_SCALE_TOKENS, H // 128, M, self.round_scale, stream)
            sca = (self.tok.data_ptr(), H // 128, N, K, H, self.row_pair.data_ptr(), E, M,
                   self.scales.data_ptr(), self.fmt, stream)
            return ((L.moe_get_layout_padded, lay), (L.moe_dispatch_fp8, dis),
                    (L.moe_scatter_scales, sca), (L.moe_combine, com))
        if self.fused:
            fu = (self.ids.data_ptr(), K, N, K, E, M, self.x.data_ptr(), H, H,
                  self.counts.data_ptr(), self.pos.data_ptr(), self.row_pair.data_ptr(),
                  self.layout_range.data_ptr(), self.recv_stats.data_ptr(),
                  self.status.data_ptr(), self.codes.data_ptr(), H, self.scales.data_ptr(),
                  self.fmt, srs, self.round_scale, stream)
            return (L.moe_dispatch_fp8_padded, fu), (L.moe_combine, com)
        return (L.moe_get_layout_padded, lay), (L.moe_dispatch_fp8, dis), (L.moe_combine, com)


def bwd_algorithmic_bytes(N, K, H, Hc, R):
    """Minimum bytes of the backward step. Combine backward: grad_out, w and
    pos in, y read for the weight gradients, grad_y and grad_w out. Dispatch
    backward: grad_recv and grad_recv_w rows in, pos, grad_x and grad_w out."""
    combine_bwd = N * Hc * 2 + 8 * N * K + R * Hc * 2 + R * Hc * 2 + 4 * N * K
    dispatch_bwd = R * H * 2 + 4 * N * K + R * K * 4 + N * H * 2 + 4 * N * K
    return combine_bwd, dispatch_bwd


class BackwardSet:
    """Device buffers of one backward step on the forward's layout: combine
    backward (grad_out -> grad_y rows and grad_w) and dispatch backward
    (grad_recv rows -> grad_x, grad_recv_w rows -> grad_w_in)."""

    def __init__(self, torch, mg, wl, host):
        d = "cuda"
        N, K, E, Hc = wl.N, wl.K, wl.E, wl.Hc
        H = host["grad_recv"].shape[1]
        self.H = H
        bf = lambda a: torch.from_numpy(a.view(np.int16)).to(d).view(torch.bfloat16)
        self.ids = torch.from_numpy(np.ascontiguousarray(wl.ids)).to(d)
        self.w = torch.from_numpy(np.ascontiguousarray(wl.weights)).to(d)
        lay = mg.layout(self.ids, E)       # the forward's layout, computed once
        torch.cuda.synchronize()
        self.pos = lay.pos
        self.y = bf(host["y"])
        self.grad_out = bf(host["grad_out"])
        self.grad_recv = bf(host["grad_recv"])
        self.grad_recv_w = torch.from_numpy(host["grad_recv_w"]).to(d)
        R = N * K
        self.grad_y = torch.empty((R, Hc), dtype=torch.bfloat16, device=d)
        self.grad_w = torch.empty((N, K), dtype=torch.float32, device=d)
        self.grad_x = torch.empty((N, H), dtype=torch.bfloat16, device=d)
        self.grad_w_in = torch.empty((N, K), dtype=torch.float32, device=d)

    def calls(self, mg, wl, stream, epilogue=False):
        L = mg._lib
        N, K, Hc, H = wl.N, wl.K, wl.Hc, self.H
        cb = (self.grad_out.data_ptr(), Hc, self.w.data_ptr(), K, self.y.data_ptr(), Hc,
              self.pos.data_ptr(), N, K, Hc, self.grad_y.data_ptr(), Hc, self.grad_w.data_ptr(), K,
              stream)
        db = (self.grad_recv.data_ptr(), H, self.grad_recv_w.data_ptr(), K, self.pos.data_ptr(),
              N, K, H, self.grad_x.data_ptr(), H, self.grad_w_in.data_ptr(), K, stream)
        return (L.moe_combine_backward, cb), (L.moe_dispatch_backward, db)


def copy_bandwidth(torch, nbytes=2 << 30, reps=10):
    """A plain device copy (read + write) of `nbytes`: the achievable-HBM
    reference next to the 8 TB/s spec."""
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) / reps * 1e-3
    del a, b
    return 2 * nbytes / t / 1e9


def cpu_baseline(wl, y, total_bytes, budget_s, epilogue=None):
    """The oracle as it stands, on the host cores: full steps of the same
    workload (layout serial, dispatch and combine OpenMP over tokens) until
    `budget_s` seconds of work are done. With `epilogue` = (residual, gamma)
    as bf16 bits, the step's combine is the oracle's combine epilogue with
    that residual add and RMSNorm, as on the GPU."""
    import oracle

    srcs = [wl.records] if wl.records is not None else [a for _, a in wl.fields]
    w = wl.weights                       # read in place (strided inside records)
    dsts = [np.empty((wl.N * wl.K, a.shape[1]), np.uint8) for a in srcs]

    def one():
        _, _, pos, _, _ = oracle.layout(wl.ids, wl.E)
        oracle.dispatch(srcs, pos, wl.K, dsts=dsts)
        if epilogue is None:
            oracle.combine(y, w, pos)
        else:
            oracle.combine_epilogue(y, w, pos, residual=epilogue[0], gamma=epilogue[1], eps=1e-6)

    what = "layout+dispatch+combine" if epilogue is None else \
        "layout+dispatch+combine with residual add and RMSNorm"
    return _time_oracle(one, wl, total_bytes, budget_s, f"full {wl.name} steps ({what})")


def _time_oracle(one, wl, total_bytes, budget_s, what):
    """Median step time of the oracle at the configured thread count, then
    again on one thread (the layout is serial either way)."""
    import oracle

    def run(budget):
        one()   # warm host caches and page in outputs
        times = []
        t_all = time.perf_counter()
        while not times or (time.perf_counter() - t_all < budget and len(times) < 50):
            t0 = time.perf_counter()
            one()
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), len(times)

    cores = int(oracle.lib().omp_get_max_threads())
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next(l.split(":", 1)[1].strip() for l in fh if l.startswith("model name"))
    except (OSError, StopIteration):
        pass
    t, n = run(budget_s)
    prev = oracle.set_threads(1)
    try:
        t1, n1 = run(budget_s / 2)
    finally:
        oracle.set_threads(prev)
    return {
        "value": round(total_bytes / t / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "cpu_model": cpu_model,
        "sample": f"{n} {what}, median {t * 1e3:.1f} ms/step, {wl.N / t:.0f} tokens/s",
        "single_thread": {"value": round(total_bytes / t1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                          "sample": f"{n1} steps, median {t1 * 1e3:.1f} ms/step"},
    }


def cpu_baseline_ll(wl, x, y, M, scale_format, round_scale, total_bytes, budget_s):
    """The oracle on the host cores for the low-latency step: padded layout
    (serial), FP8 cast on dispatch and combine (OpenMP over tokens)."""
    import oracle

    E, Hc, H = wl.E, wl.Hc, x.shape[1]
    fmt = SCALE_FORMATS[scale_format]
    w = np.ascontiguousarray(wl.weights)
    _, pos0, _, _ = oracle.layout_padded(wl.ids, E, M)
    # padded buffers are allocated untouched; only the landed rows page in
    codes = np.empty((E * M, H), np.uint8)
    sshape = {0: ((E * M, H // 128), np.float32), 1: ((E, H // 128, M), np.float32),
              2: ((E, H // 512, M), np.int32)}[fmt]
    scales = np.empty(*sshape)
    y_pad = np.empty((E * M, Hc), np.uint16)
    y_pad[pos0.reshape(-1)] = y

    def one():
        _, pos, _, _ = oracle.layout_padded(wl.ids, E, M)
        oracle.dispatch_fp8(x, pos, E * M, fmt, M, round_scale, codes=codes, scales=scales)
        oracle.combine(y_pad, w, pos)

    return _time_oracle(one, wl, total_bytes, budget_s,
                        f"full low-latency {wl.name} steps (padded layout + fp8 cast dispatch "
                        "+ combine)")


def cpu_baseline_bwd(wl, host, total_bytes, budget_s):
    """The oracle on the host cores for the backward step (OpenMP over tokens)."""
    import oracle

    _, _, pos, _, _ = oracle.layout(wl.ids, wl.E)
    w = np.ascontiguousarray(wl.weights)

    def one():
        oracle.combine_backward(host["grad_out"], w, pos, wl.N * wl.K, y=host["y"])
        oracle.dispatch_backward(host["grad_recv"], pos, host["grad_recv_w"])

    return _time_oracle(one, wl, total_bytes, budget_s,
                        f"full {wl.name} backward steps (combine backward + dispatch backward)")


def ceilings(torch, mg, mw, reps):
    """Bandwidth ceilings of the memory patterns the kernels use, timed on
    this GPU next to the dispatch and combine themselves (prefill shapes):
    streaming reads, writes and copies of 1 GiB (plain and non-temporal, 1 or
    8 KiB per wave), the combine's 8:1 read/write mix as a stream, the
    dispatch's exact stores with no loads, and the combine's exact loads with
    no stores. The pattern kernels live in libmoe_ceilings.so. Each pattern is
    launched `reps` times on alternating buffers (well beyond the 256 MB
    last-level cache), each launch timed with events; the median is kept."""
    import ctypes

    L = ctypes.CDLL(os.path.join(ROOT, "combine_moe_get_amd", "libmoe_ceilings.so"))
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.ceil_read.argtypes = [P, i64, ctypes.c_int, ctypes.c_int, P, P]
    L.ceil_write.argtypes = [P, i64, ctypes.c_int, ctypes.c_int, P]
    L.ceil_copy.argtypes = [P, P, i64, ctypes.c_int, ctypes.c_int, P]
    L.ceil_mix.argtypes = [P, P, i64, ctypes.c_int, P]
    L.ceil_dispatch_stores.argtypes = [P, P, P, i32, P, i32, i32, P]
    L.ceil_combine_reads.argtypes = [P, i64, P, i32, i32, i32, P, P]
    L.ceil_empty.argtypes = [i32, P]
    stream = torch.cuda.current_stream().cuda_stream
    gib = 1 << 30
    src = [torch.empty(gib, dtype=torch.uint8, device="cuda") for _ in range(2)]
    dst = [torch.empty(gib, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for t in src:
        t.fill_(3)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    wl = mw.make("prefill")
    y_bits = wl.y()
    sets = [BufferSet(torch, mg, wl, y_bits) for _ in range(2)]
    N, K, Hc = wl.N, wl.K, wl.Hc
    for st in sets:
        mg.moe_get_layout(st.ids, wl.E, 1, st.counts, st.offsets, st.pos, st.row_pair, st.ws,
                          st.status, order=st.order)
    torch.cuda.synchronize()
    nf = len(sets[0].dsts)
    fields = []
    for st in sets:
        d = (P * nf)(*[t.data_ptr() for t in st.dsts])
        ds = (i64 * nf)(*[t.stride(0) for t in st.dsts])
        rb = (i64 * nf)(*[a.shape[1] for a in st.srcs])
        fields.append((d, ds, rb))
    R = N * K
    disp_bytes = R * sum(a.shape[1] for a in sets[0].srcs)
    y_bytes = R * Hc * 2
    out_bytes = N * Hc * 2

    def ok(rc):
        if rc != 0:
            raise RuntimeError("a ceiling kernel failed to launch")

    patterns = [
        ("read, non-temporal, 1 KiB per wave", "read_kernel<true, 1>", gib,
         lambda i: ok(L.ceil_read(src[i].data_ptr(), gib, 1, 1, sink.data_ptr(), stream))),
        ("read, non-temporal, 8 KiB per wave", "read_kernel<true, 8>", gib,
         lambda i: ok(L.ceil_read(src[i].data_ptr(), gib, 1, 8, sink.data_ptr(), stream))),
        ("read, plain, 1 KiB per wave", "read_kernel<false, 1>", gib,
         lambda i: ok(L.ceil_read(src[i].data_ptr(), gib, 0, 1, sink.data_ptr(), stream))),
        ("write, non-temporal, 1 KiB per wave", "write_kernel<true, 1>", gib,
         lambda i: ok(L.ceil_write(dst[i].data_ptr(), gib, 1, 1, stream))),
        ("write, non-temporal, 8 KiB per wave", "write_kernel<true, 8>", gib,
         lambda i: ok(L.ceil_write(dst[i].data_ptr(), gib, 1, 8, stream))),
        ("write, plain, 1 KiB per wave", "write_kernel<false, 1>", gib,
         lambda i: ok(L.ceil_write(dst[i].data_ptr(), gib, 0, 1, stream))),
        ("copy, non-temporal, 1 KiB per wave (bytes read + written)", "copy_kernel<true, 1>",
         2 * gib, lambda i: ok(L.ceil_copy(src[i].data_ptr(), dst[i].data_ptr(), gib, 1, 1,
                                            stream))),
        ("copy, plain, 1 KiB per wave (bytes read + written)", "copy_kernel<false, 1>", 2 * gib,
         lambda i: ok(L.ceil_copy(src[i].data_ptr(), dst[i].data_ptr(), gib, 0, 1, stream))),
        ("8:1 read/write mix, streamed (the combine's bytes)", "mix_kernel", y_bytes + out_bytes,
         lambda i: ok(L.ceil_mix(sets[i].y.data_ptr(), sets[i].out.data_ptr(), out_bytes // 1024,
                                 8, stream))),
        ("dispatch stores, prefill rows from pos, no loads", "dispatch_stores_kernel<true>",
         disp_bytes, lambda i: ok(L.ceil_dispatch_stores(*fields[i], nf, sets[i].pos.data_ptr(),
                                                         N, K, stream))),
        ("dispatch stores, rows in pair order, no loads", "dispatch_stores_kernel<false>", disp_bytes,
         lambda i: ok(L.ceil_dispatch_stores(*fields[i], nf, None, N, K, stream))),
        ("combine loads, prefill rows from pos, no stores", "combine_reads_kernel<true>", y_bytes,
         lambda i: ok(L.ceil_combine_reads(sets[i].y.data_ptr(), Hc, sets[i].pos.data_ptr(), N,
                                           K, Hc, sink.data_ptr(), stream))),
        ("combine loads, rows in pair order, no stores", "combine_reads_kernel<false>", y_bytes,
         lambda i: ok(L.ceil_combine_reads(sets[i].y.data_ptr(), Hc, None, N, K, Hc,
                                           sink.data_ptr(), stream))),
        ("moe_dispatch (the product kernel), prefill, pairs in the layout's plan",
         "dispatch_kernel", algorithmic_bytes(N, K, wl.E, wl.payload_bytes(), Hc, R, sets[0].cap)[1],
         lambda i: mg.moe_dispatch(sets[i].srcs, sets[i].dsts, sets[i].pos, K,
                                   order=sets[i].order)),
        ("moe_dispatch (the product kernel), prefill, pairs in index order", "dispatch_kernel",
         algorithmic_bytes(N, K, wl.E, wl.payload_bytes(), Hc, R, sets[0].cap)[1],
         lambda i: mg.moe_dispatch(sets[i].srcs, sets[i].dsts, sets[i].pos, K)),
        ("moe_combine (the product kernel), prefill", combine_kernel_name(N, K, Hc),
         algorithmic_bytes(N, K, wl.E, wl.payload_bytes(), Hc, R, sets[0].cap)[2],
         lambda i: mg.moe_combine(sets[i].y, sets[i].w, sets[i].pos, sets[i].out)),
    ]
    res = {}
    # Launch-bound work, timed as calls per unit of time: `reps` rounds of 50
    # calls back to back between two events, the median round kept.
    for st in sets:
        mg.moe_get_layout(st.ids, wl.E, 1, st.counts, st.offsets, st.pos, st.row_pair, st.ws,
                          st.status, order=st.order)
    # The layout through the C ABI with its arguments marshalled once, so that
    # the host's per-call cost is the launch's alone: ids on a 16-byte
    # boundary (the one-pass kernel) and the same ids 4 bytes past one (the
    # two kernels).
    st0 = sets[0]
    ids_off = torch.empty(N * K + 1, dtype=torch.int32, device=st0.ids.device)[1:]
    ids_off.copy_(st0.ids.reshape(-1))
    ws_bytes = st0.ws.numel()

    def layout_call(ids_ptr):
        return lambda: ok(mg._lib.moe_get_layout(
            ids_ptr, K, N, K, wl.E, 1, st0.counts.data_ptr(), st0.offsets.data_ptr(),
            st0.pos.data_ptr(), st0.row_pair.data_ptr(), st0.row_pair.numel(),
            st0.order.data_ptr(), st0.ws.data_ptr(), ws_bytes, st0.status.data_ptr(), stream))

    calls = [
        ("launch floor: empty kernel, 64 workgroups, per launch", "empty_kernel",
         lambda: ok(L.ceil_empty(64, stream))),
        ("moe_get_layout (one launch), prefill, per call", "layout_onepass",
         layout_call(st0.ids.data_ptr())),
        ("moe_get_layout (two launches: ids off a 16-byte boundary), prefill, per call",
         "layout_hist + layout_assign", layout_call(ids_off.data_ptr())),
    ]
    for name, kernel, fn in calls:
        fn()
        torch.cuda.synchronize()
        rounds = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(50):
                fn()
            b.record()
            torch.cuda.synchronize()
            rounds.append(a.elapsed_time(b) * 1e3 / 50)
        rounds.sort()
        res[name] = {"kernel": kernel, "us_median": round(rounds[len(rounds) // 2], 2),
                     "us_min": round(rounds[0], 2), "us_max": round(rounds[-1], 2)}
        print(f"ceilings: {name}: {rounds[len(rounds) // 2]:.2f} us", flush=True)
    for name, kernel, nbytes, fn in patterns:
        for i in range(4):
            fn(i % 2)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for r, (a, b) in enumerate(evs):
            a.record()
            fn(r % 2)
            b.record()
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
        med = us[len(us) // 2]
        res[name] = {"kernel": kernel, "bytes": int(nbytes), "us_median": round(med, 2),
                     "us_min": round(us[0], 2), "us_max": round(us[-1], 2),
                     "gbs": round(nbytes / med / 1e3, 1)}
        print(f"ceilings: {name}: {med:.2f} us, {nbytes / med / 1e3:.1f} GB/s", flush=True)
    return {"mode": "ceilings", "unit": "GB/s", "peak_gbs": HBM_PEAK_GBS, "reps": reps,
            "ceilings": res}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="prefill",
                    choices=["tiny", "decode", "prefill", "skewed", "large"])
    ap.add_argument("--sets", type=int, default=2, help="rotating buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ref", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the HIP-graph replay of the step")
    ap.add_argument("--epilogue", action="store_true",
                    help="combine with the fused residual add + RMSNorm epilogue "
                         "(moe_combine_epilogue) instead of the plain combine")
    ap.add_argument("--lowlatency", action="store_true",
                    help="time the low-latency form instead: padded per-expert layout, "
                         "bf16 -> e4m3 cast on dispatch, combine from the padded buffer")
    ap.add_argument("--rows-per-expert", type=int, default=0,
                    help="padded rows per expert for --lowlatency (default: N, no drops)")
    ap.add_argument("--scale-format", choices=list(SCALE_FORMATS), default="cols",
                    help="--lowlatency scales: rows, cols (column-major fp32) or ue8m0")
    ap.add_argument("--round-scale", action="store_true",
                    help="--lowlatency: round scales up to powers of two (implied by ue8m0)")
    ap.add_argument("--scales-staged", action="store_true",
                    help="low-latency cols/ue8m0: per-token scales (MOE_SCALE_TOKENS) placed by "
                         "moe_scatter_scales, instead of the one-call dispatch writing them")
    ap.add_argument("--fused", action="store_true",
                    help="layout and dispatch in one launch for small batches (N*K <= 8192): "
                         "moe_layout_dispatch, or with --lowlatency moe_dispatch_fp8_padded")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward instead: combine backward (grad_y, grad_w) + "
                         "dispatch backward (grad_x, weight gradients) on the forward's layout")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this "
                         "bench into profiles/traffic.json and exit (no GPU needed)")
    ap.add_argument("--traffic-command", default="",
                    help="the profiled command, recorded next to the figures")
    ap.add_argument("--write-requests-from", metavar="DIR",
                    help="summarize a rocprofv3 --pmc run of TCC_EA0_WRREQ, TCC_EA0_WRREQ_64B and "
                         "TCC_EA0_WRREQ_DRAM_CREDIT_STALL (SQLite output) and exit (no GPU needed)")
    ap.add_argument("--ceilings", action="store_true",
                    help="time the bandwidth ceilings of the kernels' memory patterns "
                         "(libmoe_ceilings.so) next to moe_dispatch and moe_combine, and exit")
    args = ap.parse_args()
    workload_key = args.config + (f"-lowlatency-{args.scale_format}" if args.lowlatency else
                                  "-backward" if args.backward else "")
    if args.fused:
        workload_key += "-fused"
    if args.scales_staged:
        workload_key += "-staged"
    if args.write_requests_from:
        summarize_write_requests(args.write_requests_from)
        return
    if args.traffic_from and args.ceilings:
        summarize_ceiling_traffic(*args.traffic_from)
        return
    if args.traffic_from:
        summarize_traffic(*args.traffic_from, workload_key, args.traffic_command)
        return
    if args.lowlatency + args.epilogue + args.backward > 1:
        raise SystemExit("--lowlatency, --epilogue and --backward are separate measurements")
    if args.scales_staged and (not args.lowlatency or args.fused or args.scale_format == "rows"):
        raise SystemExit("--scales-staged applies to the unfused low-latency step with cols or "
                         "ue8m0 scales")
    if args.fused and (args.epilogue or args.backward):
        raise SystemExit("--fused applies to the plain and the low-latency step")

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this path is measured on one GPU only (one GPU's share of expert "
              "parallelism, no collectives); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_moe_get_amd as mg
    import moe_workloads as mw

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.ceilings:
        result = ceilings(torch, mg, mw, max(args.steps, 5))
        # the 2 GiB copy that calibrates the FETCH_SIZE / WRITE_SIZE counters
        result["copy_ref_gbs"] = round(copy_bandwidth(torch), 1)
        print(json.dumps(result), flush=True)
        return
    wl = mw.make(args.config)
    y = wl.y()
    N, K, E, Hc = wl.N, wl.K, wl.E, wl.Hc
    P = wl.payload_bytes()
    R = N * K
    M = args.rows_per_expert or N
    round_scale = args.round_scale or args.scale_format == "ue8m0"
    staged = args.lowlatency and args.scale_format != "rows" and args.scales_staged
    if args.lowlatency:
        x = mw.make_x(N, 7168, wl.seed + 104729)
        sets = [LowLatencySet(torch, mg, wl, x, y, M, args.scale_format, round_scale, args.fused,
                              staged)
                for _ in range(max(1, args.sets))]
        names = ("layout", "dispatch", "combine")
        op_bytes = ll_algorithmic_bytes(N, K, E, M, 7168, Hc, R, args.scale_format)
        kernels = {"dispatch": "dispatch_fp8_kernel", "combine": combine_kernel_name(N, K, Hc)}
        if staged:
            # the codes kernel and the scale placement, each with its share of
            # the algorithmic bytes (the staging buffer's traffic is overhead)
            sb = R * (7168 // 128 if args.scale_format == "ue8m0" else 4 * (7168 // 128))
            names = ("layout", "dispatch", "scales", "combine")
            op_bytes = (op_bytes[0], op_bytes[1] - sb, sb, op_bytes[2])
            kernels = {"dispatch": "dispatch_fp8_kernel", "scales": "scatter_scales_kernel",
                       "combine": combine_kernel_name(N, K, Hc)}
        if args.fused:
            names = ("layout+dispatch", "combine")
            op_bytes = (op_bytes[0] + op_bytes[1], op_bytes[2])
            kernels = {"layout+dispatch": "dispatch_fp8_padded_kernel",
                       "combine": combine_kernel_name(N, K, Hc)}
    elif args.backward:
        rng = np.random.default_rng(wl.seed + 7)
        host = {"y": y, "grad_out": mw.make_y(N, Hc, wl.seed + 11),
                "grad_recv": mw.make_y(R, 7168, wl.seed + 13),
                "grad_recv_w": rng.standard_normal((R, K)).astype(np.float32)}
        sets = [BackwardSet(torch, mg, wl, host) for _ in range(max(1, args.sets))]
        names = ("combine_backward", "dispatch_backward")
        op_bytes = bwd_algorithmic_bytes(N, K, 7168, Hc, R)
        # the dispatch backward is the combine kernel in its unit-weight form
        # rows of at most 1024 vectors with K a multiple of 4 take the grouped
        # form (four pairs of a token per workgroup)
        grouped = Hc // 8 <= 1024 and K % 4 == 0
        kernels = {"combine_backward": "combine_backward_group_kernel" if grouped
                   else "combine_backward_kernel",
                   "dispatch_backward": combine_kernel_name(N, K, 7168)}
    else:
        sets = [BufferSet(torch, mg, wl, y, args.fused) for _ in range(max(1, args.sets))]
        names = ("layout", "dispatch", "combine")
        op_bytes = algorithmic_bytes(N, K, E, P, Hc, R, sets[0].cap, args.epilogue)
        kernels = {"dispatch": "dispatch_kernel",
                   "combine": "combine_epilogue_kernel" if args.epilogue
                   else combine_kernel_name(N, K, Hc)}
        if args.fused:
            names = ("layout+dispatch", "combine")
            op_bytes = (op_bytes[0] + op_bytes[1], op_bytes[2])
            kernels = {"layout+dispatch": "layout_dispatch_kernel",
                       "combine": combine_kernel_name(N, K, Hc)}
    nops = len(names)
    stream = torch.cuda.current_stream()
    calls = [s.calls(mg, wl, stream.cuda_stream, args.epilogue) for s in sets]

    def step(i):
        for fn, a in calls[i % len(calls)]:
            rc = fn(*a)
            if rc != 0:
                raise mg.MoeError(rc, mg._lib.moe_last_error().decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    hev = HipEvents(torch)
    sh = stream.cuda_stream

    def timed_pass(op_events):
        """K steps between two synchronizations; with op_events, a
        timing-only event is also recorded before and after every op.
        Returns the mean step time and, with op_events, the per-step op
        times [K, ops]."""
        ev = [[hev.create() for _ in range(nops + 1)] for _ in range(args.steps)] if op_events else None
        t0, t1 = hev.create(), hev.create()
        torch.cuda.synchronize()
        hev.record(t0, sh)
        for i in range(args.steps):
            if op_events:
                hev.record(ev[i][0], sh)
            for j, (fn, a) in enumerate(calls[i % len(calls)]):
                if fn(*a) != 0:
                    raise mg.MoeError(-6, mg._lib.moe_last_error().decode())
                if op_events:
                    hev.record(ev[i][j + 1], sh)
        hev.record(t1, sh)
        torch.cuda.synchronize()
        step_ms = hev.ms(t0, t1) / args.steps
        op = None
        if op_events:
            op = np.array([[hev.ms(e[j], e[j + 1]) for j in range(nops)] for e in ev])
        return step_ms, op

    # The headline figure: whole steps, nothing recorded between the ops.
    ms_per_step, _ = timed_pass(False)
    # Per-op times (and the roofline kernel's duration) from a second timed
    # pass with an event between the ops.
    ms_per_step_op_events, op_all = timed_pass(True)
    op_ms = op_all.mean(axis=0)

    # The same steps captured once in a HIP graph (one step per buffer set)
    # and replayed: the launch cost the host pays per op drops out.
    graph_ms = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            cs = torch.cuda.current_stream().cuda_stream
            gcalls = [st.calls(mg, wl, cs, args.epilogue) for st in sets]
            for c in gcalls:
                for fn, a in c:
                    if fn(*a) != 0:
                        raise mg.MoeError(-6, mg._lib.moe_last_error().decode())
        reps = max(1, args.steps // len(sets))
        for _ in range(2):
            g.replay()
        t0, t1 = hev.create(), hev.create()
        torch.cuda.synchronize()
        hev.record(t0, sh)
        for _ in range(reps):
            g.replay()
        hev.record(t1, sh)
        torch.cuda.synchronize()
        graph_ms = hev.ms(t0, t1) / (reps * len(sets))
        del g, gcalls
    hev.close()

    total = sum(op_bytes)
    value = total / (ms_per_step * 1e-3) / 1e9
    # the roofline is taken on the longest of the streaming kernels
    rop = max((j for j, n in enumerate(names) if n in kernels), key=lambda j: op_ms[j])
    rkernel, rbytes = kernels[names[rop]], op_bytes[rop]
    roof_gbs = rbytes / (op_ms[rop] * 1e-3) / 1e9
    traffic = traffic_entry(rkernel, workload_key)
    if args.lowlatency:
        workload = (f"{args.config} low-latency{' (layout and dispatch fused)' if args.fused else ''}: "
                    f"N={N} tokens, top-{K} of {E} experts, padded "
                    f"{M} rows per expert, bf16 hidden 7168 cast to e4m3 on dispatch with "
                    f"{args.scale_format} scales per 128 channels"
                    + (" (power-of-two)" if round_scale else "")
                    + (" staged per token and placed by expert row" if staged else "")
                    + f", combine bf16 hidden {Hc}, fp32 accumulation")
        metric = ("low-latency dispatch (fp8 cast) + combine effective HBM GB/s and tokens/s, "
                  f"{N}×7168 top-{K}, 1 GPU")
    elif args.backward:
        workload = (f"{args.config} backward: N={N} tokens, top-{K} of {E} experts, combine "
                    f"backward (bf16 grad_out {Hc} -> grad_y rows, fp32 weight gradients from y) "
                    f"+ dispatch backward (bf16 grad rows 7168 -> grad_x, fp32 top-{K} weight "
                    f"gradient rows -> grad_w)")
        metric = ("combine backward + dispatch backward effective HBM GB/s and tokens/s, "
                  f"{N}×7168 top-{K}, 1 GPU")
    else:
        workload = (f"{args.config}{' (layout and dispatch fused)' if args.fused else ''}: "
                    f"N={N} tokens, top-{K} of {E} experts, dispatch payload "
                    f"{P} B/token ({', '.join(f'{n} {a.shape[1]} B' for n, a in wl.fields) or 'one record: ids, weights, 3584 B hidden, 448 B scales; ids and weights read in place'}), "
                    f"combine bf16 hidden {Hc}, fp32 accumulation"
                    + (", fused residual add + RMSNorm epilogue" if args.epilogue else ""))
        metric = METRIC if args.config == "prefill" else (
            f"dispatch+combine effective HBM GB/s and tokens/s, {N}×{Hc} top-{K}, 1 GPU")

    result = {
        "metric": metric,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": workload,
            "tokens": N, "topk": K, "experts": E, "hidden": Hc,
            "payload_bytes": (7168 * 2 if args.lowlatency or args.backward else P),
            "buffer_sets": len(sets), "algorithmic_bytes_per_step": total,
        },
        "tokens_per_s": round(N / (ms_per_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "ms_per_step_with_op_events": round(ms_per_step_op_events, 5),
        "ms_per_step_graph": None if graph_ms is None else round(graph_ms, 5),
        "per_op_us_p10_p50_p90": {
            name: [round(float(np.percentile(op_all[:, j], q)) * 1e3, 2) for q in (10, 50, 90)]
            for j, name in enumerate(names)},
        "per_op_us": {name: round(op_ms[j] * 1e3, 2) for j, name in enumerate(names)},
        "per_op_gbs": {name: round(op_bytes[j] / (op_ms[j] * 1e-3) / 1e9, 1)
                       for j, name in enumerate(names)},
        "roofline": {
            "kernel": rkernel,
            "bound": "hbm",
            "achieved": round(roof_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "algorithmic_bytes_per_launch": rbytes,
        },
    }
    if not args.no_copy_ref:
        result["copy_ref_gbs"] = round(copy_bandwidth(torch), 1)
    if args.lowlatency:
        result["config"]["rows_per_expert"] = M
        result["config"]["scale_format"] = args.scale_format
    if not args.no_cpu_baseline:
        if args.lowlatency:
            result["cpu_baseline"] = cpu_baseline_ll(wl, x, y, M, args.scale_format, round_scale,
                                                     total, args.cpu_seconds)
        elif args.backward:
            result["cpu_baseline"] = cpu_baseline_bwd(wl, host, total, args.cpu_seconds)
        else:
            ep = None
            if args.epilogue:
                bits = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)
                ep = (bits(sets[0].residual), bits(sets[0].gamma))
            result["cpu_baseline"] = cpu_baseline(wl, y, total, args.cpu_seconds, ep)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
