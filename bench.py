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
COMBINE_SRC = os.path.join(ROOT, "combine_moe_get_amd", "csrc", "combine.hip")


def algorithmic_bytes(N, K, E, P, Hc, R, cap):
    """Bytes each op must move at minimum: every input read once, every
    output written once."""
    layout = 4 * N * K + 8 * E + 4 + 4 * N * K + 4 * cap
    dispatch = N * P + 4 * N * K + R * P
    combine = R * Hc * 2 + 8 * N * K + N * Hc * 2
    return layout, dispatch, combine


def source_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_entry(kernel, workload):
    """Measured HBM bytes per launch for `kernel` on `workload`, if the
    counters were taken on the current kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(f"{kernel}/{workload}")
    if not e or e.get("source_sha256_16") != source_hash(COMBINE_SRC):
        return None
    return e


class BufferSet:
    """Device inputs and outputs of one step."""

    def __init__(self, torch, mg, wl, y_bits):
        d = "cuda"
        self.ids = torch.from_numpy(np.ascontiguousarray(wl.ids)).to(d)
        self.w = torch.from_numpy(np.ascontiguousarray(wl.weights)).to(d)
        self.srcs = [torch.from_numpy(a).to(d) for _, a in wl.fields]
        self.y = torch.from_numpy(y_bits.view(np.int16)).to(d).view(torch.bfloat16)
        N, K, E = wl.N, wl.K, wl.E
        self.cap = cap = mg.moe_required_capacity(N, K, E, 1)
        self.counts = torch.empty(E, dtype=torch.int32, device=d)
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=d)
        self.pos = torch.empty((N, K), dtype=torch.int32, device=d)
        self.row_pair = torch.empty(cap, dtype=torch.int32, device=d)
        self.status = torch.empty(1, dtype=torch.int32, device=d)
        self.ws = torch.empty(mg.moe_layout_workspace_bytes(N, K, E), dtype=torch.uint8, device=d)
        self.dsts = [torch.empty((cap, a.shape[1]), dtype=torch.uint8, device=d) for a in self.srcs]
        self.out = torch.empty((N, wl.Hc), dtype=torch.bfloat16, device=d)

    def calls(self, mg, wl, stream):
        """Argument tuples of the three C-ABI calls, marshalled once."""
        L = mg._lib
        N, K, E = wl.N, wl.K, wl.E
        fields = (mg.moe_field * len(self.srcs))()
        for i, (s, t) in enumerate(zip(self.srcs, self.dsts)):
            fields[i] = mg.moe_field(s.data_ptr(), s.stride(0), t.data_ptr(), t.stride(0), s.shape[1])
        self._fields = fields
        lay = (self.ids.data_ptr(), K, N, K, E, 1, self.counts.data_ptr(), self.offsets.data_ptr(),
               self.pos.data_ptr(), self.row_pair.data_ptr(), self.cap, self.ws.data_ptr(),
               self.ws.numel(), self.status.data_ptr(), stream)
        dis = (fields, len(self.srcs), N, K, self.pos.data_ptr(), stream)
        com = (self.y.data_ptr(), wl.Hc, self.w.data_ptr(), K, self.pos.data_ptr(), N, K, wl.Hc,
               self.out.data_ptr(), wl.Hc, stream)
        return (L.moe_get_layout, lay), (L.moe_dispatch, dis), (L.moe_combine, com)


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


def cpu_baseline(wl, y, total_bytes, budget_s):
    """The oracle as it stands, on the host cores: full steps of the same
    workload (layout serial, dispatch and combine OpenMP over tokens) until
    `budget_s` seconds of work are done."""
    import oracle

    srcs = [a for _, a in wl.fields]
    w = np.ascontiguousarray(wl.weights)
    dsts = [np.empty((wl.N * wl.K, a.shape[1]), np.uint8) for a in srcs]

    def one():
        _, _, pos, _, _ = oracle.layout(wl.ids, wl.E)
        oracle.dispatch(srcs, pos, wl.K, dsts=dsts)
        oracle.combine(y, w, pos)

    one()   # warm host caches and page in outputs
    times = []
    t_all = time.perf_counter()
    while not times or (time.perf_counter() - t_all < budget_s and len(times) < 50):
        t0 = time.perf_counter()
        one()
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {
        "value": round(total_bytes / t / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{len(times)} full {wl.name} steps (layout+dispatch+combine), median "
                  f"{t * 1e3:.1f} ms/step, {wl.N / t:.0f} tokens/s",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="prefill",
                    choices=["tiny", "decode", "prefill", "skewed"])
    ap.add_argument("--sets", type=int, default=2, help="rotating buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-ref", action="store_true")
    args = ap.parse_args()

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
    wl = mw.make(args.config)
    y = wl.y()
    N, K, E, Hc = wl.N, wl.K, wl.E, wl.Hc
    P = wl.payload_bytes()
    R = N * K
    sets = [BufferSet(torch, mg, wl, y) for _ in range(max(1, args.sets))]
    stream = torch.cuda.current_stream()
    calls = [s.calls(mg, wl, stream.cuda_stream) for s in sets]

    def step(i):
        for fn, a in calls[i % len(calls)]:
            rc = fn(*a)
            if rc != 0:
                raise mg.MoeError(rc, mg._lib.moe_last_error().decode())

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        fns = calls[i % len(calls)]
        e = ev[i]
        e[0].record(stream)
        for j, (fn, a) in enumerate(fns):
            if fn(*a) != 0:
                raise mg.MoeError(-6, mg._lib.moe_last_error().decode())
            e[j + 1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    per_op = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(3)] for e in ev])  # ms
    op_ms = per_op.mean(axis=0)

    b_lay, b_dis, b_com = algorithmic_bytes(N, K, E, P, Hc, R, sets[0].cap)
    total = b_lay + b_dis + b_com
    value = total / (ms_per_step * 1e-3) / 1e9
    combine_gbs = b_com / (op_ms[2] * 1e-3) / 1e9
    traffic = traffic_entry("combine_kernel", args.config)

    result = {
        "metric": METRIC,
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
            "workload": f"{args.config}: N={N} tokens, top-{K} of {E} experts, dispatch payload "
                        f"{P} B/token ({', '.join(f'{n} {a.shape[1]} B' for n, a in wl.fields)}), "
                        f"combine bf16 hidden {Hc}, fp32 accumulation",
            "tokens": N, "topk": K, "experts": E, "hidden": Hc, "payload_bytes": P,
            "buffer_sets": len(sets), "algorithmic_bytes_per_step": total,
        },
        "tokens_per_s": round(N / (ms_per_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "per_op_us": {"layout": round(op_ms[0] * 1e3, 2), "dispatch": round(op_ms[1] * 1e3, 2),
                      "combine": round(op_ms[2] * 1e3, 2)},
        "per_op_gbs": {"layout": round(b_lay / (op_ms[0] * 1e-3) / 1e9, 1),
                       "dispatch": round(b_dis / (op_ms[1] * 1e-3) / 1e9, 1),
                       "combine": round(combine_gbs, 1)},
        "roofline": {
            "kernel": "combine_kernel",
            "bound": "hbm",
            "achieved": round(combine_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(combine_gbs / HBM_PEAK_GBS, 4),
            "traffic": None if traffic is None else traffic["bytes_per_launch"],
            "algorithmic_bytes_per_launch": b_com,
        },
    }
    if not args.no_copy_ref:
        result["copy_ref_gbs"] = round(copy_bandwidth(torch), 1)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, y, total, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
