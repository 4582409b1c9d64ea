"""Host-side logic of bench.py (CPU only): the one-GPU refusal, the
algorithmic byte counts the throughput figures divide by, the HBM-counter
calibration and the source-hash check that keeps stale counters out of the
JSON line."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus must be 1" in r.stderr


def test_prefill_algorithmic_bytes():
    # N=4096, K=8, E=256, P=7456 (7168 fp8 + 224 scales + 32 ids + 32 weights),
    # Hc=7168, R=N*K, cap=R
    N, K, E, P, Hc = 4096, 8, 256, 7456, 7168
    R = N * K
    layout, dispatch, combine = bench.algorithmic_bytes(N, K, E, P, Hc, R, R)
    assert layout == 4 * R + 8 * E + 4 + 4 * R + 4 * R == 395268
    assert dispatch == N * P + 4 * R + R * P == 274989056
    assert combine == R * Hc * 2 + 8 * R + N * Hc * 2 == 528744448
    assert round((layout + dispatch + combine) / 1e6, 1) == 804.1
    _, _, epi = bench.algorithmic_bytes(N, K, E, P, Hc, R, R, epilogue=True)
    assert epi == combine + 2 * N * Hc * 2 + Hc * 2 == 646199296


def test_low_latency_and_backward_bytes():
    N, K, E, M, H, Hc = 4096, 8, 256, 4096, 7168, 7168
    R = N * K
    lay, rows, com = bench.ll_algorithmic_bytes(N, K, E, M, H, Hc, R, "rows")
    assert lay == 4 * R + 4 * E + 4 * R + 4 * E * M + 8 == 4457480
    assert rows == 2 * N * H + 4 * R + R * (H + 4 * H // 128) == 301072384
    assert bench.ll_algorithmic_bytes(N, K, E, M, H, Hc, R, "cols")[1] == rows
    assert bench.ll_algorithmic_bytes(N, K, E, M, H, Hc, R, "ue8m0")[1] == 295567360
    cb, db = bench.bwd_algorithmic_bytes(N, K, H, Hc, R)
    assert cb == 998637568 and db == 529793024


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_calibration_and_hash_check(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE are scaled by what they read for the 2 GiB
    copy; an entry is reported only for the kernel source it was taken on."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy = bench.COPY_BYTES / 1024                      # KiB per copy launch
    k = "void moe::(anonymous namespace)::combine_kernel<4, false>(args)"
    fetch = [{"Kernel_Name": bench.COPY_KERNEL, "Counter_Name": "FETCH_SIZE",
              "Counter_Value": copy / 2} for _ in range(3)]
    fetch += [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
               "Counter_Value": 1.0}]                   # a small upload: ignored
    fetch += [{"Kernel_Name": k, "Counter_Name": "FETCH_SIZE", "Counter_Value": v}
              for v in (1000.0, 1002.0)]
    write = [{"Kernel_Name": bench.COPY_KERNEL, "Counter_Name": "WRITE_SIZE",
              "Counter_Value": copy} for _ in range(3)]
    write += [{"Kernel_Name": k, "Counter_Name": "WRITE_SIZE", "Counter_Value": 100.0}] * 2
    # a kernel whose name contains another's is not counted as that one
    ld = "void moe::(anonymous namespace)::layout_dispatch_kernel<unsigned int __vector(4)>(a)"
    d = "void moe::(anonymous namespace)::dispatch_kernel<unsigned int __vector(4)>(a)"
    fetch += [{"Kernel_Name": ld, "Counter_Name": "FETCH_SIZE", "Counter_Value": 7.0},
              {"Kernel_Name": d, "Counter_Name": "FETCH_SIZE", "Counter_Value": 3.0}]
    write += [{"Kernel_Name": ld, "Counter_Name": "WRITE_SIZE", "Counter_Value": 5.0},
              {"Kernel_Name": d, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1.0}]
    _counter_csv(str(tmp_path / "f"), fetch)
    _counter_csv(str(tmp_path / "w"), write)
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "wl", "cmd")
    data = json.load(open(tmp_path / "traffic.json"))
    e = data["combine_kernel/wl"]
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0
    assert e["bytes_per_launch"] == int((1001.0 * 2 + 100.0) * 1024)
    assert e["launches"] == 2 and e["command"] == "cmd"
    assert data["dispatch_kernel/wl"]["bytes_per_launch"] == int((3.0 * 2 + 1.0) * 1024)
    assert data["layout_dispatch_kernel/wl"]["bytes_per_launch"] == int((7.0 * 2 + 5.0) * 1024)
    assert bench.traffic_entry("combine_kernel", "wl") == e
    e["source_sha256_16"] = "0" * 16                    # counters of another source
    json.dump(data, open(tmp_path / "traffic.json", "w"))
    assert bench.traffic_entry("combine_kernel", "wl") is None
    assert bench.traffic_entry("combine_kernel", "other") is None


def test_copy_launches_must_agree(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    copy = bench.COPY_BYTES / 1024
    bad = [{"Kernel_Name": bench.COPY_KERNEL, "Counter_Name": "FETCH_SIZE", "Counter_Value": v}
           for v in (copy / 2, copy / 2, copy)]
    ok = [{"Kernel_Name": bench.COPY_KERNEL, "Counter_Name": "WRITE_SIZE", "Counter_Value": copy}] * 3
    _counter_csv(str(tmp_path / "f"), bad)
    _counter_csv(str(tmp_path / "w"), ok)
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), "wl", "cmd")


def test_source_hash_ignores_comments_not_code(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\n__global__ void k(int* p) {\n    p[0] = 1;  /* one */\n}\n")
    h = bench.source_hash(str(a))
    a.write_text("// another header\n\n__global__ void k(int* p) {\n  p[0] = 1;  // one\n}\n")
    assert bench.source_hash(str(a)) == h
    a.write_text("// header\n__global__ void k(int* p) {\n    p[0] = 2;  /* one */\n}\n")
    assert bench.source_hash(str(a)) != h


def test_kernel_names_keep_template_arguments():
    k = bench.kernel_name_with_args
    assert k("void (anonymous namespace)::read_kernel<true, 1>(unsigned int __vector(4) const*, "
             "long, unsigned int*)") == "read_kernel<true, 1>"
    assert k("(anonymous namespace)::mix_kernel(unsigned int __vector(4) const*, long, int)") == \
        "mix_kernel"
    assert k("void moe::(anonymous namespace)::combine_kernel<4, false, false>(unsigned short "
             "const*, long)") == "combine_kernel<4, false, false>"
    assert k("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_write_request_summary(tmp_path, capsys):
    """Per-channel counter rows of a rocprofv3 database become requests per
    launch, the 64-byte share, bytes, and the channel spread."""
    import sqlite3

    con = sqlite3.connect(tmp_path / "q_results.db")
    con.execute("create table pmc_events (id integer primary key, dispatch_id int, name text, "
                "counter_name text, counter_value real)")
    name = "void moe::(anonymous namespace)::dispatch_kernel<int>(Args)"
    rows = []
    for disp in (1, 2):
        for ch in range(128):
            rows += [(disp, name, "TCC_EA0_WRREQ", 100.0 + ch % 2),
                     (disp, name, "TCC_EA0_WRREQ_64B", 90.0),
                     (disp, name, "TCC_EA0_WRREQ_DRAM_CREDIT_STALL", float(ch))]
    con.executemany("insert into pmc_events (dispatch_id, name, counter_name, counter_value) "
                    "values (?, ?, ?, ?)", rows)
    con.commit()
    con.close()
    bench.summarize_write_requests(str(tmp_path))
    out = capsys.readouterr().out.splitlines()
    line = next(l for l in out if l.startswith("| dispatch_kernel<int>"))
    cells = [c.strip() for c in line.strip("|").split("|")]
    req = 64 * 100 + 64 * 101
    b64 = 128 * 90
    assert cells[1] == "2" and cells[2] == str(req)
    assert cells[3] == f"{b64 / req:.3f}"
    assert cells[4] == f"{(64 * b64 + 32 * (req - b64)) / 1e6:.2f}"
    assert cells[5] == "100 / 100 / 101" and cells[6] == "0 / 64 / 127"


def test_combine_kernel_name_follows_the_held_form_rule():
    """bench.py names the kernel moe_combine runs: the held form past 32768
    waves with K <= 8 and 8 to 224 segments of 64 16-byte vectors per row."""
    import bench

    assert bench.combine_kernel_name(4096, 8, 7168) == "combine_held_kernel"    # 57344 waves
    assert bench.combine_kernel_name(4096, 8, 4096) == "combine_kernel"         # 32768 waves
    assert bench.combine_kernel_name(4097, 8, 4096) == "combine_held_kernel"
    assert bench.combine_kernel_name(4097, 9, 4096) == "combine_kernel"         # K > 8
    assert bench.combine_kernel_name(40000, 8, 3584) == "combine_kernel"        # 7 segments
    assert bench.combine_kernel_name(147, 3, 114688) == "combine_held_kernel"   # 224 segments
    assert bench.combine_kernel_name(150, 2, 115200) == "combine_kernel"        # 225 segments
    assert bench.combine_kernel_name(128, 8, 7168) == "combine_kernel"          # decode
