"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

A private copy of oracle/ is built with -fsanitize=address,undefined (every
finding fatal) and the oracle's pin files run against it in a child Python
with the ASan runtime preloaded: an out-of-bounds access, a use after free,
signed overflow, a bad shift or a misaligned access anywhere the pins reach
aborts the run. Two more cases plant an out-of-bounds write and a signed
overflow in copies to show that the harness reports each. CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
PINS = ["test_oracle_layout.py", "test_oracle_dispatch.py", "test_oracle_combine.py",
        "test_oracle_epilogue.py", "test_oracle_lowlatency.py", "test_oracle_backward.py",
        "test_oracle_threads.py"]
SAN_FLAGS = '"-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", ' \
            '"-fno-sanitize-recover=all",'


def _libasan():
    try:
        p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                           text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return p if os.path.isabs(p) and os.path.exists(p) else None


LIBASAN = _libasan()
pytestmark = pytest.mark.skipif(LIBASAN is None, reason="gcc's AddressSanitizer runtime not found")


def _sanitized_copy(tmp_path, src_edit=None):
    d = tmp_path / "san"
    pkg = d / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    init = (pkg / "__init__.py").read_text()
    site = 'cmd = ["gcc", "-O2",'
    assert init.count(site) == 1, "oracle build command not found"
    (pkg / "__init__.py").write_text(init.replace(site, 'cmd = ["gcc", ' + SAN_FLAGS))
    if src_edit is not None:
        src = (pkg / "moe_oracle.c").read_text()
        old, new = src_edit
        assert src.count(old) == 1
        (pkg / "moe_oracle.c").write_text(src.replace(old, new))
    return d


def _run(d, pin_files):
    env = dict(os.environ, ORACLE_DIR=str(d), OMP_NUM_THREADS="2", LD_PRELOAD=LIBASAN,
               ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    # -s: a sanitizer report is written to the child's stderr as the process
    # ends, which pytest's own output capture would swallow. The slow
    # full-size thread test runs the unsanitized oracle in a child of its own.
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-m",
                           "not gpu and not slow",
                           "-p", "no:cacheprovider"] + [os.path.join(TESTS, f) for f in pin_files],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_oracle_pins_pass_under_sanitizers(tmp_path):
    d = _sanitized_copy(tmp_path)
    r = _run(d, PINS)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "Sanitizer" not in r.stderr, out
    so = d / "oracle" / "liboracle.so"
    deps = subprocess.run(["ldd", str(so)], capture_output=True, text=True).stdout
    assert "libasan" in deps and "libubsan" in deps, deps


PLANTED = [
    # (helper planted before oracle_required_cap, statement at the top of
    #  oracle_layout, words the report must hold)
    ("static void oob(int32_t* c, int32_t E) { c[E] = 0; }\n", "oob(counts, E);",
     ["AddressSanitizer", "heap-buffer-overflow"]),
    ("static int32_t add(int32_t a, int32_t b) { return a + b; }\n",
     "{ volatile int32_t big = 2147483647; if (add(big, E) == 0) return ORC_ERR_ARG; }",
     ["runtime error", "signed integer overflow"]),
]


@pytest.mark.parametrize("helper,stmt,words", PLANTED, ids=["write past counts", "int32 overflow"])
def test_planted_error_is_reported(tmp_path, helper, stmt, words):
    d = _sanitized_copy(tmp_path, ("int64_t oracle_required_cap(",
                                   helper + "int64_t oracle_required_cap("))
    src = (d / "oracle" / "moe_oracle.c").read_text()
    i = src.index("int oracle_layout(const int32_t* ids,")
    body = src.index("{", i) + 1
    (d / "oracle" / "moe_oracle.c").write_text(src[:body] + "\n    " + stmt + src[body:])
    r = _run(d, ["test_oracle_layout.py"])
    assert r.returncode != 0
    for w in words:
        assert w in r.stderr, r.stderr[-3000:]
