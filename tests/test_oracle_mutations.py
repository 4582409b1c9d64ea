"""The pins must catch plausible mistakes in the oracle: each case plants one
mistake in a private copy of oracle/moe_oracle.c (a dropped term, a wrong
order, index or rounding), builds it, and runs the pin file that covers that
function against the copy. Every planted mistake must make that file fail;
the unmodified copy must pass one of them (so a failure is the mistake's,
not the harness's)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")

# (name, text in moe_oracle.c, replacement, pin file)
MUTANTS = [
    ("layout ignores align",
     "int32_t padded = (counts[e] + align - 1) / align * align;",
     "int32_t padded = counts[e];", "test_oracle_layout.py"),
    ("layout reverses rows inside a segment",
     "                p = cursor[e];\n                cursor[e] += 1;",
     "                p = 2 * offsets[e] + counts[e] - 1 - cursor[e];\n                cursor[e] += 1;",
     "test_oracle_layout.py"),
    ("layout does not count ids >= E",
     "if (e >= E) { ++bad; continue; }", "if (e >= E) { continue; }", "test_oracle_layout.py"),
    ("dispatch copies the wrong token",
     "(const char*)d->src + (int64_t)t * d->src_row_stride",
     "(const char*)d->src + (int64_t)(pos ? (t + k) % N : t) * d->src_row_stride",
     "test_oracle_dispatch.py"),
    ("bf16 rounding ties away from zero",
     "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;", "test_oracle_combine.py"),
    ("combine uses multiply then add",
     "acc = fmaf(w[(int64_t)t * w_row_stride + k], yv, acc);",
     "acc = w[(int64_t)t * w_row_stride + k] * yv + acc;", "test_oracle_combine.py"),
    ("combine sums k descending",
     "    float acc = 0.0f;\n    for (int32_t k = 0; k < K; ++k) {\n        int32_t p = pos[(int64_t)t * K + k];",
     "    float acc = 0.0f;\n    for (int32_t k = K - 1; k >= 0; --k) {\n        int32_t p = pos[(int64_t)t * K + k];",
     "test_oracle_combine.py"),
    ("rmsnorm adds eps outside the root",
     "double scale = 1.0 / sqrt(ss / (double)Hc + (double)eps);",
     "double scale = 1.0 / (sqrt(ss / (double)Hc) + (double)eps);", "test_oracle_epilogue.py"),
    ("e4m3 truncates",
     "double r = rint(m / q) * q;         /* exact */",
     "double r = floor(m / q) * q;         /* exact */", "test_oracle_lowlatency.py"),
    ("fp8 scale uses the wrong maximum",
     "float s = amax / 448.0f;", "float s = amax / 240.0f;", "test_oracle_lowlatency.py"),
    ("round_scale rounds down",
     "s = (g == 0.5f) ? s : ldexpf(1.0f, e);", "s = (g == 0.5f) ? s : ldexpf(1.0f, e - 1);",
     "test_oracle_lowlatency.py"),
    ("round_scale rounds an infinite scale",
     "if (round_scale && isfinite(s)) {", "if (round_scale) {", "test_oracle_lowlatency.py"),
    ("padded layout keeps pairs past M",
     "if (counts[e] < M) {", "if (counts[e] <= M && e * M + counts[e] < E * M) {",
     "test_oracle_lowlatency.py"),
    ("scale scatter takes the pair's index as the token",
     "const float* ts = token_scales + (int64_t)(r / K) * token_scale_row_stride;",
     "const float* ts = token_scales + (int64_t)(r % N) * token_scale_row_stride;",
     "test_oracle_lowlatency.py"),
    ("scale scatter transposes blocks and rows",
     "((float*)scales)[((int64_t)e * nb + b) * M + m] = ts[b];",
     "((float*)scales)[((int64_t)e * M + m) * nb + b] = ts[b];", "test_oracle_lowlatency.py"),
    ("token scales skip tokens without a pair",
     "        if (scale_mode == 3)\n            for (int32_t b = 0; b < nb; ++b)",
     "        if (scale_mode == 3 && pos[(int64_t)t * K] >= 0)\n            for (int32_t b = 0; b < nb; ++b)",
     "test_oracle_lowlatency.py"),
    ("receive range swaps begin and count",
     "if (layout_range) layout_range[e] = (begin << 32) | count;",
     "if (layout_range) layout_range[e] = (count << 32) | begin;", "test_oracle_lowlatency.py"),
    ("receive stats overwritten instead of added",
     "if (recv_stats) recv_stats[e] += counts[e];",
     "if (recv_stats) recv_stats[e] = counts[e];", "test_oracle_lowlatency.py"),
    ("combine backward scales by the first weight",
     "float wk = w[(int64_t)t * w_row_stride + k];", "float wk = w[(int64_t)t * w_row_stride];",
     "test_oracle_backward.py"),
    ("combine backward forms the dot product in fp32",
     "double dot = 0.0;", "float dot = 0.0f;", "test_oracle_backward.py"),
    ("dispatch backward transposes the weight-gradient index",
     "acc = acc + grad_recv_w[(int64_t)p * grad_recv_w_row_stride + j];",
     "acc = acc + grad_recv_w[(int64_t)p * grad_recv_w_row_stride + k];", "test_oracle_backward.py"),
]


def _run_pins(tmp_path, name, src_text, pin_file):
    d = tmp_path / name.replace(" ", "_")
    pkg = d / "oracle"
    shutil.copytree(os.path.join(ROOT, "oracle"), pkg,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    (pkg / "moe_oracle.c").write_text(src_text)
    env = dict(os.environ, ORACLE_DIR=str(d), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", os.path.join(TESTS, pin_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r


def test_unmodified_copy_passes(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "moe_oracle.c")).read()
    r = _run_pins(tmp_path, "unmodified", src, "test_oracle_backward.py")
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new,pin_file", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, pin_file):
    src = open(os.path.join(ROOT, "oracle", "moe_oracle.c")).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    r = _run_pins(tmp_path, name, src.replace(old, new), pin_file)
    assert r.returncode == 1, f"{name}: pins in {pin_file} did not fail\n{r.stdout[-2000:]}"
    # the copy built and loaded; a pin's assertion is what failed
    assert "CalledProcessError" not in r.stdout and "AssertionError" in r.stdout, r.stdout[-2000:]
