"""Builds tests/fp8_encode/fp8_encode_check: the FP8 dispatch's e4m3fn
encoder checked on every fp32 input (test infrastructure)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "fp8_encode_check")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(out: str = BIN) -> str:
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "combine_moe_get_amd", "csrc"),
           os.path.join(HERE, "fp8_encode_check.hip"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"fp8_encode_check build failed:\n{r.stderr}")
    return out


if __name__ == "__main__":
    print(build())
