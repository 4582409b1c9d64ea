"""Builds tests/c_abi/abi_check: the C ABI exercised from plain C and
checked against the CPU oracle (test infrastructure; needs the library and
the oracle built first)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
BIN = os.path.join(HERE, "abi_check")


def build(out: str = BIN) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(HERE, "abi_check.c"), "-o", out,
           "-L", os.path.join(ROOT, "combine_moe_get_amd"), "-lmoe_get",
           "-L", os.path.join(ROOT, "oracle"), "-loracle", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath," + ":".join([os.path.join(ROOT, "combine_moe_get_amd"),
                                     os.path.join(ROOT, "oracle"), "/opt/rocm/lib"])]
    subprocess.check_call(cmd)
    return out


if __name__ == "__main__":
    print(build())
