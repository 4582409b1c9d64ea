"""The FP8 dispatch's e4m3fn encoder (fp8.hpp: the correctly rounded
quotient, clamped to +-448, converted by gfx950's v_cvt_pk_fp8_f32, NaN
mapped to 0x7F) equals the bit-level definition of the cast on all 2^32 fp32
inputs, in every byte position (tests/fp8_encode/fp8_encode_check.hip, built
by __graft_entry__.build())."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fp8_encode", "fp8_encode_check")


def test_encoder_on_every_fp32_input():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build()"
    print("[gpu-fp8-encode] running fp8_encode_check", flush=True)
    sys.stdout.flush()
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0 and "mismatches: 0" in r.stdout, r.stdout + r.stderr
