"""The C-ABI library loads and exports every symbol include/*.h declares, and
argument validation rejects bad calls before anything touches a GPU (CPU
only: none of these calls reaches a launch)."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("moe_get_layout", "moe_dispatch", "moe_combine", "moe_layout_workspace_bytes",
              "moe_required_capacity", "moe_last_error", "moe_version"):
        assert n in names


@pytest.mark.parametrize("name", ["libmoe_get.so", "libmoe_get_debug.so"])
def test_library_exports_every_declared_symbol(name):
    """The release library and its debug build (MOE_DEBUG) both export every
    declared entry point."""
    import combine_moe_get_amd as m

    path = os.path.join(os.path.dirname(m.__file__), name)
    lib = ctypes.CDLL(path)
    for n in _declared_functions():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared_functions()) <= exported


def test_debug_build_is_selected_by_the_environment():
    """MOE_DEBUG=1 makes the binding load libmoe_get_debug.so (checked in a
    child process, which only imports the package)."""
    code = ("import combine_moe_get_amd as m, os; "
            "print(os.path.basename(m.LIB_PATH), m.DEBUG)")
    for env_value, expect in (("1", "libmoe_get_debug.so True"), ("", "libmoe_get.so False")):
        env = dict(os.environ, MOE_DEBUG=env_value)
        r = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env,
                           cwd=ROOT, timeout=300)
        assert r.returncode == 0, r.stderr
        assert r.stdout.strip().splitlines()[-1] == expect


def test_debug_status_release_and_debug_argument_errors():
    """moe_debug_status: the release build refuses (MOE_ERR_LIMIT); the debug
    build rejects a NULL out before touching a GPU."""
    import combine_moe_get_amd as m

    pkg = os.path.dirname(m.__file__)
    for name, code in (("libmoe_get.so", m.MOE_ERR_LIMIT), ("libmoe_get_debug.so", m.MOE_ERR_ARG)):
        L = ctypes.CDLL(os.path.join(pkg, name))
        L.moe_debug_status.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
        L.moe_last_error.restype = ctypes.c_char_p
        buf = (ctypes.c_int32 * 5)()
        out = None if name.endswith("debug.so") else ctypes.cast(buf, ctypes.c_void_p)
        assert L.moe_debug_status(out, 0, None) == code
        assert b"moe_debug_status" in L.moe_last_error()


def test_build_targets_gfx950_only():
    from combine_moe_get_amd import build

    arch = [f for f in build.CFLAGS if f.startswith("--offload-arch")]
    assert arch == ["--offload-arch=gfx950"]
    assert "-ffp-contract=off" in build.CFLAGS and "-packed-fp32-ops" in build.CFLAGS
    assert not any("fast-math" in f and not f.startswith("-fno-") for f in build.CFLAGS)


def test_header_compiles_as_c():
    src = '#include "moe_get.h"\nint main(void){ return moe_version() > 0 ? 0 : 1; }\n'
    r = subprocess.run(["gcc", "-fsyntax-only", "-x", "c", "-std=c11", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-"],
                       input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.fixture(scope="module")
def lib():
    import combine_moe_get_amd as m

    return m


def test_version_and_sizes(lib):
    assert lib.version() >= 200
    assert lib.moe_required_capacity(4096, 8, 256, 1) == 32768
    assert lib.moe_required_capacity(4, 2, 3, 2) == 11
    assert lib.moe_required_capacity(-1, 8, 256, 1) == -1
    ws = lib.moe_layout_workspace_bytes(4096, 8, 256)
    assert ws > 0 and ws % 256 == 0
    assert lib.moe_layout_workspace_bytes(1, 33, 8) == 0
    assert lib.moe_layout_workspace_bytes(1, 8, 1025) == 0
    # the workspace stays small for every supported size
    for E in (1, 64, 256, 1024):
        for N in (0, 1, 4096, 262144):
            assert lib.moe_layout_workspace_bytes(N, 8, E) <= 1 << 20


def _err(lib):
    return lib._lib.moe_last_error().decode()


def test_layout_validation(lib):
    L = lib._lib
    P = 0x1000  # a fake, aligned pointer: validation must fail before any use
    ws = lib.moe_layout_workspace_bytes(8, 8, 64)
    cases = [
        ((P, 8, -1, 8, 64, 1, P, P, P, P, 64, 0, P, ws, 0, 0), lib.MOE_ERR_ARG),
        ((P, 8, 8, 0, 64, 1, P, P, P, P, 64, 0, P, ws, 0, 0), lib.MOE_ERR_ARG),
        ((P, 8, 8, 33, 64, 1, P, P, P, P, 264, 0, P, ws, 0, 0), lib.MOE_ERR_LIMIT),
        ((P, 8, 8, 8, 1025, 1, P, P, P, P, 64, 0, P, ws, 0, 0), lib.MOE_ERR_LIMIT),
        ((P, 8, 8, 8, 64, 0, P, P, P, P, 64, 0, P, ws, 0, 0), lib.MOE_ERR_ARG),
        ((P, 4, 8, 8, 64, 1, P, P, P, P, 64, 0, P, ws, 0, 0), lib.MOE_ERR_ARG),      # stride < K
        ((0, 8, 8, 8, 64, 1, P, P, P, P, 64, 0, P, ws, 0, 0), lib.MOE_ERR_ARG),      # NULL ids
        ((P, 8, 8, 8, 64, 1, P, P, P, P, 63, 0, P, ws, 0, 0), lib.MOE_ERR_CAPACITY),
        ((P, 8, 8, 8, 64, 2, P, P, P, P, 64, 0, P, ws, 0, 0), lib.MOE_ERR_CAPACITY), # padding room
        ((P, 8, 8, 8, 64, 1, P, P, P, P, 64, 0, 0, ws, 0, 0), lib.MOE_ERR_WORKSPACE),
        ((P, 8, 8, 8, 64, 1, P, P, P, P, 64, 0, P, ws - 4, 0, 0), lib.MOE_ERR_WORKSPACE),
        ((P, 8, 8, 8, 64, 1, P, P, P, P, 64, 0, P + 2, ws, 0, 0), lib.MOE_ERR_ALIGN),
        ((P + 2, 8, 8, 8, 64, 1, P, P, P, P, 64, 0, P, ws, 0, 0), lib.MOE_ERR_ALIGN),
        ((P, 8, 8, 8, 64, 1, P, P, P, P, 1 << 31, 0, P, ws, 0, 0), lib.MOE_ERR_LIMIT),
        ((P, 8, 1 << 28, 8, 64, 1, P, P, P, P, 1 << 31, 0, P, ws, 0, 0), lib.MOE_ERR_LIMIT),
        ((P, 8, 8, 8, 64, 1, P, P, P, P, 64, P + 2, P, ws, 0, 0), lib.MOE_ERR_ALIGN),  # order
    ]
    for args, code in cases:
        assert L.moe_get_layout(*args) == code, (args, _err(lib))
        assert _err(lib)


def test_layout_noalloc_validation(lib):
    """The layout that allocates nothing rejects what moe_get_layout rejects
    (it has no workspace to check), before any GPU call."""
    L = lib._lib
    P = 0x1000
    cases = [
        ((P, 8, -1, 8, 64, 1, P, P, P, P, 64, 0, 0, 0), lib.MOE_ERR_ARG),
        ((P, 8, 8, 33, 64, 1, P, P, P, P, 264, 0, 0, 0), lib.MOE_ERR_LIMIT),
        ((P, 8, 8, 8, 1025, 1, P, P, P, P, 64, 0, 0, 0), lib.MOE_ERR_LIMIT),
        ((P, 4, 8, 8, 64, 1, P, P, P, P, 64, 0, 0, 0), lib.MOE_ERR_ARG),
        ((0, 8, 8, 8, 64, 1, P, P, P, P, 64, 0, 0, 0), lib.MOE_ERR_ARG),
        ((P, 8, 8, 8, 64, 1, P, P, P, P, 63, 0, 0, 0), lib.MOE_ERR_CAPACITY),
        ((P + 2, 8, 8, 8, 64, 1, P, P, P, P, 64, 0, 0, 0), lib.MOE_ERR_ALIGN),
        ((P, 8, 1 << 28, 8, 64, 1, P, P, P, P, 1 << 31, 0, 0, 0), lib.MOE_ERR_LIMIT),
    ]
    for args, code in cases:
        assert L.moe_get_layout_noalloc(*args) == code, (args, _err(lib))
        assert "moe_get_layout_noalloc" in _err(lib)


def _fields(lib, specs):
    arr = (lib.moe_field * len(specs))()
    for i, s in enumerate(specs):
        arr[i] = lib.moe_field(*s)
    return arr


def test_dispatch_validation(lib):
    L = lib._lib
    P = 0x10000
    good = (P, 64, P * 2, 64, 64)
    f = _fields(lib, [good])
    assert L.moe_dispatch(f, 0, 4, 2, P, 0, 0) == lib.MOE_ERR_ARG
    assert L.moe_dispatch(f, 5, 4, 2, P, 0, 0) == lib.MOE_ERR_ARG
    assert L.moe_dispatch(None, 1, 4, 2, P, 0, 0) == lib.MOE_ERR_ARG
    assert L.moe_dispatch(f, 1, -1, 2, P, 0, 0) == lib.MOE_ERR_ARG
    assert L.moe_dispatch(f, 1, 4, 33, P, 0, 0) == lib.MOE_ERR_LIMIT
    assert L.moe_dispatch(f, 1, 1 << 28, 8, P, 0, 0) == lib.MOE_ERR_LIMIT  # N*K = 2^31
    # one wave per (pair, 64-vector segment): 2^31 waves are refused
    two = _fields(lib, [(P, 1040, P * 2, 1040, 1040)])                 # 65 vectors: 2 segments
    assert L.moe_dispatch(two, 1, 1 << 27, 8, P, 0, 0) == lib.MOE_ERR_LIMIT
    assert L.moe_dispatch(f, 1, 4, 2, 0, 0, 0) == lib.MOE_ERR_ARG         # identity needs K == 1
    assert L.moe_dispatch(f, 1, 4, 2, P + 1, 0, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_dispatch(f, 1, 4, 2, P, P + 2, 0) == lib.MOE_ERR_ALIGN    # order
    for bad in [(P + 2, 64, P * 2, 64, 64), (P, 66, P * 2, 64, 64), (P, 64, P * 2, 64, 62),
                (P, 64, P * 2 + 6, 64, 64)]:
        assert L.moe_dispatch(_fields(lib, [bad]), 1, 4, 2, P, 0, 0) == lib.MOE_ERR_ALIGN, bad
    assert L.moe_dispatch(_fields(lib, [(P, 32, P * 2, 64, 64)]), 1, 4, 2, P, 0, 0) == lib.MOE_ERR_ARG
    assert L.moe_dispatch(_fields(lib, [(P, 64, P * 2, 32, 64)]), 1, 4, 2, P, 0, 0) == lib.MOE_ERR_ARG
    assert L.moe_dispatch(_fields(lib, [(0, 64, P * 2, 64, 64)]), 1, 4, 2, P, 0, 0) == lib.MOE_ERR_ARG
    assert L.moe_dispatch(_fields(lib, [(P, -1, P, 64, -16)]), 1, 4, 2, P, 0, 0) == lib.MOE_ERR_ARG
    # nothing to copy: returns before any launch
    assert L.moe_dispatch(f, 1, 0, 2, P, 0, 0) == lib.MOE_OK
    assert L.moe_dispatch(_fields(lib, [(P, 64, P, 64, 0)]), 1, 4, 2, P, 0, 0) == lib.MOE_OK


def test_combine_validation(lib):
    L = lib._lib
    P = 0x10000
    assert L.moe_combine(P, 64, P, 8, P, -1, 8, 64, P, 64, 0) == lib.MOE_ERR_ARG
    assert L.moe_combine(P, 64, P, 8, P, 4, 0, 64, P, 64, 0) == lib.MOE_ERR_ARG
    assert L.moe_combine(P, 64, P, 8, P, 4, 33, 64, P, 64, 0) == lib.MOE_ERR_LIMIT
    assert L.moe_combine(0, 64, P, 8, P, 4, 8, 64, P, 64, 0) == lib.MOE_ERR_ARG
    assert L.moe_combine(P, 64, P, 7, P, 4, 8, 64, P, 64, 0) == lib.MOE_ERR_ARG     # w stride < K
    assert L.moe_combine(P, 32, P, 8, P, 4, 8, 64, P, 64, 0) == lib.MOE_ERR_ARG     # y stride < Hc
    assert L.moe_combine(P, 64, P, 8, P, 4, 8, 63, P, 64, 0) == lib.MOE_ERR_ALIGN   # odd Hc
    assert L.moe_combine(P + 2, 64, P, 8, P, 4, 8, 64, P, 64, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_combine(P, 64, P + 2, 8, P, 4, 8, 64, P, 64, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_combine(P, 64, P, 8, P, 0, 8, 64, P, 64, 0) == lib.MOE_OK          # N = 0
    assert L.moe_combine(P, 64, P, 8, P, 4, 8, 0, P, 64, 0) == lib.MOE_OK           # Hc = 0
    assert _err(lib) == ""


def test_combine_epilogue_validation(lib):
    import ctypes

    L = lib._lib
    P = 0x10000

    def ep(**kw):
        e = lib.moe_epilogue()
        e.eps = 1e-6
        for k, v in kw.items():
            setattr(e, k, v)
        return ctypes.byref(e)

    args = (P, 64, P, 8, P, 4, 8, 64)
    # a residual needs gamma and residual_out
    assert L.moe_combine_epilogue(*args, ep(residual=P, residual_row_stride=64), P, 64, 0) == lib.MOE_ERR_ARG
    assert L.moe_combine_epilogue(*args, ep(residual=P, residual_row_stride=64, gamma=P), P, 64, 0) == lib.MOE_ERR_ARG
    full = dict(residual=P, residual_row_stride=64, gamma=P, residual_out=P, residual_out_row_stride=64)
    assert L.moe_combine_epilogue(*args, ep(**full, eps=-1.0), P, 64, 0) == lib.MOE_ERR_ARG
    assert L.moe_combine_epilogue(*args, ep(**full, eps=float("nan")), P, 64, 0) == lib.MOE_ERR_ARG
    # alignment: Hc multiple of 8, 16-byte rows, gamma 16-byte aligned
    assert L.moe_combine_epilogue(P, 60, P, 8, P, 4, 8, 60, ep(**full), P, 60, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_combine_epilogue(*args, ep(bias0=P + 4, bias0_row_stride=64), P, 64, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_combine_epilogue(*args, ep(bias0=P, bias0_row_stride=68), P, 64, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_combine_epilogue(*args, ep(**dict(full, gamma=P + 8)), P, 64, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_combine_epilogue(*args, ep(bias1=P, bias1_row_stride=32), P, 64, 0) == lib.MOE_ERR_ARG
    # the register-resident token row bounds Hc
    assert L.moe_combine_epilogue(P, 65544, P, 8, P, 4, 8, 65544, ep(bias0=P, bias0_row_stride=65544),
                                  P, 65544, 0) == lib.MOE_ERR_LIMIT
    assert L.moe_combine_epilogue(P, 64, P, 8, P, 0, 8, 64, ep(**full), P, 64, 0) == lib.MOE_OK   # N = 0


def test_layout_padded_and_fp8_validation(lib):
    L = lib._lib
    P = 0x10000
    ws = lib.moe_layout_workspace_bytes(8, 8, 64)
    assert L.moe_get_layout_padded(P, 8, 8, 8, 64, 0, P, P, P, 0, 0, P, ws, P, 0) == lib.MOE_ERR_ARG    # M = 0
    assert L.moe_get_layout_padded(P, 8, 8, 8, 1025, 4, P, P, P, 0, 0, P, ws, P, 0) == lib.MOE_ERR_LIMIT
    assert L.moe_get_layout_padded(P, 8, 8, 8, 1024, 1 << 21, P, P, P, 0, 0, P, ws, P, 0) == lib.MOE_ERR_LIMIT
    assert L.moe_get_layout_padded(P, 8, 8, 8, 64, 4, P, P, P, 0, 0, 0, ws, P, 0) == lib.MOE_ERR_WORKSPACE
    assert L.moe_get_layout_padded(P + 2, 8, 8, 8, 64, 4, P, P, P, 0, 0, P, ws, P, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_get_layout_padded(P, 8, 8, 8, 64, 4, P, P, P, P + 4, 0, P, ws, P, 0) == lib.MOE_ERR_ALIGN
    assert L.moe_get_layout_padded(P, 8, 8, 8, 64, 4, P, P, P, 0, P + 2, P, ws, P, 0) == lib.MOE_ERR_ALIGN
    F = L.moe_dispatch_fp8
    assert F(P, 256, 4, 2, 200, P, P, 256, P, 0, 2, 0, 0, 0) == lib.MOE_ERR_ALIGN         # H % 128
    assert F(P, 512, 4, 2, 256, P, P, 256, P, 2, 0, 4, 0, 0) == lib.MOE_ERR_ARG           # ue8m0 w/o round
    assert F(P, 256, 4, 2, 256, P, P, 256, P, 2, 0, 4, 1, 0) == lib.MOE_ERR_ARG           # ue8m0, H % 512
    assert F(P, 256, 4, 2, 256, P, P, 256, P, 1, 0, 0, 0, 0) == lib.MOE_ERR_ARG           # cols need M
    assert F(P, 256, 4, 2, 256, P, P, 256, P, 0, 1, 0, 0, 0) == lib.MOE_ERR_ARG           # row stride
    assert F(P, 256, 4, 2, 256, P, P, 256, P, 7, 2, 0, 0, 0) == lib.MOE_ERR_ARG           # format
    assert F(P + 8, 256, 4, 2, 256, P, P, 256, P, 0, 2, 0, 0, 0) == lib.MOE_ERR_ALIGN     # x alignment
    assert F(P, 256, 4, 2, 256, P, P + 8, 256, P, 0, 2, 0, 0, 0) == lib.MOE_ERR_ALIGN     # dst alignment
    assert F(P, 256, 4, 2, 256, P, P, 264, P, 0, 2, 0, 0, 0) == lib.MOE_ERR_ALIGN         # dst stride
    assert F(P, 256, 4, 2, 256, 0, P, 256, P, 0, 2, 0, 0, 0) == lib.MOE_ERR_ARG           # identity, K=2
    assert F(P, 256, 4, 33, 256, P, P, 256, P, 0, 2, 0, 0, 0) == lib.MOE_ERR_LIMIT
    assert F(P, 256, 0, 2, 256, P, P, 256, P, 0, 2, 0, 0, 0) == lib.MOE_OK                # N = 0
    # per-token scales: a row stride of at least H/128, no rows per expert needed
    assert F(P, 256, 4, 2, 256, P, P, 256, P, 3, 1, 0, 0, 0) == lib.MOE_ERR_ARG           # row stride
    assert F(P, 256, 0, 2, 256, P, P, 256, P, 3, 2, 0, 0, 0) == lib.MOE_OK                # N = 0, M = 0


def test_scatter_scales_validation(lib):
    S = lib._lib.moe_scatter_scales
    P = 0x10000
    # (token_scales, tss, N, K, H, row_pair, E, M, scales, fmt, stream)
    ok = lambda **kw: [kw.get(n, d) for n, d in (
        ("ts", P), ("tss", 4), ("N", 16), ("K", 8), ("H", 512), ("rp", P), ("E", 32), ("M", 64),
        ("sc", P), ("fmt", 1), ("stream", 0))]
    assert S(*ok(fmt=0)) == lib.MOE_ERR_ARG                # row-major is not a placed form
    assert S(*ok(fmt=3)) == lib.MOE_ERR_ARG
    assert S(*ok(K=0)) == lib.MOE_ERR_ARG
    assert S(*ok(M=0)) == lib.MOE_ERR_ARG
    assert S(*ok(N=-1)) == lib.MOE_ERR_ARG
    assert S(*ok(H=200)) == lib.MOE_ERR_ALIGN              # H % 128
    assert S(*ok(H=384, tss=3, fmt=2)) == lib.MOE_ERR_ARG  # ue8m0: H % 512
    assert S(*ok(tss=3)) == lib.MOE_ERR_ARG                # stride < H/128
    assert S(*ok(E=1 << 16, M=1 << 15)) == lib.MOE_ERR_LIMIT   # E*M >= 2^31
    assert S(*ok(rp=0)) == lib.MOE_ERR_ARG
    assert S(*ok(ts=0)) == lib.MOE_ERR_ARG
    assert S(*ok(sc=P + 2)) == lib.MOE_ERR_ALIGN
    assert S(*ok(N=0, ts=0)) == lib.MOE_OK                 # no pair can be valid: nothing to do
    assert S(*ok(E=0)) == lib.MOE_OK


def test_check_layout_validation(lib):
    C = lib._lib.moe_check_layout
    P = 0x10000
    # (pos, N, K, row_pair, cap, order, status, stream)
    ok = lambda **kw: [kw.get(n, d) for n, d in (
        ("pos", P), ("N", 16), ("K", 8), ("rp", P), ("cap", 128), ("order", P), ("st", P),
        ("stream", 0))]
    assert C(*ok(N=-1)) == lib.MOE_ERR_ARG
    assert C(*ok(K=0)) == lib.MOE_ERR_ARG
    assert C(*ok(cap=-1)) == lib.MOE_ERR_ARG
    assert C(*ok(N=1 << 28, K=8)) == lib.MOE_ERR_LIMIT     # N*K >= 2^31
    assert C(*ok(cap=1 << 31)) == lib.MOE_ERR_LIMIT
    assert C(*ok(st=0)) == lib.MOE_ERR_ARG
    assert C(*ok(pos=0)) == lib.MOE_ERR_ARG
    assert C(*ok(pos=P + 2)) == lib.MOE_ERR_ALIGN
    assert C(*ok(rp=P + 1)) == lib.MOE_ERR_ALIGN
    assert C(*ok(order=P + 3)) == lib.MOE_ERR_ALIGN
    assert C(*ok(st=P + 2)) == lib.MOE_ERR_ALIGN


def test_backward_validation(lib):
    L = lib._lib
    P = 0x10000
    D = L.moe_dispatch_backward
    # (grad_recv, grs, grad_recv_w, grws, pos, N, K, H, grad_x, gxs, grad_w, gws, stream)
    assert D(P, 64, P, 8, P, 4, 0, 64, P, 64, P, 8, 0) == lib.MOE_ERR_ARG        # K = 0
    assert D(P, 64, P, 8, P, 4, 33, 64, P, 64, P, 33, 0) == lib.MOE_ERR_LIMIT    # K > 32
    assert D(P, 64, P, 8, P, 4, 8, 64, P, 64, 0, 8, 0) == lib.MOE_ERR_ARG        # w grads unpaired
    assert D(P, 64, 0, 8, P, 4, 8, 64, P, 64, P, 8, 0) == lib.MOE_ERR_ARG
    assert D(P, 64, P, 4, P, 4, 8, 64, P, 64, P, 8, 0) == lib.MOE_ERR_ARG        # grws < K
    assert D(P, 32, 0, 8, P, 4, 8, 64, P, 64, 0, 8, 0) == lib.MOE_ERR_ARG        # stride < H
    assert D(P, 64, 0, 8, P, 4, 8, 63, P, 64, 0, 8, 0) == lib.MOE_ERR_ALIGN      # odd H
    assert D(P + 2, 64, 0, 8, P, 4, 8, 64, P, 64, 0, 8, 0) == lib.MOE_ERR_ALIGN  # grad_recv
    assert D(0, 64, 0, 8, P, 4, 8, 64, P, 64, 0, 8, 0) == lib.MOE_ERR_ARG        # NULL
    assert D(P, 64, 0, 8, P, 0, 8, 64, P, 64, 0, 8, 0) == lib.MOE_OK             # N = 0
    C = L.moe_combine_backward
    # (grad_out, gos, w, ws, y, ys, pos, N, K, Hc, grad_y, gys, grad_w, gws, stream)
    assert C(P, 64, P, 8, P, 64, P, 4, 0, 64, P, 64, P, 8, 0) == lib.MOE_ERR_ARG        # K = 0
    assert C(P, 64, P, 8, 0, 64, P, 4, 8, 64, P, 64, P, 8, 0) == lib.MOE_ERR_ARG        # grad_w, no y
    assert C(P, 32776, P, 8, P, 32776, P, 4, 8, 32776, P, 32776, P, 8, 0) == lib.MOE_ERR_LIMIT
    assert C(P, 64, P, 8, P, 64, P, 4, 8, 60, P, 64, P, 8, 0) == lib.MOE_ERR_ALIGN      # Hc % 8
    assert C(P + 8, 64, P, 8, P, 64, P, 4, 8, 64, P, 64, P, 8, 0) == lib.MOE_ERR_ALIGN  # grad_out
    assert C(P, 64, P, 8, P, 60, P, 4, 8, 56, P, 64, P, 8, 0) == lib.MOE_ERR_ALIGN      # y stride
    assert C(P, 64, P, 4, P, 64, P, 4, 8, 64, P, 64, P, 8, 0) == lib.MOE_ERR_ARG        # ws < K
    assert C(P, 64, P, 8, P, 64, P, 4, 8, 64, 0, 64, P, 8, 0) == lib.MOE_ERR_ARG        # NULL grad_y
    assert C(P, 64, P, 8, 0, 64, P, 0, 8, 64, P, 64, 0, 8, 0) == lib.MOE_OK             # N = 0
    assert C(P, 64, P, 8, 0, 64, P, 4, 8, 0, P, 64, 0, 8, 0) == lib.MOE_OK              # Hc = 0, no w


def test_fused_padded_fp8_validation(lib):
    F = lib._lib.moe_dispatch_fp8_padded
    P = 0x10000
    # (ids, istr, N, K, E, M, x, xs, H, counts, pos, row_pair, layout_range, recv_stats, status,
    #  dst, ds, scales, fmt, srs, round, stream)
    ok = lambda **kw: [kw.get(n, d) for n, d in (
        ("ids", P), ("istr", 8), ("N", 16), ("K", 8), ("E", 32), ("M", 16), ("x", P), ("xs", 256),
        ("H", 256), ("counts", P), ("pos", P), ("rp", P), ("lr", 0), ("rs", 0), ("st", P),
        ("dst", P), ("ds", 256), ("sc", P), ("fmt", 1), ("srs", 0), ("rnd", 0), ("stream", 0))]
    assert F(*ok(N=1025)) == lib.MOE_ERR_LIMIT            # N*K > 8192
    assert F(*ok(K=33)) == lib.MOE_ERR_LIMIT
    assert F(*ok(M=0)) == lib.MOE_ERR_ARG
    assert F(*ok(H=200)) == lib.MOE_ERR_ALIGN              # H % 128
    assert F(*ok(fmt=2, rnd=0)) == lib.MOE_ERR_ARG         # ue8m0 needs round_scale
    assert F(*ok(fmt=0, srs=1)) == lib.MOE_ERR_ARG         # row scale stride
    assert F(*ok(fmt=3, srs=1)) == lib.MOE_ERR_ARG         # token scale stride
    assert F(*ok(st=0)) == lib.MOE_ERR_ARG
    assert F(*ok(istr=4)) == lib.MOE_ERR_ARG               # ids stride < K
    assert F(*ok(x=P + 8)) == lib.MOE_ERR_ALIGN
    assert F(*ok(ds=264)) == lib.MOE_ERR_ALIGN
    assert F(*ok(pos=P + 2)) == lib.MOE_ERR_ALIGN
    assert F(*ok(lr=P + 4)) == lib.MOE_ERR_ALIGN               # layout_range is int64
    assert F(*ok(rs=P + 2)) == lib.MOE_ERR_ALIGN
    # one launch: 8192 tokens x ceil(H/4096) workgroups must stay within 2^23
    H = 4096 * 1024 + 128
    assert F(*ok(N=8192, K=1, H=H, xs=H, ds=H)) == lib.MOE_ERR_LIMIT


def test_builder_loads_without_the_package():
    """build() must work when the library is missing or stale: the builder
    is loaded by path, without importing the package that loads the library."""
    code = ("import importlib.util, sys\n"
            f"spec = importlib.util.spec_from_file_location('b', {os.path.join(ROOT, 'combine_moe_get_amd', 'build.py')!r})\n"
            "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
            "assert callable(m.build) and 'combine_moe_get_amd' not in sys.modules\n")
    r = subprocess.run(["python3", "-c", code], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    src = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    assert "spec_from_file_location" in src and "from combine_moe_get_amd import build" not in src


def test_c_program_builds_against_the_header(tmp_path):
    """The C ABI check program (tests/c_abi) compiles and links from plain C
    against the header, the library and the oracle."""
    import importlib.util

    import oracle

    oracle.lib()                      # builds liboracle.so when it is missing
    spec = importlib.util.spec_from_file_location("cb", os.path.join(ROOT, "tests", "c_abi", "build.py"))
    cb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(cb)
    out = cb.build(str(tmp_path / "abi_check"))
    assert os.path.exists(out)


def test_layout_dispatch_validation(lib):
    F = lib._lib.moe_layout_dispatch
    P = 0x10000
    fld = (lib.moe_field * 1)(lib.moe_field(P, 64, P, 64, 64))
    # (ids, istr, N, K, E, align, counts, offsets, pos, row_pair, cap, status, fields, nf, stream)
    assert F(P, 8, 1025, 8, 64, 1, P, P, P, P, 8200, P, fld, 1, 0) == lib.MOE_ERR_LIMIT   # N*K > 8192
    assert F(P, 8, 16, 8, 64, 1, P, P, P, P, 100, P, fld, 1, 0) == lib.MOE_ERR_CAPACITY
    assert F(P, 8, 16, 8, 1025, 1, P, P, P, P, 128, P, fld, 1, 0) == lib.MOE_ERR_LIMIT
    assert F(P, 8, 16, 8, 64, 0, P, P, P, P, 128, P, fld, 1, 0) == lib.MOE_ERR_ARG       # align 0
    assert F(P, 4, 16, 8, 64, 1, P, P, P, P, 128, P, fld, 1, 0) == lib.MOE_ERR_ARG       # ids stride
    # one launch: 8192 tokens x ceil(segments / 4) workgroups must stay within 2^23
    rb = 16 * 64 * 4 * 1024 + 16                                 # 1025 workgroups per token
    big = (lib.moe_field * 1)(lib.moe_field(P, rb, P, rb, rb))
    assert F(P, 1, 8192, 1, 64, 1, P, P, P, P, 8192, P, big, 1, 0) == lib.MOE_ERR_LIMIT
    assert F(P + 2, 8, 16, 8, 64, 1, P, P, P, P, 128, P, fld, 1, 0) == lib.MOE_ERR_ALIGN
    assert F(P, 8, 16, 8, 64, 1, P, P, P, P, 128, P, fld, 0, 0) == lib.MOE_ERR_ARG       # no fields
    bad = (lib.moe_field * 1)(lib.moe_field(P + 2, 64, P, 64, 64))
    assert F(P, 8, 16, 8, 64, 1, P, P, P, P, 128, P, bad, 1, 0) == lib.MOE_ERR_ALIGN


def test_record_offsets_and_pack_validation(lib):
    """moe_record_offsets is host-only: the packed-record workload's layout
    (ids 32 B @0, weights 32 B @32, hidden 3584 B @64, scales 448 B @3648, a
    4096-B record) and the 16-byte rounding of odd sizes."""
    offs, size = lib.record_offsets([32, 32, 3584, 448])
    assert offs == [0, 32, 64, 3648] and size == 4096
    offs, size = lib.record_offsets([4, 20, 8])
    assert offs == [0, 16, 48] and size == 64
    assert lib.record_offsets([0])[1] == 0
    for bad in ([], [4] * 5, [3], [-4]):
        with pytest.raises(lib.MoeError):
            lib.record_offsets(bad)
    L = lib._lib
    P = 0x10000
    fld = (lib.moe_field * 2)(lib.moe_field(P, 64, 0, 0, 64), lib.moe_field(P, 16, 0, 0, 16))
    assert L.moe_pack_records(fld, 2, 8, P, 64, 0) == lib.MOE_ERR_ARG      # record is 80 B
    assert L.moe_pack_records(fld, 2, 8, 0, 80, 0) == lib.MOE_ERR_ARG      # NULL records
    assert L.moe_pack_records(fld, 0, 8, P, 80, 0) == lib.MOE_ERR_ARG
    assert L.moe_unpack_records(P, 64, 8, fld, 2, 0) == lib.MOE_ERR_ARG
    assert L.moe_pack_records(fld, 2, 0, P, 80, 0) == lib.MOE_OK           # N = 0
