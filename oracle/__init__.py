"""CPU oracle for the MoE layout / dispatch / combine path (numpy in, numpy out).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product library never does.
It shares no code with the GPU library. The arithmetic lives in
``moe_oracle.c`` (plain C, fp32 fmaf chain, built without fast-math); this
file only marshals numpy arrays into it.

Every function here is pinned by ``tests/test_oracle_*.py`` against library
routines, invariants, closed forms, brute force and hand-worked fixtures.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

OK, ERR_ARG, ERR_ALIGN, ERR_LIMIT, ERR_CAPACITY, ERR_NOMEM = 0, -1, -2, -3, -4, -5


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into liboracle.so (gcc, -O2, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-std=c11",
               "-Wall", "-Wextra", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Field(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("src_row_stride", ctypes.c_int64),
                ("dst", ctypes.c_void_p), ("dst_row_stride", ctypes.c_int64),
                ("row_bytes", ctypes.c_int64)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, i64, P]
        L.oracle_layout.restype = ctypes.c_int
        L.oracle_dispatch.argtypes = [ctypes.POINTER(_Field), i32, i32, i32, P]
        L.oracle_dispatch.restype = ctypes.c_int
        L.oracle_combine.argtypes = [P, i64, P, i64, P, i32, i32, i32, P, i64]
        L.oracle_combine.restype = ctypes.c_int
        L.oracle_combine_acc.argtypes = [P, i64, P, i64, P, i32, i32, i32, P]
        L.oracle_combine_acc.restype = ctypes.c_int
        L.oracle_combine_epilogue.argtypes = [P, i64, P, i64, P, i32, i32, i32, P, P, P, P,
                                              ctypes.c_float, P, P]
        L.oracle_combine_epilogue.restype = ctypes.c_int
        L.oracle_bf16_from_f64.argtypes = [ctypes.c_double]
        L.oracle_bf16_from_f64.restype = ctypes.c_uint16
        L.oracle_layout_padded.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P]
        L.oracle_layout_padded.restype = ctypes.c_int
        L.oracle_padded_recv_meta.argtypes = [P, i32, P, P]
        L.oracle_padded_recv_meta.restype = None
        L.oracle_f32_to_e4m3.argtypes = [ctypes.c_float]
        L.oracle_f32_to_e4m3.restype = ctypes.c_uint8
        L.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_to_f32.restype = ctypes.c_float
        L.oracle_fp8_block_scale.argtypes = [P, ctypes.c_int]
        L.oracle_fp8_block_scale.restype = ctypes.c_float
        L.oracle_dispatch_fp8.argtypes = [P, i64, i32, i32, i32, P, P, i64, P, i32, i64, i32, i32]
        L.oracle_dispatch_fp8.restype = ctypes.c_int
        L.oracle_scatter_scales.argtypes = [P, i64, i32, i32, i32, P, i32, i32, P, i32]
        L.oracle_scatter_scales.restype = ctypes.c_int
        L.oracle_dispatch_backward.argtypes = [P, i64, P, i64, P, i32, i32, i32, P, i64, P, i64]
        L.oracle_dispatch_backward.restype = ctypes.c_int
        L.oracle_combine_backward.argtypes = [P, i64, P, i64, P, i64, P, i32, i32, i32, P, i64, P,
                                              i64]
        L.oracle_combine_backward.restype = ctypes.c_int
        L.oracle_required_cap.argtypes = [i32, i32, i32, i32]
        L.oracle_required_cap.restype = i64
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f32.restype = ctypes.c_float
        _lib = L
    return _lib


def set_threads(n: int) -> int:
    """OpenMP threads for the oracle's parallel loops (per-token work, whose
    results do not depend on the thread count); returns the previous count."""
    L = lib()
    prev = int(L.omp_get_max_threads())
    L.omp_set_num_threads(int(n))
    return prev


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: oracle returned {code}")
        self.code = code


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _row_view(a: np.ndarray) -> Tuple[int, int]:
    """(base pointer, row stride in elements) of a 2-D array whose rows may be
    strided but whose elements inside a row are contiguous."""
    assert a.ndim == 2 and (a.shape[1] <= 1 or a.strides[1] == a.itemsize)
    return _ptr(a), a.strides[0] // a.itemsize


def required_cap(N: int, K: int, E: int, align: int = 1) -> int:
    return int(lib().oracle_required_cap(N, K, E, align))


def layout(ids: np.ndarray, E: int, align: int = 1, cap: Optional[int] = None):
    """Routing layout of ``ids`` [N, K] int32 (rows may be strided).

    Returns (counts [E], offsets [E+1], pos [N, K], row_pair [cap], status).
    """
    assert ids.dtype == np.int32
    N, K = ids.shape
    if cap is None:
        cap = max(required_cap(N, K, E, align), 0)
    base, stride = _row_view(ids) if N > 0 else (0, K)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    pos = np.empty((N, K), np.int32)
    row_pair = np.empty(max(cap, 0), np.int32)
    status = np.zeros(1, np.int32)
    rc = lib().oracle_layout(base, stride, N, K, E, align, _ptr(counts), _ptr(offsets),
                             _ptr(pos), _ptr(row_pair), cap, _ptr(status))
    if rc != OK:
        raise OracleError(rc, "layout")
    return counts, offsets, pos, row_pair, int(status[0])


def dispatch(srcs: Sequence[np.ndarray], pos: Optional[np.ndarray], K: int,
             dsts: Optional[List[np.ndarray]] = None, rows: Optional[int] = None,
             fill: int = 0) -> List[np.ndarray]:
    """Copy each token's row of every ``srcs[f]`` [N, bytes] (uint8) into
    ``dsts[f]`` [rows, bytes] at row pos[t, k]. ``pos=None`` is the identity
    (K must be 1). Missing ``dsts`` are allocated and filled with ``fill``."""
    N = srcs[0].shape[0]
    if dsts is None:
        rows = N * K if rows is None else rows
        dsts = [np.full((rows, s.shape[1]), fill, np.uint8) for s in srcs]
    fs = (_Field * len(srcs))()
    for i, (s, d) in enumerate(zip(srcs, dsts)):
        assert s.dtype == np.uint8 and d.dtype == np.uint8 and s.shape[1] == d.shape[1]
        sb, ss = _row_view(s) if s.shape[0] else (0, s.shape[1])
        db, ds = _row_view(d) if d.shape[0] else (0, d.shape[1])
        fs[i] = _Field(sb, ss, db, ds, s.shape[1])
    pos_c = None if pos is None else np.ascontiguousarray(pos, dtype=np.int32)
    rc = lib().oracle_dispatch(fs, len(srcs), N, K, 0 if pos_c is None else _ptr(pos_c))
    if rc != OK:
        raise OracleError(rc, "dispatch")
    return dsts


def combine(y: np.ndarray, w: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """out [N, Hc] (bf16 bits, uint16) = bf16(sum_k w[t,k] * y[pos[t,k]])."""
    assert y.dtype == np.uint16 and w.dtype == np.float32
    N, K = pos.shape
    Hc = y.shape[1]
    out = np.empty((N, Hc), np.uint16)
    pos_c = np.ascontiguousarray(pos, dtype=np.int32)
    yb, ys = _row_view(y) if y.shape[0] else (0, Hc)
    wb, ws = _row_view(w) if N else (0, K)
    rc = lib().oracle_combine(yb, ys, wb, ws, _ptr(pos_c), N, K, Hc, _ptr(out), Hc)
    if rc != OK:
        raise OracleError(rc, "combine")
    return out


def dispatch_backward(grad_recv: np.ndarray, pos: np.ndarray,
                      grad_recv_w: Optional[np.ndarray] = None):
    """Backward of the dispatch: grad_x [N, H] (bf16 bits) = bf16(sum over
    valid k, ascending, of grad_recv[pos[t,k]]) and, given grad_recv_w
    [rows, K] fp32, grad_w [N, K] = the same sum of grad_recv_w rows (else
    None)."""
    assert grad_recv.dtype == np.uint16
    N, K = pos.shape
    H = grad_recv.shape[1]
    grad_x = np.empty((N, H), np.uint16)
    pos_c = np.ascontiguousarray(pos, dtype=np.int32)
    gb, gs = _row_view(grad_recv) if grad_recv.shape[0] else (0, H)
    grad_w = None
    wb, ws = 0, K
    if grad_recv_w is not None:
        assert grad_recv_w.dtype == np.float32 and grad_recv_w.shape[1] >= K
        wb, ws = _row_view(grad_recv_w) if grad_recv_w.shape[0] else (0, K)
        grad_w = np.empty((N, K), np.float32)
    rc = lib().oracle_dispatch_backward(gb, gs, wb if grad_recv_w is not None else None, ws,
                                        _ptr(pos_c), N, K, H, _ptr(grad_x), H,
                                        _ptr(grad_w) if grad_w is not None else None, K)
    if rc != OK:
        raise OracleError(rc, "dispatch_backward")
    return grad_x, grad_w


def combine_backward(grad_out: np.ndarray, w: np.ndarray, pos: np.ndarray, rows: int,
                     y: Optional[np.ndarray] = None, fill: int = 0):
    """Backward of the combine: grad_y [rows, Hc] (bf16 bits; rows no pair
    lands on keep `fill`) with grad_y[pos[t,k]] = bf16(w[t,k] * grad_out[t])
    and, given y, grad_w [N, K] fp32 = <grad_out[t], y[pos[t,k]]> formed in
    double (0 for masked pairs; else None)."""
    assert grad_out.dtype == np.uint16 and w.dtype == np.float32
    N, K = pos.shape
    Hc = grad_out.shape[1]
    grad_y = np.full((rows, Hc), fill, np.uint16)
    pos_c = np.ascontiguousarray(pos, dtype=np.int32)
    gb, gs = _row_view(grad_out) if N else (0, Hc)
    wb, ws = _row_view(w) if N else (0, K)
    grad_w = None
    yb, ys = None, Hc
    if y is not None:
        assert y.dtype == np.uint16 and y.shape[1] == Hc
        yb, ys = _row_view(y) if y.shape[0] else (0, Hc)
        grad_w = np.empty((N, K), np.float32)
    rc = lib().oracle_combine_backward(gb, gs, wb, ws, yb, ys, _ptr(pos_c), N, K, Hc,
                                       _ptr(grad_y) if rows else None, Hc,
                                       _ptr(grad_w) if grad_w is not None else None, K)
    if rc != OK:
        raise OracleError(rc, "combine_backward")
    return grad_y, grad_w


def combine_acc(y: np.ndarray, w: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """The fp32 accumulators [N, Hc] of ``combine`` before the bf16 rounding."""
    assert y.dtype == np.uint16 and w.dtype == np.float32
    N, K = pos.shape
    Hc = y.shape[1]
    acc = np.empty((N, Hc), np.float32)
    pos_c = np.ascontiguousarray(pos, dtype=np.int32)
    yb, ys = _row_view(y) if y.shape[0] else (0, Hc)
    wb, ws = _row_view(w) if N else (0, K)
    rc = lib().oracle_combine_acc(yb, ys, wb, ws, _ptr(pos_c), N, K, Hc, _ptr(acc))
    if rc != OK:
        raise OracleError(rc, "combine_acc")
    return acc


def combine_epilogue(y: np.ndarray, w: np.ndarray, pos: np.ndarray,
                     bias0: Optional[np.ndarray] = None, bias1: Optional[np.ndarray] = None,
                     residual: Optional[np.ndarray] = None, gamma: Optional[np.ndarray] = None,
                     eps: float = 1e-6):
    """Combine followed by the optional biases and, with a residual, the
    residual add and RMSNorm. Returns (out, residual_out or None), bf16 bits.
    bias0 / bias1 / residual are [N, Hc] bf16 bits, gamma [Hc]."""
    assert y.dtype == np.uint16 and w.dtype == np.float32
    N, K = pos.shape
    Hc = y.shape[1]
    out = np.empty((N, Hc), np.uint16)
    res_out = np.empty((N, Hc), np.uint16) if residual is not None else None
    pos_c = np.ascontiguousarray(pos, dtype=np.int32)
    yb, ys = _row_view(y) if y.shape[0] else (0, Hc)
    wb, ws = _row_view(w) if N else (0, K)

    def opt(a, shape):
        if a is None:
            return None, 0
        a = np.ascontiguousarray(a, dtype=np.uint16)
        assert a.shape == shape
        return a, _ptr(a)

    b0, p0 = opt(bias0, (N, Hc))
    b1, p1 = opt(bias1, (N, Hc))
    r, pr = opt(residual, (N, Hc))
    g, pg = opt(gamma, (Hc,))
    rc = lib().oracle_combine_epilogue(yb, ys, wb, ws, _ptr(pos_c), N, K, Hc, p0, p1, pr, pg,
                                       eps, 0 if res_out is None else _ptr(res_out), _ptr(out))
    if rc != OK:
        raise OracleError(rc, "combine_epilogue")
    return out, res_out


def layout_padded(ids: np.ndarray, E: int, M: int):
    """Padded per-expert layout: expert e owns rows e*M .. e*M+M-1.
    Returns (counts [E], pos [N, K], row_pair [E*M], status (ids >= E, dropped))."""
    assert ids.dtype == np.int32
    N, K = ids.shape
    base, stride = _row_view(ids) if N > 0 else (0, K)
    counts = np.empty(E, np.int32)
    pos = np.empty((N, K), np.int32)
    row_pair = np.empty(E * M, np.int32)
    status = np.zeros(2, np.int32)
    rc = lib().oracle_layout_padded(base, stride, N, K, E, M, _ptr(counts), _ptr(pos),
                                    _ptr(row_pair), _ptr(status))
    if rc != OK:
        raise OracleError(rc, "layout_padded")
    return counts, pos, row_pair, (int(status[0]), int(status[1]))


def padded_recv_meta(counts: np.ndarray, recv_stats: Optional[np.ndarray] = None):
    """The padded layout's receive metadata for one source: (layout_range
    int64 [E], recv_stats int32 [E] after adding counts; a zeroed array when
    none is given)."""
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    E = counts.size
    rng = np.empty(E, np.int64)
    stats = np.zeros(E, np.int32) if recv_stats is None else np.array(recv_stats, np.int32)
    lib().oracle_padded_recv_meta(_ptr(counts), E, _ptr(rng), _ptr(stats))
    return rng, stats


SCALE_ROWS, SCALE_COLS, SCALE_UE8M0, SCALE_TOKENS = 0, 1, 2, 3


def dispatch_fp8(x: np.ndarray, pos: np.ndarray, rows: int, scale_mode: int = SCALE_ROWS,
                 M: int = 0, round_scale: bool = False, fill: int = 0,
                 codes: np.ndarray = None, scales: np.ndarray = None):
    """Quantising dispatch of bf16 x [N, H] (bits). Returns (codes [rows, H]
    uint8, scales): fp32 [rows, H/128] (SCALE_ROWS), fp32 [rows/M, H/128, M]
    (SCALE_COLS), int32 [rows/M, H/512, M] (SCALE_UE8M0) or fp32 [N, H/128]
    per token (SCALE_TOKENS). Given `codes`
    and `scales` (contiguous, of those shapes), writes into them instead;
    rows no pair lands on are left as they are."""
    assert x.dtype == np.uint16
    N, H = x.shape
    K = pos.shape[1]
    if scale_mode == SCALE_ROWS:
        sshape, sdtype = (rows, H // 128), np.float32
    elif scale_mode == SCALE_TOKENS:
        sshape, sdtype = (N, H // 128), np.float32
    elif scale_mode == SCALE_COLS:
        sshape, sdtype = (rows // M, H // 128, M), np.float32
    else:
        sshape, sdtype = (rows // M, H // 512, M), np.int32
    if codes is None:
        codes = np.full((rows, H), fill, np.uint8)
    if scales is None:
        scales = np.zeros(sshape, sdtype)
    assert codes.shape == (rows, H) and codes.dtype == np.uint8 and codes.flags.c_contiguous
    assert scales.shape == sshape and scales.dtype == sdtype and scales.flags.c_contiguous
    pos_c = np.ascontiguousarray(pos, dtype=np.int32)
    xb, xs = _row_view(x) if N else (0, H)
    rc = lib().oracle_dispatch_fp8(xb, xs, N, K, H, _ptr(pos_c), _ptr(codes), H, _ptr(scales),
                                   scale_mode, H // 128, M, int(round_scale))
    if rc != OK:
        raise OracleError(rc, "dispatch_fp8")
    return codes, scales


def scatter_scales(token_scales: np.ndarray, K: int, row_pair: np.ndarray, E: int, M: int,
                   scale_mode: int = SCALE_COLS, scales: np.ndarray = None) -> np.ndarray:
    """Scales of the padded layout's rows from per-token ones (fp32 [N, H/128]):
    fp32 [E, H/128, M] (SCALE_COLS) or int32 [E, H/512, M] (SCALE_UE8M0).
    Given `scales`, writes into it; rows without a pair are left as they are."""
    ts = np.ascontiguousarray(token_scales, dtype=np.float32)
    N, nb = ts.shape
    H = nb * 128
    if scale_mode == SCALE_COLS:
        sshape, sdtype = (E, nb, M), np.float32
    else:
        sshape, sdtype = (E, H // 512, M), np.int32
    if scales is None:
        scales = np.zeros(sshape, sdtype)
    assert scales.shape == sshape and scales.dtype == sdtype and scales.flags.c_contiguous
    rp = np.ascontiguousarray(row_pair, dtype=np.int32).reshape(-1)
    assert rp.size >= E * M
    rc = lib().oracle_scatter_scales(_ptr(ts), nb, N, K, H, _ptr(rp), E, M, _ptr(scales),
                                     scale_mode)
    if rc != OK:
        raise OracleError(rc, "scatter_scales")
    return scales


def f32_to_e4m3(x: float) -> int:
    return int(lib().oracle_f32_to_e4m3(x))


def e4m3_to_f32(c: int) -> float:
    return float(lib().oracle_e4m3_to_f32(c))


def fp8_block_scale(block: np.ndarray, round_scale: bool) -> float:
    b = np.ascontiguousarray(block, dtype=np.uint16)
    assert b.size == 128
    return float(lib().oracle_fp8_block_scale(_ptr(b), int(round_scale)))


def bf16_from_f64(x: float) -> int:
    return int(lib().oracle_bf16_from_f64(x))


def f32_to_bf16(x: float) -> int:
    return int(lib().oracle_f32_to_bf16(x))


def bf16_to_f32(b: int) -> float:
    return float(lib().oracle_bf16_to_f32(b))
