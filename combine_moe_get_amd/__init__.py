"""Python binding of libmoe_get.so: MoE routing layout, dispatch and combine
on one MI355X (gfx950).

The functions named like the C ABI (``moe_get_layout``, ``moe_dispatch``,
``moe_combine``, ...) only check tensor shapes, dtypes and alignment and pass
device pointers plus ``torch.cuda.current_stream()`` to the library; every
step of the path runs in the library's HIP kernels. PyTorch provides device
memory and streams only. There is no CPU path: importing this package fails
if the library has not been built (``python combine_moe_get_amd/build.py``).

Convenience wrappers (``layout``, ``dispatch``, ``combine``,
``pack_records``, ``unpack_records``) allocate outputs with torch and call the
same entry points. Given ``stream=``, they allocate on that stream, so that
torch's caching allocator orders any reuse of those blocks (the layout's
workspace is freed on return) after the kernels that stream runs; inputs
must be ready on that stream, which is the caller's ordering.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch  # loaded first so the library binds to the same HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_DEBUG=1 loads the debug build, in which every layout call also checks
# its outputs on the device (read the counts with debug_status()).
DEBUG = os.environ.get("MOE_DEBUG", "") == "1"
LIB_PATH = os.path.join(_PKG, "libmoe_get_debug.so" if DEBUG else "libmoe_get.so")

MOE_OK = 0
MOE_ERR_ARG = -1
MOE_ERR_ALIGN = -2
MOE_ERR_LIMIT = -3
MOE_ERR_CAPACITY = -4
MOE_ERR_WORKSPACE = -5
MOE_ERR_HIP = -6
MOE_SCALE_ROWS = 0
MOE_SCALE_COLS = 1
MOE_SCALE_UE8M0 = 2
MOE_SCALE_TOKENS = 3
MAX_TOPK = 32
MAX_EXPERTS = 1024
MAX_FIELDS = 4

_ERR_NAMES = {MOE_ERR_ARG: "MOE_ERR_ARG", MOE_ERR_ALIGN: "MOE_ERR_ALIGN",
              MOE_ERR_LIMIT: "MOE_ERR_LIMIT", MOE_ERR_CAPACITY: "MOE_ERR_CAPACITY",
              MOE_ERR_WORKSPACE: "MOE_ERR_WORKSPACE", MOE_ERR_HIP: "MOE_ERR_HIP"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python combine_moe_get_amd/build.py` "
                      "(there is no fallback path)")


class moe_field(ctypes.Structure):
    _fields_ = [("src", ctypes.c_void_p), ("src_row_stride", ctypes.c_int64),
                ("dst", ctypes.c_void_p), ("dst_row_stride", ctypes.c_int64),
                ("row_bytes", ctypes.c_int64)]


class moe_epilogue(ctypes.Structure):
    _fields_ = [("bias0", ctypes.c_void_p), ("bias0_row_stride", ctypes.c_int64),
                ("bias1", ctypes.c_void_p), ("bias1_row_stride", ctypes.c_int64),
                ("residual", ctypes.c_void_p), ("residual_row_stride", ctypes.c_int64),
                ("gamma", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("residual_out", ctypes.c_void_p), ("residual_out_row_stride", ctypes.c_int64)]


def _load(path: str = LIB_PATH):
    """The library at `path` (default: the one selected above) with every
    entry point's argument and result types set."""
    L = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.moe_version.restype = ctypes.c_int
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_required_capacity.argtypes = [i32, i32, i32, i32]
    L.moe_required_capacity.restype = i64
    L.moe_layout_workspace_bytes.argtypes = [i32, i32, i32]
    L.moe_layout_workspace_bytes.restype = sz
    L.moe_get_layout.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, i64, P, P, sz, P, P]
    L.moe_get_layout.restype = ctypes.c_int
    L.moe_get_layout_noalloc.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, i64, P, P, P]
    L.moe_get_layout_noalloc.restype = ctypes.c_int
    L.moe_dispatch.argtypes = [ctypes.POINTER(moe_field), i32, i32, i32, P, P, P]
    L.moe_dispatch.restype = ctypes.c_int
    L.moe_combine.argtypes = [P, i64, P, i64, P, i32, i32, i32, P, i64, P]
    L.moe_combine.restype = ctypes.c_int
    L.moe_get_layout_padded.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, P, P, sz, P, P]
    L.moe_get_layout_padded.restype = ctypes.c_int
    L.moe_dispatch_fp8.argtypes = [P, i64, i32, i32, i32, P, P, i64, P, i32, i64, i32, i32, P]
    L.moe_dispatch_fp8.restype = ctypes.c_int
    L.moe_combine_epilogue.argtypes = [P, i64, P, i64, P, i32, i32, i32,
                                       ctypes.POINTER(moe_epilogue), P, i64, P]
    L.moe_combine_epilogue.restype = ctypes.c_int
    L.moe_record_offsets.argtypes = [P, i32, P]
    L.moe_record_offsets.restype = i64
    L.moe_pack_records.argtypes = [ctypes.POINTER(moe_field), i32, i32, P, i64, P]
    L.moe_pack_records.restype = ctypes.c_int
    L.moe_unpack_records.argtypes = [P, i64, i32, ctypes.POINTER(moe_field), i32, P]
    L.moe_unpack_records.restype = ctypes.c_int
    L.moe_layout_dispatch.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, P, i64, P,
                                      ctypes.POINTER(moe_field), i32, P]
    L.moe_layout_dispatch.restype = ctypes.c_int
    L.moe_dispatch_fp8_padded.argtypes = [P, i64, i32, i32, i32, i32, P, i64, i32, P, P, P, P, P, P,
                                          P, i64, P, i32, i64, i32, P]
    L.moe_dispatch_fp8_padded.restype = ctypes.c_int
    L.moe_dispatch_backward.argtypes = [P, i64, P, i64, P, i32, i32, i32, P, i64, P, i64, P]
    L.moe_dispatch_backward.restype = ctypes.c_int
    L.moe_combine_backward.argtypes = [P, i64, P, i64, P, i64, P, i32, i32, i32, P, i64, P, i64,
                                       P]
    L.moe_combine_backward.restype = ctypes.c_int
    L.moe_scatter_scales.argtypes = [P, i64, i32, i32, i32, P, i32, i32, P, i32, P]
    L.moe_scatter_scales.restype = ctypes.c_int
    L.moe_check_layout.argtypes = [P, i32, i32, P, i64, P, P, P]
    L.moe_check_layout.restype = ctypes.c_int
    L.moe_debug_status.argtypes = [P, i32, P]
    L.moe_debug_status.restype = ctypes.c_int
    return L


try:
    _lib = _load()
except AttributeError as exc:   # a library built from older sources
    raise ImportError(f"{LIB_PATH} lacks an entry point ({exc}); rebuild it with "
                      "`python combine_moe_get_amd/build.py`") from None


class MoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {message}")
        self.code = code


def _check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, _lib.moe_last_error().decode(errors="replace"))


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on(stream):
    """Context under which a wrapper allocates: the launch stream when one is
    given (torch's caching allocator then reuses the blocks only in that
    stream's order), else the current stream."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _dev(t: Optional[torch.Tensor], name: str) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr()


def _rows(t: torch.Tensor, name: str) -> Tuple[int, int]:
    """(pointer, row stride in elements) of a 2-D tensor with contiguous rows."""
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.numel() == 0:
        return _dev(t, name), t.shape[1]
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return _dev(t, name), t.stride(0) if t.shape[0] > 1 else max(t.stride(0), t.shape[1])


def version() -> int:
    return int(_lib.moe_version())


# ---------------------------------------------------------------------------
# Entry points named like the C ABI (marshalling only).
# ---------------------------------------------------------------------------

def moe_required_capacity(N: int, K: int, E: int, align: int = 1) -> int:
    return int(_lib.moe_required_capacity(N, K, E, align))


def moe_layout_workspace_bytes(N: int, K: int, E: int) -> int:
    return int(_lib.moe_layout_workspace_bytes(N, K, E))


def _layout_outputs(ids, num_experts, counts, offsets, pos, row_pair, order, status):
    if ids.dtype != torch.int32:
        raise TypeError("ids must be int32")
    for n, t in (("counts", counts), ("offsets", offsets), ("pos", pos), ("row_pair", row_pair),
                 ("order", order)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise TypeError(f"{n} must be a contiguous int32 tensor")
    if status is not None and (status.dtype != torch.int32 or status.numel() < 1):
        raise TypeError("status must be an int32 tensor with at least one element")
    N, K = ids.shape
    if counts.numel() < num_experts or offsets.numel() < num_experts + 1 or pos.numel() < N * K:
        raise ValueError("counts, offsets or pos too small")
    if order is not None and order.numel() < N * K:
        raise ValueError("order needs N*K entries")


def moe_get_layout(ids: torch.Tensor, num_experts: int, align: int, counts: torch.Tensor,
                   offsets: torch.Tensor, pos: torch.Tensor, row_pair: torch.Tensor,
                   workspace: torch.Tensor, status: Optional[torch.Tensor] = None,
                   stream=None, order: Optional[torch.Tensor] = None) -> None:
    """ids: int32 [N, K] (rows may be strided, e.g. a view into records).
    order (optional, int32 [N*K]) receives the dispatch plan."""
    _layout_outputs(ids, num_experts, counts, offsets, pos, row_pair, order, status)
    N, K = ids.shape
    ip, istride = _rows(ids, "ids") if N > 0 else (0, K)
    _check(_lib.moe_get_layout(ip, istride, N, K, num_experts, align, _dev(counts, "counts"),
                               _dev(offsets, "offsets"), _dev(pos, "pos"),
                               _dev(row_pair, "row_pair"), row_pair.numel(),
                               _dev(order, "order"), _dev(workspace, "workspace"),
                               workspace.numel() * workspace.element_size(),
                               _dev(status, "status"), _stream(stream)))


def moe_get_layout_noalloc(ids: torch.Tensor, num_experts: int, align: int,
                           counts: torch.Tensor, offsets: torch.Tensor, pos: torch.Tensor,
                           row_pair: torch.Tensor, status: Optional[torch.Tensor] = None,
                           stream=None, order: Optional[torch.Tensor] = None) -> None:
    """moe_get_layout without a workspace argument: the library's own static
    scratch on the stream's GPU is used instead, so nothing is allocated.
    Calls that overlap on one GPU race on that scratch."""
    _layout_outputs(ids, num_experts, counts, offsets, pos, row_pair, order, status)
    N, K = ids.shape
    ip, istride = _rows(ids, "ids") if N > 0 else (0, K)
    _check(_lib.moe_get_layout_noalloc(ip, istride, N, K, num_experts, align,
                                       _dev(counts, "counts"), _dev(offsets, "offsets"),
                                       _dev(pos, "pos"), _dev(row_pair, "row_pair"),
                                       row_pair.numel(), _dev(order, "order"),
                                       _dev(status, "status"), _stream(stream)))


def _range_and_stats(layout_range, recv_stats, E):
    if layout_range is not None and (layout_range.dtype != torch.int64 or
                                     not layout_range.is_contiguous() or layout_range.numel() < E):
        raise TypeError("layout_range must be a contiguous int64 tensor of E entries")
    if recv_stats is not None and (recv_stats.dtype != torch.int32 or
                                   not recv_stats.is_contiguous() or recv_stats.numel() < E):
        raise TypeError("recv_stats must be a contiguous int32 tensor of E entries")


def moe_get_layout_padded(ids: torch.Tensor, num_experts: int, rows_per_expert: int,
                          counts: torch.Tensor, pos: torch.Tensor, row_pair: torch.Tensor,
                          workspace: torch.Tensor, status: Optional[torch.Tensor] = None,
                          stream=None, layout_range: Optional[torch.Tensor] = None,
                          recv_stats: Optional[torch.Tensor] = None) -> None:
    """Padded per-expert layout: expert e owns rows e*M .. e*M+M-1.
    layout_range (int64 [E]) receives each expert's (begin << 32) | count;
    counts are added to recv_stats (int32 [E])."""
    _range_and_stats(layout_range, recv_stats, num_experts)
    if ids.dtype != torch.int32:
        raise TypeError("ids must be int32")
    for n, t in (("counts", counts), ("pos", pos), ("row_pair", row_pair)):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 tensor")
    if status is not None and (status.dtype != torch.int32 or status.numel() < 2):
        raise TypeError("status must be an int32 tensor with at least two elements")
    N, K = ids.shape
    if (counts.numel() < num_experts or pos.numel() < N * K
            or row_pair.numel() < num_experts * rows_per_expert):
        raise ValueError("counts, pos or row_pair too small")
    ip, istride = _rows(ids, "ids") if N > 0 else (0, K)
    _check(_lib.moe_get_layout_padded(ip, istride, N, K, num_experts, rows_per_expert,
                                      _dev(counts, "counts"), _dev(pos, "pos"),
                                      _dev(row_pair, "row_pair"),
                                      _dev(layout_range, "layout_range"),
                                      _dev(recv_stats, "recv_stats"), _dev(workspace, "workspace"),
                                      workspace.numel() * workspace.element_size(),
                                      _dev(status, "status"), _stream(stream)))


def moe_dispatch_fp8(x: torch.Tensor, pos: Optional[torch.Tensor], K: int, dst: torch.Tensor,
                     scales: torch.Tensor, scale_format: int = MOE_SCALE_ROWS,
                     rows_per_expert: int = 0, round_scale: bool = False, stream=None) -> None:
    """Quantising dispatch: bf16 x [N, H] -> e4m3 codes in dst [rows, H]
    (uint8) at rows pos[t, k], scales as scale_format (see moe_get.h)."""
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if dst.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("dst must be uint8 or float8_e4m3fn")
    N, H = x.shape
    xp, xs = _rows(x, "x") if N else (0, H)
    dp, ds = _rows(dst, "dst") if dst.shape[0] else (0, H)
    if scale_format in (MOE_SCALE_ROWS, MOE_SCALE_TOKENS):
        if scales.dtype != torch.float32 or scales.dim() != 2 or scales.stride(1) != 1:
            raise TypeError("row or token scales must be float32 [rows, >= H/128] with "
                            "contiguous rows")
        srs = scales.stride(0)
    else:
        if not scales.is_contiguous():
            raise TypeError("column-major scales must be a contiguous tensor")
        srs = 0
    if pos is not None and (pos.dtype != torch.int32 or not pos.is_contiguous()
                            or pos.numel() != N * K):
        raise ValueError("pos must be a contiguous int32 [N, K] tensor")
    _check(_lib.moe_dispatch_fp8(xp, xs, N, K, H, _dev(pos, "pos"), dp, ds,
                                 _dev(scales, "scales"), scale_format, srs, rows_per_expert,
                                 int(bool(round_scale)), _stream(stream)))


def moe_scatter_scales(token_scales: torch.Tensor, K: int, H: int, row_pair: torch.Tensor,
                       num_experts: int, rows_per_expert: int, scales: torch.Tensor,
                       scale_format: int = MOE_SCALE_COLS, stream=None) -> None:
    """Column-major (fp32 [E, H/128, M]) or UE8M0 (int32 [E, H/512, M]) scales
    of the padded layout from token-major ones (fp32 [N, >= H/128], as written
    by moe_dispatch_fp8 with MOE_SCALE_TOKENS), placed by row_pair [E*M]."""
    if token_scales.dtype != torch.float32 or token_scales.dim() != 2 or \
            token_scales.stride(1) != 1:
        raise TypeError("token_scales must be float32 [N, >= H/128] with contiguous rows")
    if row_pair.dtype != torch.int32 or not row_pair.is_contiguous():
        raise TypeError("row_pair must be a contiguous int32 tensor")
    if not scales.is_contiguous():
        raise TypeError("scales must be a contiguous tensor")
    E, M = num_experts, rows_per_expert
    if row_pair.numel() < E * M:
        raise ValueError("row_pair has fewer than E*M entries")
    per_word = 128 if scale_format == MOE_SCALE_COLS else 512
    if scales.numel() < E * M * (H // per_word):
        raise ValueError("scales too small for [E, H/%d, M]" % per_word)
    N = token_scales.shape[0]
    _check(_lib.moe_scatter_scales(_dev(token_scales, "token_scales"), token_scales.stride(0), N,
                                   K, H, _dev(row_pair, "row_pair"), E, M,
                                   _dev(scales, "scales"), scale_format, _stream(stream)))


def _as_bytes2d(t: torch.Tensor, name: str) -> Tuple[int, int, int]:
    """(pointer, row stride in bytes, row bytes) of a 2-D tensor with
    contiguous rows, any dtype."""
    ptr, stride = _rows(t, name)
    es = t.element_size()
    return ptr, stride * es, t.shape[1] * es


def moe_dispatch(srcs: Sequence[torch.Tensor], dsts: Sequence[torch.Tensor],
                 pos: Optional[torch.Tensor], K: int, stream=None,
                 order: Optional[torch.Tensor] = None) -> None:
    """Copy row t of every srcs[f] into rows pos[t, k] of dsts[f].

    ``pos=None`` is the identity (K must be 1). Tensors are 2-D with
    contiguous rows; each field's row size in bytes must match. ``order``
    (the layout's dispatch plan) sets the order the pairs are visited in."""
    N = srcs[0].shape[0] if len(srcs) else 0
    arr = _fields(srcs, dsts, N)
    if pos is not None and (pos.dtype != torch.int32 or not pos.is_contiguous()
                            or pos.numel() != N * K):
        raise ValueError("pos must be a contiguous int32 [N, K] tensor")
    if order is not None and (order.dtype != torch.int32 or not order.is_contiguous()
                              or order.numel() != N * K):
        raise ValueError("order must be a contiguous int32 tensor of N*K entries")
    _check(_lib.moe_dispatch(arr, len(srcs), N, K, _dev(pos, "pos"), _dev(order, "order"),
                             _stream(stream)))


def _fields(srcs: Sequence[torch.Tensor], dsts: Sequence[torch.Tensor], N: int):
    """moe_field array of matching source [N, ...] / destination tensors."""
    if len(srcs) != len(dsts) or not 1 <= len(srcs) <= MAX_FIELDS:
        raise ValueError("need 1..4 matching source / destination fields")
    arr = (moe_field * len(srcs))()
    for i, (s, d) in enumerate(zip(srcs, dsts)):
        if s.shape[0] != N:
            raise ValueError("all sources need the same number of tokens")
        sp, ss, sb = _as_bytes2d(s, f"srcs[{i}]")
        dp, ds, db = _as_bytes2d(d, f"dsts[{i}]")
        if sb != db:
            raise ValueError(f"field {i}: source rows {sb} B, destination rows {db} B")
        arr[i] = moe_field(sp, ss, dp, ds, sb)
    return arr


def moe_combine(y: torch.Tensor, weights: torch.Tensor, pos: torch.Tensor, out: torch.Tensor,
                stream=None) -> None:
    """out [N, Hc] bf16 = sum_k weights[t, k] * y[pos[t, k]] (fp32 accumulate)."""
    if y.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("y and out must be bfloat16")
    if weights.dtype != torch.float32:
        raise TypeError("weights must be float32")
    if pos.dtype != torch.int32 or not pos.is_contiguous() or pos.dim() != 2:
        raise TypeError("pos must be a contiguous int32 [N, K] tensor")
    N, K = pos.shape
    Hc = out.shape[1]
    if y.shape[1] != Hc or out.shape[0] != N or tuple(weights.shape) != (N, K):
        raise ValueError("shape mismatch between y, weights, pos and out")
    yp, ys = _rows(y, "y") if y.shape[0] else (_dev(y, "y"), Hc)
    wp, ws = _rows(weights, "weights") if N else (0, K)
    op, os_ = _rows(out, "out") if N else (0, Hc)
    _check(_lib.moe_combine(yp, ys, wp, ws, _dev(pos, "pos"), N, K, Hc, op, os_,
                            _stream(stream)))


def moe_layout_dispatch(ids: torch.Tensor, num_experts: int, align: int, counts: torch.Tensor,
                        offsets: torch.Tensor, pos: torch.Tensor, row_pair: torch.Tensor,
                        status: Optional[torch.Tensor], srcs: Sequence[torch.Tensor],
                        dsts: Sequence[torch.Tensor], stream=None) -> None:
    """moe_get_layout + moe_dispatch in one launch (N*K <= 8192)."""
    if ids.dtype != torch.int32 or ids.dim() != 2:
        raise TypeError("ids must be int32 [N, K]")
    N, K = ids.shape
    for t, n in ((counts, "counts"), (offsets, "offsets"), (pos, "pos"), (row_pair, "row_pair")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 tensor")
    if status is not None and (status.dtype != torch.int32 or status.numel() < 1):
        raise TypeError("status must be an int32 tensor")
    if counts.numel() < num_experts or offsets.numel() < num_experts + 1 or pos.numel() != N * K:
        raise ValueError("counts, offsets or pos too small")
    fields = _fields(srcs, dsts, N)
    ip, istr = _rows(ids, "ids") if N else (0, K)
    _check(_lib.moe_layout_dispatch(ip, istr, N, K, num_experts, align, _dev(counts, "counts"),
                                    _dev(offsets, "offsets"), _dev(pos, "pos"),
                                    _dev(row_pair, "row_pair"), row_pair.numel(),
                                    _dev(status, "status"), fields, len(srcs), _stream(stream)))


def moe_dispatch_fp8_padded(ids: torch.Tensor, num_experts: int, rows_per_expert: int,
                            x: torch.Tensor, counts: torch.Tensor, pos: torch.Tensor,
                            row_pair: torch.Tensor, status: torch.Tensor, dst: torch.Tensor,
                            scales: torch.Tensor, scale_format: int = MOE_SCALE_COLS,
                            round_scale: bool = False, stream=None,
                            layout_range: Optional[torch.Tensor] = None,
                            recv_stats: Optional[torch.Tensor] = None) -> None:
    """moe_get_layout_padded + moe_dispatch_fp8 in one launch (N*K <= 8192)."""
    _range_and_stats(layout_range, recv_stats, num_experts)
    if ids.dtype != torch.int32 or ids.dim() != 2:
        raise TypeError("ids must be int32 [N, K]")
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if dst.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("dst must be uint8 or float8_e4m3fn")
    for t, n in ((counts, "counts"), (pos, "pos"), (row_pair, "row_pair"), (status, "status")):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous int32 tensor")
    N, K = ids.shape
    E, M = num_experts, rows_per_expert
    H = x.shape[1]
    if x.shape[0] != N or pos.numel() != N * K or counts.numel() < E or \
            row_pair.numel() < E * M or status.numel() < 2:
        raise ValueError("shape mismatch between ids, x, counts, pos, row_pair and status")
    ip, istr = _rows(ids, "ids") if N else (0, K)
    xp, xs = _rows(x, "x") if N else (0, H)
    dp, ds = _rows(dst, "dst") if dst.shape[0] else (0, H)
    if scale_format in (MOE_SCALE_ROWS, MOE_SCALE_TOKENS):
        if scales.dtype != torch.float32 or scales.dim() != 2 or scales.stride(1) != 1:
            raise TypeError("row or token scales must be float32 [rows, >= H/128] with "
                            "contiguous rows")
        srs = scales.stride(0)
    else:
        if not scales.is_contiguous():
            raise TypeError("column-major scales must be a contiguous tensor")
        srs = 0
    _check(_lib.moe_dispatch_fp8_padded(ip, istr, N, K, E, M, xp, xs, H, _dev(counts, "counts"),
                                        _dev(pos, "pos"), _dev(row_pair, "row_pair"),
                                        _dev(layout_range, "layout_range"),
                                        _dev(recv_stats, "recv_stats"),
                                        _dev(status, "status"), dp, ds, _dev(scales, "scales"),
                                        scale_format, srs, int(bool(round_scale)),
                                        _stream(stream)))


def moe_dispatch_backward(grad_recv: torch.Tensor, pos: torch.Tensor, grad_x: torch.Tensor,
                          grad_recv_w: Optional[torch.Tensor] = None,
                          grad_w: Optional[torch.Tensor] = None, stream=None) -> None:
    """grad_x [N, H] bf16 = sum over valid k of grad_recv[pos[t, k]] (fp32
    accumulate); with grad_recv_w [rows, K] fp32, also grad_w [N, K] fp32 =
    the same sum of grad_recv_w rows."""
    if grad_recv.dtype != torch.bfloat16 or grad_x.dtype != torch.bfloat16:
        raise TypeError("grad_recv and grad_x must be bfloat16")
    if pos.dtype != torch.int32 or not pos.is_contiguous() or pos.dim() != 2:
        raise TypeError("pos must be a contiguous int32 [N, K] tensor")
    if (grad_recv_w is None) != (grad_w is None):
        raise ValueError("grad_recv_w and grad_w go together")
    N, K = pos.shape
    H = grad_x.shape[1]
    if grad_recv.shape[1] != H or grad_x.shape[0] != N:
        raise ValueError("shape mismatch between grad_recv, pos and grad_x")
    gp, gs = _rows(grad_recv, "grad_recv") if grad_recv.shape[0] else (_dev(grad_recv, "grad_recv"), H)
    xp, xs = _rows(grad_x, "grad_x") if N else (0, H)
    wp, ws, op, os_ = 0, K, 0, K
    if grad_w is not None:
        if grad_recv_w.dtype != torch.float32 or grad_w.dtype != torch.float32:
            raise TypeError("weight gradients must be float32")
        if grad_recv_w.shape[1] < K or tuple(grad_w.shape[:1]) != (N,) or grad_w.shape[1] < K:
            raise ValueError("grad_recv_w must be [rows, >= K] and grad_w [N, >= K]")
        wp, ws = _rows(grad_recv_w, "grad_recv_w") if grad_recv_w.shape[0] else (_dev(grad_recv_w, "grad_recv_w"), K)
        op, os_ = _rows(grad_w, "grad_w") if N else (0, K)
    _check(_lib.moe_dispatch_backward(gp, gs, wp, ws, _dev(pos, "pos"), N, K, H, xp, xs, op, os_,
                                      _stream(stream)))


def moe_combine_backward(grad_out: torch.Tensor, weights: torch.Tensor, pos: torch.Tensor,
                         grad_y: torch.Tensor, y: Optional[torch.Tensor] = None,
                         grad_w: Optional[torch.Tensor] = None, stream=None) -> None:
    """grad_y[pos[t, k]] = bf16(weights[t, k] * grad_out[t]); with y and
    grad_w [N, K] fp32, also grad_w[t, k] = <grad_out[t], y[pos[t, k]]>."""
    if grad_out.dtype != torch.bfloat16 or grad_y.dtype != torch.bfloat16:
        raise TypeError("grad_out and grad_y must be bfloat16")
    if weights.dtype != torch.float32:
        raise TypeError("weights must be float32")
    if pos.dtype != torch.int32 or not pos.is_contiguous() or pos.dim() != 2:
        raise TypeError("pos must be a contiguous int32 [N, K] tensor")
    if grad_w is not None and y is None:
        raise ValueError("weight gradients need y")
    N, K = pos.shape
    Hc = grad_out.shape[1]
    if grad_out.shape[0] != N or grad_y.shape[1] != Hc or tuple(weights.shape[:1]) != (N,):
        raise ValueError("shape mismatch between grad_out, weights, pos and grad_y")
    gp, gs = _rows(grad_out, "grad_out") if N else (0, Hc)
    wp, ws = _rows(weights, "weights") if N else (0, K)
    yp, ys = 0, Hc
    if grad_w is not None:
        if y.dtype != torch.bfloat16 or y.shape[1] != Hc:
            raise TypeError("y must be bfloat16 [rows, Hc]")
        if grad_w.dtype != torch.float32 or grad_w.shape[0] != N or grad_w.shape[1] < K:
            raise TypeError("grad_w must be float32 [N, >= K]")
        yp, ys = _rows(y, "y") if y.shape[0] else (_dev(y, "y"), Hc)
    dp, ds = _rows(grad_y, "grad_y") if grad_y.shape[0] else (_dev(grad_y, "grad_y"), Hc)
    op, os_ = (_rows(grad_w, "grad_w") if N else (0, K)) if grad_w is not None else (0, K)
    _check(_lib.moe_combine_backward(gp, gs, wp, ws, yp, ys, _dev(pos, "pos"), N, K, Hc, dp, ds,
                                     op, os_, _stream(stream)))


def moe_combine_epilogue(y: torch.Tensor, weights: torch.Tensor, pos: torch.Tensor,
                         out: torch.Tensor, bias0: Optional[torch.Tensor] = None,
                         bias1: Optional[torch.Tensor] = None,
                         residual: Optional[torch.Tensor] = None,
                         gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                         residual_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """Combine, then + bias0 + bias1 and, with a residual, residual add
    (written to residual_out) and RMSNorm with gamma into out. All bf16."""
    if y.dtype != torch.bfloat16 or out.dtype != torch.bfloat16:
        raise TypeError("y and out must be bfloat16")
    if weights.dtype != torch.float32:
        raise TypeError("weights must be float32")
    if pos.dtype != torch.int32 or not pos.is_contiguous() or pos.dim() != 2:
        raise TypeError("pos must be a contiguous int32 [N, K] tensor")
    N, K = pos.shape
    Hc = out.shape[1]
    if y.shape[1] != Hc or out.shape[0] != N or tuple(weights.shape) != (N, K):
        raise ValueError("shape mismatch between y, weights, pos and out")

    def rows(t, name):
        if t is None:
            return 0, 0
        if t.dtype != torch.bfloat16 or tuple(t.shape) != (N, Hc):
            raise ValueError(f"{name} must be bfloat16 [N, Hc]")
        return _rows(t, name) if N else (_dev(t, name), Hc)

    ep = moe_epilogue()
    ep.bias0, ep.bias0_row_stride = rows(bias0, "bias0")
    ep.bias1, ep.bias1_row_stride = rows(bias1, "bias1")
    ep.residual, ep.residual_row_stride = rows(residual, "residual")
    ep.residual_out, ep.residual_out_row_stride = rows(residual_out, "residual_out")
    if gamma is not None:
        if gamma.dtype != torch.bfloat16 or gamma.numel() != Hc or not gamma.is_contiguous():
            raise ValueError("gamma must be a contiguous bfloat16 [Hc] tensor")
        ep.gamma = _dev(gamma, "gamma")
    ep.eps = eps
    yp, ys = _rows(y, "y") if y.shape[0] else (_dev(y, "y"), Hc)
    wp, ws = _rows(weights, "weights") if N else (0, K)
    op, os_ = _rows(out, "out") if N else (0, Hc)
    _check(_lib.moe_combine_epilogue(yp, ys, wp, ws, _dev(pos, "pos"), N, K, Hc,
                                     ctypes.byref(ep), op, os_, _stream(stream)))


def moe_check_layout(pos: torch.Tensor, row_pair: Optional[torch.Tensor],
                     order: Optional[torch.Tensor], status: torch.Tensor, stream=None) -> None:
    """Adds to status (int32 [4], device) the counts of a layout's
    inconsistencies: pos entries outside [-1, cap), pairs whose row does not
    name them, rows that name a pair not pointing back, plan entries that are
    not pairs with a row. cap = row_pair.numel() (row_pair may be None only
    with cap 0: then every valid pos counts as out of range)."""
    if pos.dim() != 2:
        raise ValueError("pos must be [N, K]")
    N, K = pos.shape
    for n, t in (("pos", pos), ("row_pair", row_pair), ("order", order), ("status", status)):
        if t is not None and (t.dtype != torch.int32 or not t.is_contiguous()):
            raise TypeError(f"{n} must be a contiguous int32 tensor")
    if status.numel() < 4:
        raise ValueError("status needs 4 entries")
    if order is not None and order.numel() != N * K:
        raise ValueError("order must hold N*K entries")
    cap = row_pair.numel() if row_pair is not None else 0
    _check(_lib.moe_check_layout(_dev(pos, "pos"), N, K, _dev(row_pair, "row_pair"), cap,
                                 _dev(order, "order"), _dev(status, "status"), _stream(stream)))


def debug_status(reset: bool = False, stream=None) -> Tuple[int, int, int, int, int]:
    """The debug build's counters (MOE_DEBUG=1): the sums of moe_check_layout's
    four counts over every layout call since the library loaded or the last
    reset, then the number of layout calls checked. Raises MoeError in the
    release build."""
    out = (ctypes.c_int32 * 5)()
    _check(_lib.moe_debug_status(ctypes.cast(out, ctypes.c_void_p), int(bool(reset)),
                                 _stream(stream)))
    return tuple(int(v) for v in out)


# ---------------------------------------------------------------------------
# Convenience wrappers that allocate their outputs.
# ---------------------------------------------------------------------------

@dataclass
class Layout:
    counts: torch.Tensor      # int32 [E]
    offsets: torch.Tensor     # int32 [E+1]
    pos: torch.Tensor         # int32 [N, K]
    row_pair: torch.Tensor    # int32 [cap]
    status: torch.Tensor      # int32 [1]: ids >= E seen
    num_experts: int
    align: int
    order: Optional[torch.Tensor] = None   # int32 [N*K]: the dispatch plan

    @property
    def cap(self) -> int:
        return self.row_pair.numel()

    @property
    def K(self) -> int:
        return self.pos.shape[1]


def layout(ids: torch.Tensor, num_experts: int, align: int = 1, cap: Optional[int] = None,
           workspace: Optional[torch.Tensor] = None, stream=None) -> Layout:
    N, K = ids.shape
    if cap is None:
        cap = moe_required_capacity(N, K, num_experts, align)
        if cap < 0:
            raise MoeError(MOE_ERR_ARG, "invalid layout sizes")
    dev = ids.device
    with _on(stream):
        if workspace is None:
            nbytes = moe_layout_workspace_bytes(N, K, num_experts)
            workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        lay = Layout(torch.empty(num_experts, dtype=torch.int32, device=dev),
                     torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
                     torch.empty((N, K), dtype=torch.int32, device=dev),
                     torch.empty(max(cap, 0), dtype=torch.int32, device=dev),
                     torch.empty(1, dtype=torch.int32, device=dev), num_experts, align,
                     torch.empty(N * K, dtype=torch.int32, device=dev))
        moe_get_layout(ids, num_experts, align, lay.counts, lay.offsets, lay.pos, lay.row_pair,
                       workspace, lay.status, stream, order=lay.order)
    return lay


def dispatch(srcs: Sequence[torch.Tensor], lay: Layout, stream=None) -> List[torch.Tensor]:
    """Receive buffers [cap, ...] of every field, filled at the rows ``lay``
    assigned (other rows are left uninitialized)."""
    with _on(stream):
        dsts = [torch.empty((lay.cap,) + tuple(s.shape[1:]), dtype=s.dtype, device=s.device)
                for s in srcs]
        moe_dispatch(srcs, dsts, lay.pos, lay.K, stream, order=lay.order)
    return dsts


def combine(y: torch.Tensor, weights: torch.Tensor, lay: Layout,
            out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    N = lay.pos.shape[0]
    with _on(stream):
        if out is None:
            out = torch.empty((N, y.shape[1]), dtype=torch.bfloat16, device=y.device)
        moe_combine(y, weights, lay.pos, out, stream)
    return out


def record_offsets(row_bytes: Sequence[int]) -> Tuple[List[int], int]:
    """16-byte aligned offset of each field inside a per-token record and the
    record size rounded up to 16 bytes (fields in the given order), from the
    library's moe_record_offsets."""
    n = len(row_bytes)
    rb = (ctypes.c_int64 * max(n, 1))(*row_bytes)
    offs = (ctypes.c_int64 * max(n, 1))()
    size = _lib.moe_record_offsets(rb, n, offs)
    if size < 0:
        _check(int(size))
    return list(offs[:n]), int(size)


def _bytes2d(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.uint8) if t.dim() == 2 else t.reshape(t.shape[0], -1).view(torch.uint8)


def _record_fields(tensors: Sequence[torch.Tensor], as_src: bool):
    arr = (moe_field * len(tensors))()
    for i, t in enumerate(tensors):
        p, s, b = _as_bytes2d(t, f"field {i}")
        arr[i] = moe_field(p, s, 0, 0, b) if as_src else moe_field(0, 0, p, s, b)
    return arr


def pack_records(tensors: Sequence[torch.Tensor], stream=None) -> torch.Tensor:
    """Pack per-token tensors (e.g. ids, weights, hidden, scales) into one
    uint8 record per token, each field at a 16-byte aligned offset
    (moe_pack_records)."""
    if not 1 <= len(tensors) <= MAX_FIELDS:
        raise ValueError("need 1..4 tensors")
    N = tensors[0].shape[0]
    b = [_bytes2d(t) for t in tensors]
    if any(x.shape[0] != N for x in b):
        raise ValueError("all tensors need the same number of tokens")
    _, rec_bytes = record_offsets([x.shape[1] for x in b])
    with _on(stream):
        rec = torch.zeros((N, rec_bytes), dtype=torch.uint8, device=tensors[0].device)
        _check(_lib.moe_pack_records(_record_fields(b, True), len(b), N, _dev(rec, "records"),
                                     rec_bytes, _stream(stream)))
    return rec


def unpack_records(records: torch.Tensor, like: Sequence[torch.Tensor],
                   stream=None) -> List[torch.Tensor]:
    """Inverse of ``pack_records``: tensors shaped like ``like`` (row count
    taken from ``records``; moe_unpack_records)."""
    if not 1 <= len(like) <= MAX_FIELDS:
        raise ValueError("need 1..4 tensors")
    N = records.shape[0]
    with _on(stream):
        outs = [torch.empty((N,) + tuple(t.shape[1:]), dtype=t.dtype, device=records.device)
                for t in like]
        b = [_bytes2d(o) for o in outs]
        rp, rs = _rows(records, "records") if N else (0, records.shape[1])
        _check(_lib.moe_unpack_records(rp, rs, N, _record_fields(b, False), len(b),
                                       _stream(stream)))
    return outs
