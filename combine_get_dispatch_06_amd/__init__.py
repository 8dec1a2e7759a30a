"""MoE expert-parallel layout / dispatch / combine on AMD MI355X (gfx950).

A thin binding over libcgd, whose C ABI is declared in include/cgd.h. This
module only marshals arguments: every step of the path runs in libcgd's HIP
kernels, on the caller's current HIP stream. PyTorch supplies device memory
and streams.

Expert-granular path (one received row per selected expert):

    ntpr, _, ntpe, is_token_in_rank, _ = get_dispatch_layout(topk_idx, num_experts, num_ranks)
    recv_x, num_recv_tokens_per_expert, handle = dispatch(x, topk_idx, num_experts, num_ranks)
    recv_x2, _, _ = dispatch(x2, handle=handle)         # cached: reuses the layout
    combined = combine(expert_out, handle, topk_weights)
    layout, plan = layout_and_dispatch_plan(topk_idx, num_experts, num_ranks)   # one routing pass
    recv_x, num_recv_tokens_per_expert, handle = dispatch_apply(x, plan)
    layout, recv_x, num_recv_tokens_per_expert, handle = layout_and_dispatch(x, topk_idx, num_experts, num_ranks)

Rank-granular path (normal mode, one row per (token, flagged rank)):

    recv_x, recv_topk_idx, recv_topk_weights, num_recv_per_expert, h = normal_dispatch(
        x, is_token_in_rank, ntpe, topk_idx, topk_weights, num_experts=E)
    layout, plan = layout_and_normal_dispatch_plan(topk_idx, E, R)     # one launch
    recv_x, recv_topk_idx, recv_topk_weights, _, h = normal_dispatch_apply(x, plan, topk_idx, topk_weights)
    combined_x, combined_topk_weights = normal_combine(expert_out, h, recv_topk_weights, bias=(b0, b1))

FP8 payload: per_token_cast_to_fp8 / per_token_cast_back; every dispatch
accepts and returns (codes, scales) tuples, and dispatch(..., cast_fp8=fmt)
casts on the way. Fixed-capacity packed layout (low-latency dispatch):
low_latency_dispatch / low_latency_combine. copy_(dst, src) is libcgd's plain
16-byte copy, the measured copy ceiling the bandwidths are compared with.

The calls follow the DeepEP-style Buffer API described by the DeepEP Python
interface notes ("4 Python接口", section "Dispatch API") and the
get_dispatch_layout API page ("Interface", "Return Values"); the tuple order of
get_dispatch_layout is kept, with None in the num_tokens_per_rdma_rank and
event slots (single node, stream-ordered calls).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = ["get_dispatch_layout", "dispatch", "dispatch_plan", "dispatch_apply", "combine", "DispatchHandle",
           "CgdError", "library_path", "dispatch_capacity", "load", "normal_capacity", "NormalHandle",
           "normal_dispatch", "normal_dispatch_plan", "normal_dispatch_apply", "NormalPlan", "normal_combine",
           "per_token_cast_to_fp8", "per_token_cast_back", "SCALE_F32", "SCALE_POW2", "SCALE_UE8M0",
           "PackedHandle", "low_latency_dispatch", "layout_and_low_latency_dispatch", "low_latency_combine", "layout_and_dispatch_plan", "copy_",
           "layout_and_normal_dispatch_plan", "layout_and_dispatch", "normal_workspace_bytes",
           "layout_and_normal_workspace_bytes", "empty_", "layout_and_dispatch_noalloc", "init",
           "layout_and_normal_dispatch"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_BUILT_LIB = os.path.join(_PKG, "libcgd.so")
# CGD_LIBRARY names another build of libcgd to load instead (e.g. one with
# host-side sanitizers); it must exist, nothing is built for it
_LIB_PATH = os.environ.get("CGD_LIBRARY") or _BUILT_LIB

CGD_OK = 0
_STATUS = {-1: "invalid argument", -2: "capacity", -3: "workspace", -4: "HIP error"}


class CgdError(RuntimeError):
    """A libcgd call returned a non-OK status."""

    def __init__(self, call: str, status: int, message: str):
        super().__init__(f"{call}: {_STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


_lib = None


def load():
    """Load libcgd.so (building it first only if no build exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        if _LIB_PATH != _BUILT_LIB:
            raise FileNotFoundError(f"CGD_LIBRARY names {_LIB_PATH}, which does not exist")
        from . import build as _build
        _build.build()
    _lib = configure(ctypes.CDLL(_LIB_PATH))
    return _lib


def configure(lib):
    """Declare the C signatures of libcgd's entry points on a loaded library."""
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.cgd_version.restype = ctypes.c_char_p
    lib.cgd_version.argtypes = []
    lib.cgd_last_error.restype = ctypes.c_char_p
    lib.cgd_last_error.argtypes = []
    lib.cgd_init.restype = i32
    lib.cgd_init.argtypes = []
    lib.cgd_layout_workspace_bytes.restype = sz
    lib.cgd_layout_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.cgd_dispatch_workspace_bytes.restype = sz
    lib.cgd_dispatch_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.cgd_dispatch_capacity.restype = i64
    lib.cgd_dispatch_capacity.argtypes = [i64, i32, i32, i32]
    lib.cgd_get_dispatch_layout.restype = i32
    lib.cgd_get_dispatch_layout.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    lib.cgd_dispatch.restype = i32
    lib.cgd_dispatch.argtypes = [vp, i64, i32, vp, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.cgd_dispatch_plan.restype = i32
    lib.cgd_dispatch_plan.argtypes = [vp, i64, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, sz, vp]
    lib.cgd_layout_and_dispatch.restype = i32
    lib.cgd_layout_and_dispatch.argtypes = [vp, i64, i32, vp, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]
    lib.cgd_layout_and_dispatch_noalloc.restype = i32
    lib.cgd_layout_and_dispatch_noalloc.argtypes = [vp, i64, i32, vp, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp,
                                                    vp, vp, vp]
    lib.cgd_layout_and_dispatch_plan.restype = i32
    lib.cgd_layout_and_dispatch_plan.argtypes = [vp, i64, i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                                 sz, vp]
    lib.cgd_packed_workspace_bytes.restype = sz
    lib.cgd_packed_workspace_bytes.argtypes = [i64, i32, i32]
    lib.cgd_dispatch_packed.restype = i32
    lib.cgd_dispatch_packed.argtypes = [vp, i64, i32, vp, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.cgd_dispatch_packed_cast_fp8.restype = i32
    lib.cgd_dispatch_packed_cast_fp8.argtypes = [vp, i64, i32, vp, i32, i32, i32, i64, i32, vp, vp, vp, vp, vp, vp,
                                                 vp, sz, vp]
    lib.cgd_layout_and_dispatch_packed.restype = i32
    lib.cgd_layout_and_dispatch_packed.argtypes = [vp, i64, i32, vp, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp,
                                                   vp, vp, sz, vp]
    lib.cgd_layout_and_dispatch_packed_cast_fp8.restype = i32
    lib.cgd_layout_and_dispatch_packed_cast_fp8.argtypes = [vp, i64, i32, vp, i32, i32, i32, i64, i32, vp, vp, vp,
                                                            vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.cgd_dispatch_cached.restype = i32
    lib.cgd_dispatch_cached.argtypes = [vp, i64, i32, i32, vp, vp, i64, vp]
    lib.cgd_combine.restype = i32
    lib.cgd_combine.argtypes = [vp, i64, i32, vp, vp, i64, i32, vp, vp]
    lib.cgd_normal_workspace_bytes.restype = sz
    lib.cgd_normal_workspace_bytes.argtypes = [i64, i32]
    lib.cgd_normal_capacity.restype = i64
    lib.cgd_normal_capacity.argtypes = [i64, i32, i32]
    lib.cgd_normal_dispatch.restype = i32
    lib.cgd_normal_dispatch.argtypes = [vp, i64, i32, vp, vp, vp, vp, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp,
                                        vp, vp, vp, sz, vp]
    lib.cgd_normal_dispatch_plan.restype = i32
    lib.cgd_normal_dispatch_plan.argtypes = [vp, i64, i32, vp, i32, i32, vp, vp, vp, sz, vp]
    lib.cgd_normal_dispatch_apply.restype = i32
    lib.cgd_normal_dispatch_apply.argtypes = [vp, i64, i32, vp, vp, i32, i32, i32, vp, i64, vp, vp, vp, vp, vp, vp,
                                              sz, vp]
    lib.cgd_cast_to_fp8.restype = i32
    lib.cgd_cast_to_fp8.argtypes = [vp, i64, i32, vp, vp, i64, i64, i32, vp]
    lib.cgd_cast_back.restype = i32
    lib.cgd_cast_back.argtypes = [vp, vp, i64, i64, i32, i64, i32, vp, vp]
    lib.cgd_dispatch_cached_cast_fp8.restype = i32
    lib.cgd_dispatch_cached_cast_fp8.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp, i64, vp]
    lib.cgd_dispatch_cast_fp8.restype = i32
    lib.cgd_dispatch_cast_fp8.argtypes = [vp, i64, i32, vp, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp, vp, vp, vp,
                                          sz, vp]
    lib.cgd_layout_and_dispatch_cast_fp8.restype = i32
    lib.cgd_layout_and_dispatch_cast_fp8.argtypes = [vp, i64, i32, vp, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp,
                                                     vp, vp, vp, vp, vp, vp, sz, vp]
    lib.cgd_dispatch_cached_fp8.restype = i32
    lib.cgd_dispatch_cached_fp8.argtypes = [vp, vp, i64, i64, i32, i64, i32, i32, vp, vp, vp, i64, vp]
    lib.cgd_normal_dispatch_apply_fp8.restype = i32
    lib.cgd_normal_dispatch_apply_fp8.argtypes = [vp, vp, i64, i64, i32, i64, i32, vp, vp, i32, i32, i32, vp, vp,
                                                  i64, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.cgd_normal_dispatch_cached_fp8.restype = i32
    lib.cgd_normal_dispatch_cached_fp8.argtypes = [vp, vp, i64, i64, i32, i64, i32, i32, vp, vp, vp, i64, vp]
    lib.cgd_normal_dispatch_cached.restype = i32
    lib.cgd_normal_dispatch_cached.argtypes = [vp, i64, i32, i32, vp, vp, i64, vp]
    lib.cgd_normal_combine.restype = i32
    lib.cgd_normal_combine.argtypes = [vp, i64, i32, vp, i64, i32, vp, i32, vp, vp, vp, vp, vp]
    lib.cgd_copy.restype = i32
    lib.cgd_copy.argtypes = [vp, vp, i64, vp]
    lib.cgd_empty.restype = i32
    lib.cgd_empty.argtypes = [vp]
    lib.cgd_layout_and_normal_workspace_bytes.restype = sz
    lib.cgd_layout_and_normal_workspace_bytes.argtypes = [i64, i32, i32, i32]
    lib.cgd_layout_and_normal_dispatch.restype = i32
    lib.cgd_layout_and_normal_dispatch.argtypes = [vp, i64, i32, vp, vp, i32, i32, i32, i32, vp, i64, vp, vp, vp, vp,
                                                   vp, vp, vp, vp, vp, vp, sz, vp]
    lib.cgd_layout_and_normal_dispatch_cast_fp8.restype = i32
    lib.cgd_layout_and_normal_dispatch_cast_fp8.argtypes = [vp, i64, i32, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp,
                                                            vp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.cgd_layout_and_normal_dispatch_plan.restype = i32
    lib.cgd_layout_and_normal_dispatch_plan.argtypes = [vp, i64, i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]
    return lib


def _check(call: str, status: int):
    if status != CGD_OK:
        raise CgdError(call, status, load().cgd_last_error().decode())


def _dev_tensor(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


# One zero-initialised workspace per (device, stream, kind). libcgd leaves a
# workspace zeroed after every call, and calls on one stream are ordered, so a
# workspace is reused for every later call on that stream. A workspace that a
# larger call outgrows is replaced but kept alive until the process ends: a
# HIP graph captured earlier still launches kernels on its address. Sizes at
# least double on each replacement, so few are ever kept.
_workspaces: dict = {}
_outgrown: list = []

# Writes of plans into each workspace (by address): a rank-granular plan
# leaves its group words and tile bases there for the apply, so an apply
# checks that no later plan has overwritten them.
_plan_writes: dict = {}


def _workspace(device: torch.device, kind: str, nbytes: int) -> torch.Tensor:
    key = (device.index, torch.cuda.current_stream(device).cuda_stream, kind)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        size = max(nbytes, 256) if ws is None else max(nbytes, 2 * ws.numel())
        if ws is not None:
            _outgrown.append(ws)
        ws = torch.zeros(size, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _caller_workspace(ws: torch.Tensor, nbytes: int, device: torch.device) -> torch.Tensor:
    """A workspace the caller owns: uint8, contiguous, on the device, >= nbytes,
    256-byte aligned; it must be zero-filled before its first use."""
    _dev_tensor(ws, "workspace", torch.uint8, 1)
    if ws.device != device:
        raise ValueError("workspace must be on the inputs' device")
    if ws.numel() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes (got {ws.numel()})")
    if ws.data_ptr() % 256:
        raise ValueError("workspace must be 256-byte aligned")
    return ws


def _note_plan_write(ws: torch.Tensor) -> int:
    n = _plan_writes.get(ws.data_ptr(), 0) + 1
    _plan_writes[ws.data_ptr()] = n
    return n


# ---------------------------------------------------------------------------
# FP8 payload: (codes float8_e4m3fn [T, H], scales [T, H/128]) tuples.
# ---------------------------------------------------------------------------
SCALE_F32, SCALE_POW2, SCALE_UE8M0 = 0, 1, 2


def _fp8_parts(x, name: str = "x"):
    """Validate an FP8 tuple -> (codes uint8 view, scales, scale format for
    moving them, token stride, block stride)."""
    if not (isinstance(x, tuple) and len(x) == 2):
        raise TypeError(f"{name} must be a (codes, scales) tuple")
    q, sc = x
    if not isinstance(q, torch.Tensor) or q.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"{name} codes must be float8_e4m3fn (or uint8)")
    if q.dim() != 2 or not q.is_contiguous() or q.device.type != "cuda":
        raise ValueError(f"{name} codes must be a contiguous 2-D GPU tensor")
    if not isinstance(sc, torch.Tensor) or sc.dtype not in (torch.float32, torch.uint8) or sc.dim() != 2:
        raise TypeError(f"{name} scales must be a 2-D float32 (or uint8 UE8M0) tensor")
    T, H = q.shape
    if H % 128 != 0 or tuple(sc.shape) != (T, H // 128) or sc.device != q.device:
        raise ValueError(f"{name} scales must be [num_tokens, hidden/128] on the codes' device")
    fmt = SCALE_UE8M0 if sc.dtype == torch.uint8 else SCALE_F32
    return q.view(torch.uint8), sc, fmt, sc.stride(0), sc.stride(1)


def _fp8_empty(rows: int, H: int, fmt: int, dev):
    q = torch.empty((rows, H), dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
    sc = torch.empty((rows, H // 128), dtype=torch.uint8 if fmt == SCALE_UE8M0 else torch.float32, device=dev)
    return q, sc


def per_token_cast_to_fp8(x: torch.Tensor, scale_format: int = SCALE_F32, column_major_scales: bool = False):
    """bf16 [T, H] -> (codes float8_e4m3fn [T, H], scales [T, H/128]); the
    scales are fp32 (formats 0, 1) or UE8M0 bytes (format 2), optionally laid
    out column-major (a transposed view of a [H/128, T] buffer)."""
    lib = load()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    dev = x.device
    with torch.cuda.device(dev):
        q = torch.empty((T, H), dtype=torch.uint8, device=dev)
        sdt = torch.uint8 if scale_format == SCALE_UE8M0 else torch.float32
        if column_major_scales:
            sc = torch.empty((H // 128, T), dtype=sdt, device=dev).t()
        else:
            sc = torch.empty((T, H // 128), dtype=sdt, device=dev)
        _check("cgd_cast_to_fp8",
               lib.cgd_cast_to_fp8(_ptr(x), T, H, _ptr(q), _ptr(sc), sc.stride(0), sc.stride(1), scale_format,
                                   _stream(dev)))
    return q.view(torch.float8_e4m3fn), sc


def per_token_cast_back(x, scale_format: int | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """(codes, scales) -> bf16 [T, H]. scale_format defaults to the scales'
    dtype (uint8: UE8M0, float32: fp32 scale)."""
    lib = load()
    q, sc, fmt, st, sb = _fp8_parts(x)
    if scale_format is not None:
        if sc.dtype != _scale_dtype(scale_format):
            raise TypeError(f"scales must be {_scale_dtype(scale_format)} for scale format {scale_format}")
        fmt = scale_format
    T, H = q.shape
    dev = q.device
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        _dev_tensor(out, "out", torch.bfloat16, 2)
        _check("cgd_cast_back", lib.cgd_cast_back(_ptr(q), _ptr(sc), st, sb, fmt, T, H, _ptr(out), _stream(dev)))
    return out


def copy_(dst: torch.Tensor, src: torch.Tensor) -> torch.Tensor:
    """dst <- src bitwise with libcgd's plain 16-byte copy (the measured copy
    ceiling); contiguous device tensors of the same byte size."""
    lib = load()
    if not (src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous device tensors")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    with torch.cuda.device(src.device):
        _check("cgd_copy", lib.cgd_copy(_ptr(src), _ptr(dst), nbytes, _stream(src.device)))
    return dst


def init(device: torch.device | str | int | None = None) -> None:
    """Load libcgd's GPU code on the device now rather than inside the first
    call of each entry point (optional; allocates and enqueues nothing)."""
    lib = load()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(dev):
        _check("cgd_init", lib.cgd_init())


def empty_(device: torch.device | str | int | None = None) -> None:
    """Enqueue libcgd's empty kernel on the current stream of `device` (the
    launch floor that bench.py times beside the latency-bound calls)."""
    lib = load()
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    if dev.type != "cuda":
        raise ValueError("empty_ needs a GPU device")
    with torch.cuda.device(dev):
        _check("cgd_empty", lib.cgd_empty(_stream(dev)))


def dispatch_capacity(num_tokens: int, num_topk: int, num_experts: int, expert_alignment: int = 1) -> int:
    cap = int(load().cgd_dispatch_capacity(num_tokens, num_topk, num_experts, expert_alignment))
    if cap < 0:
        raise ValueError("invalid sizes for a receive buffer")
    return cap


def get_dispatch_layout(topk_idx: torch.Tensor, num_experts: int, num_ranks: int):
    """-> (num_tokens_per_rank int32 [R], None, num_tokens_per_expert int32 [E],
    is_token_in_rank bool [T,R], None)."""
    lib = load()
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    dev = topk_idx.device
    with torch.cuda.device(dev):
        ntpr = torch.empty(num_ranks, dtype=torch.int32, device=dev)
        ntpe = torch.empty(num_experts, dtype=torch.int32, device=dev)
        itr = torch.empty((T, num_ranks), dtype=torch.bool, device=dev)
        nbytes = lib.cgd_layout_workspace_bytes(T, K, num_experts, num_ranks)
        ws = _workspace(dev, "layout", nbytes)
        _check("cgd_get_dispatch_layout",
               lib.cgd_get_dispatch_layout(_ptr(topk_idx), T, K, num_experts, num_ranks, _ptr(ntpr), _ptr(ntpe),
                                           _ptr(itr), _ptr(ws), ws.numel(), _stream(dev)))
    return ntpr, None, ntpe, itr, None


@dataclass
class DispatchHandle:
    """Layout of one dispatch, reusable for cached dispatch and for combine.

    expert_offset int32 [E+1]: segment of expert e is rows [off[e], off[e+1]).
    recv_src_idx  int32 [recv_capacity]: source token of each row, -1 if none.
    dst_row       int32 [T, K]: receive row of each slot, -1 if not selected.
    num_recv_tokens_per_expert int32 [E]: aligned segment sizes (device).
    """
    expert_offset: torch.Tensor
    recv_src_idx: torch.Tensor
    dst_row: torch.Tensor
    num_recv_tokens_per_expert: torch.Tensor
    num_experts: int
    num_ranks: int
    expert_alignment: int
    recv_capacity: int

    @property
    def num_tokens(self) -> int:
        return self.dst_row.shape[0]

    @property
    def num_topk(self) -> int:
        return self.dst_row.shape[1]

    def num_recv_tokens_per_expert_list(self) -> list:
        """Aligned rows per expert as a host list (copies to the host and waits)."""
        return self.num_recv_tokens_per_expert.tolist()


def _scale_dtype(fmt: int) -> torch.dtype:
    """Storage of one scale: a UE8M0 byte (format 2), else fp32."""
    return torch.uint8 if fmt == SCALE_UE8M0 else torch.float32


def _recv_fp8(recv_x, cap: int, H: int, fmt: int, dev):
    """A caller's FP8 receive tuple, checked against the rows and the scale
    format the kernel will write (1-byte UE8M0 or 4-byte fp32 scales)."""
    if recv_x is None:
        return _fp8_empty(cap, H, fmt, dev)
    q, sc, _, st, sb = _fp8_parts(recv_x, "recv_x")
    if q.shape != (cap, H) or not sc.is_contiguous() or q.device != dev:
        raise ValueError("recv_x must be ([recv_capacity, hidden] codes, row-major [recv_capacity, hidden/128] scales) "
                         "on the inputs' device")
    if sc.dtype != _scale_dtype(fmt):
        raise TypeError(f"recv_x scales must be {_scale_dtype(fmt)} for scale format {fmt} (got {sc.dtype})")
    return recv_x


def dispatch(x, topk_idx: torch.Tensor | None = None, num_experts: int | None = None,
             num_ranks: int | None = None, expert_alignment: int = 1, handle: DispatchHandle | None = None,
             recv_capacity: int | None = None, recv_x=None, cast_fp8: int | None = None):
    """Scatter each token's row into the receive segments of its experts.

    x is bf16 [T, H], or the FP8 tuple (codes [T, H], scales [T, H/128]);
    with cast_fp8 = a scale format, a bf16 x is cast to FP8 on the way.
    Non-cached (handle=None): needs topk_idx, num_experts, num_ranks; returns
    (recv_x, num_recv_tokens_per_expert, DispatchHandle), the order of the
    outputs in the "Dispatch API" section of the DeepEP Python interface notes
    (num_recv_tokens_per_expert: int32 [E] on the device, each expert's row
    count rounded up to expert_alignment). Cached (handle given, topk_idx
    None): reuses the handle's layout; returns (recv_x, the handle's
    num_recv_tokens_per_expert, handle). recv_x is [recv_capacity, H] bf16, or
    an FP8 tuple for FP8 payloads. recv_capacity defaults to the worst case for
    the sizes, so no device-to-host copy is needed; rows past
    handle.expert_offset[-1] are unused.
    """
    lib = load()
    fp8 = isinstance(x, tuple)
    if fp8 and cast_fp8 is not None:
        raise ValueError("cast_fp8 casts a bf16 x; x is already an FP8 tuple")
    if fp8:
        q, sc, fmt, st, sb = _fp8_parts(x)
        T, H = q.shape
        dev = q.device
    else:
        _dev_tensor(x, "x", torch.bfloat16, 2)
        T, H = x.shape
        dev = x.device
    if handle is None and cast_fp8 is not None:
        if topk_idx is None or num_experts is None or num_ranks is None:
            raise ValueError("non-cached dispatch needs topk_idx, num_experts and num_ranks")
        _, recv_x, nre, h = _dispatch_cast(x, topk_idx, num_experts, num_ranks, expert_alignment, recv_capacity,
                                           recv_x, cast_fp8, layout=False)
        return recv_x, nre, h
    if handle is None and fp8:
        if topk_idx is None or num_experts is None or num_ranks is None:
            raise ValueError("non-cached dispatch needs topk_idx, num_experts and num_ranks")
        if recv_x is not None:  # checked before the plan is enqueued
            _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
            cap = recv_capacity
            if cap is None:
                cap = int(lib.cgd_dispatch_capacity(T, topk_idx.shape[1], num_experts, expert_alignment))
            _recv_fp8(recv_x, cap, H, fmt, dev)
        plan = dispatch_plan(topk_idx, num_experts, num_ranks, expert_alignment, recv_capacity)
        return dispatch_apply(x, plan, recv_x=recv_x)
    with torch.cuda.device(dev):
        if handle is not None:
            if topk_idx is not None:
                raise ValueError("cached dispatch takes handle and no topk_idx")
            if handle.num_tokens != T:
                raise ValueError("x has a different number of tokens than the handle")
            cap = handle.recv_capacity
            if cast_fp8 is not None and not fp8:
                recv_x = _recv_fp8(recv_x, cap, H, cast_fp8, dev)
                _check("cgd_dispatch_cached_cast_fp8",
                       lib.cgd_dispatch_cached_cast_fp8(_ptr(x), T, H, handle.num_topk, cast_fp8,
                                                        _ptr(handle.dst_row), _ptr(recv_x[0]), _ptr(recv_x[1]), cap,
                                                        _stream(dev)))
                return recv_x, handle.num_recv_tokens_per_expert, handle
            if fp8:
                recv_x = _recv_fp8(recv_x, cap, H, fmt, dev)
                _check("cgd_dispatch_cached_fp8",
                       lib.cgd_dispatch_cached_fp8(_ptr(q), _ptr(sc), st, sb, fmt, T, H, handle.num_topk,
                                                   _ptr(handle.dst_row), _ptr(recv_x[0]), _ptr(recv_x[1]), cap,
                                                   _stream(dev)))
                return recv_x, handle.num_recv_tokens_per_expert, handle
            if recv_x is None:
                recv_x = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
            _dev_tensor(recv_x, "recv_x", torch.bfloat16, 2)
            if recv_x.shape != (cap, H):
                raise ValueError("recv_x must be [recv_capacity, hidden]")
            _check("cgd_dispatch_cached",
                   lib.cgd_dispatch_cached(_ptr(x), T, H, handle.num_topk, _ptr(handle.dst_row), _ptr(recv_x), cap,
                                           _stream(dev)))
            return recv_x, handle.num_recv_tokens_per_expert, handle

        if topk_idx is None or num_experts is None or num_ranks is None:
            raise ValueError("non-cached dispatch needs topk_idx, num_experts and num_ranks")
        _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
        if topk_idx.shape[0] != T or topk_idx.device != dev:
            raise ValueError("topk_idx must be [num_tokens, num_topk] on x's device")
        K = topk_idx.shape[1]
        need = int(lib.cgd_dispatch_capacity(T, K, num_experts, expert_alignment))
        cap = need if recv_capacity is None else int(recv_capacity)
        if recv_x is None:
            recv_x = torch.empty((max(cap, 0), H), dtype=torch.bfloat16, device=dev)
        _dev_tensor(recv_x, "recv_x", torch.bfloat16, 2)
        if recv_x.shape[1] != H or recv_x.shape[0] != cap:
            raise ValueError("recv_x must be [recv_capacity, hidden]")
        off = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
        nre = torch.empty(num_experts, dtype=torch.int32, device=dev)
        src = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
        dst = torch.empty((T, K), dtype=torch.int32, device=dev)
        nbytes = lib.cgd_dispatch_workspace_bytes(T, K, num_experts, num_ranks)
        ws = _workspace(dev, "dispatch", nbytes)
        _check("cgd_dispatch",
               lib.cgd_dispatch(_ptr(x), T, H, _ptr(topk_idx), K, num_experts, num_ranks, expert_alignment,
                                _ptr(recv_x), cap, _ptr(off), _ptr(nre), _ptr(src), _ptr(dst), _ptr(ws), ws.numel(),
                                _stream(dev)))
    return recv_x, nre, DispatchHandle(off, src, dst, nre, num_experts, num_ranks, expert_alignment, cap)


@dataclass
class DispatchPlan:
    """Result of dispatch_plan: the handle (complete once the plan has run on
    the stream) and the workspace the plan used (not needed afterwards)."""
    handle: DispatchHandle
    workspace: torch.Tensor
    num_tokens: int


def dispatch_plan(topk_idx: torch.Tensor, num_experts: int, num_ranks: int, expert_alignment: int = 1,
                  recv_capacity: int | None = None) -> DispatchPlan:
    """First step of dispatch: the handle (receive-buffer layout, dst_row,
    recv_src_idx) from the routing alone."""
    lib = load()
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    dev = topk_idx.device
    with torch.cuda.device(dev):
        need = int(lib.cgd_dispatch_capacity(T, K, num_experts, expert_alignment))
        cap = need if recv_capacity is None else int(recv_capacity)
        off = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
        nre = torch.empty(num_experts, dtype=torch.int32, device=dev)
        src = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
        dst = torch.empty((T, K), dtype=torch.int32, device=dev)
        nbytes = lib.cgd_dispatch_workspace_bytes(T, K, num_experts, num_ranks)
        ws = _workspace(dev, "dispatch", nbytes)
        _check("cgd_dispatch_plan",
               lib.cgd_dispatch_plan(_ptr(topk_idx), T, K, num_experts, num_ranks, expert_alignment, cap, _ptr(off),
                                     _ptr(nre), _ptr(src), _ptr(dst), _ptr(ws), ws.numel(), _stream(dev)))
    h = DispatchHandle(off, src, dst, nre, num_experts, num_ranks, expert_alignment, cap)
    return DispatchPlan(h, ws, T)


def layout_and_dispatch_plan(topk_idx: torch.Tensor, num_experts: int, num_ranks: int, expert_alignment: int = 1,
                             recv_capacity: int | None = None):
    """get_dispatch_layout and dispatch_plan in one pass over the routing.
    -> ((num_tokens_per_rank, None, num_tokens_per_expert, is_token_in_rank, None), DispatchPlan)."""
    lib = load()
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    dev = topk_idx.device
    with torch.cuda.device(dev):
        need = int(lib.cgd_dispatch_capacity(T, K, num_experts, expert_alignment))
        cap = need if recv_capacity is None else int(recv_capacity)
        ntpr = torch.empty(num_ranks, dtype=torch.int32, device=dev)
        ntpe = torch.empty(num_experts, dtype=torch.int32, device=dev)
        itr = torch.empty((T, num_ranks), dtype=torch.bool, device=dev)
        off = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
        nre = torch.empty(num_experts, dtype=torch.int32, device=dev)
        src = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
        dst = torch.empty((T, K), dtype=torch.int32, device=dev)
        ws = _workspace(dev, "dispatch", lib.cgd_dispatch_workspace_bytes(T, K, num_experts, num_ranks))
        _check("cgd_layout_and_dispatch_plan",
               lib.cgd_layout_and_dispatch_plan(_ptr(topk_idx), T, K, num_experts, num_ranks, expert_alignment, cap,
                                                _ptr(ntpr), _ptr(ntpe), _ptr(itr), _ptr(off), _ptr(nre), _ptr(src),
                                                _ptr(dst), _ptr(ws), ws.numel(), _stream(dev)))
    h = DispatchHandle(off, src, dst, nre, num_experts, num_ranks, expert_alignment, cap)
    return (ntpr, None, ntpe, itr, None), DispatchPlan(h, ws, T)


def _dispatch_cast(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, num_ranks: int, expert_alignment: int,
                   recv_capacity: int | None, recv_x, fmt: int, layout: bool):
    """The non-cached cast on dispatch (cgd_dispatch_cast_fp8, or with the
    layout outputs cgd_layout_and_dispatch_cast_fp8): bf16 x in, the FP8
    tuple out. -> (layout tuple or None, recv_x, num_recv_tokens_per_expert,
    DispatchHandle)."""
    lib = load()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, H = x.shape
    dev = x.device
    if topk_idx.shape[0] != T or topk_idx.device != dev:
        raise ValueError("topk_idx must be [num_tokens, num_topk] on x's device")
    K = topk_idx.shape[1]
    with torch.cuda.device(dev):
        need = int(lib.cgd_dispatch_capacity(T, K, num_experts, expert_alignment))
        cap = need if recv_capacity is None else int(recv_capacity)
        recv_x = _recv_fp8(recv_x, max(cap, 0), H, fmt, dev)
        off = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
        nre = torch.empty(num_experts, dtype=torch.int32, device=dev)
        src = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
        dst = torch.empty((T, K), dtype=torch.int32, device=dev)
        ws = _workspace(dev, "dispatch", lib.cgd_dispatch_workspace_bytes(T, K, num_experts, num_ranks))
        lay = None
        if layout:
            ntpr = torch.empty(num_ranks, dtype=torch.int32, device=dev)
            ntpe = torch.empty(num_experts, dtype=torch.int32, device=dev)
            itr = torch.empty((T, num_ranks), dtype=torch.bool, device=dev)
            _check("cgd_layout_and_dispatch_cast_fp8",
                   lib.cgd_layout_and_dispatch_cast_fp8(_ptr(x), T, H, _ptr(topk_idx), K, num_experts, num_ranks,
                                                        expert_alignment, fmt, _ptr(recv_x[0]), _ptr(recv_x[1]), cap,
                                                        _ptr(ntpr), _ptr(ntpe), _ptr(itr), _ptr(off), _ptr(nre),
                                                        _ptr(src), _ptr(dst), _ptr(ws), ws.numel(), _stream(dev)))
            lay = (ntpr, None, ntpe, itr, None)
        else:
            _check("cgd_dispatch_cast_fp8",
                   lib.cgd_dispatch_cast_fp8(_ptr(x), T, H, _ptr(topk_idx), K, num_experts, num_ranks,
                                             expert_alignment, fmt, _ptr(recv_x[0]), _ptr(recv_x[1]), cap, _ptr(off),
                                             _ptr(nre), _ptr(src), _ptr(dst), _ptr(ws), ws.numel(), _stream(dev)))
    h = DispatchHandle(off, src, dst, nre, num_experts, num_ranks, expert_alignment, cap)
    return lay, recv_x, nre, h


def layout_and_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                        expert_alignment: int = 1, recv_capacity: int | None = None, recv_x=None,
                        cast_fp8: int | None = None):
    """get_dispatch_layout and dispatch (bf16 x) in one call; a batch of at most
    256 tokens takes one launch. cast_fp8 (a scale format) casts x to FP8 on
    the way: recv_x is then the (codes, scales) tuple.
    -> ((num_tokens_per_rank, None, num_tokens_per_expert, is_token_in_rank, None), recv_x,
        num_recv_tokens_per_expert, DispatchHandle)."""
    if cast_fp8 is not None:
        return _dispatch_cast(x, topk_idx, num_experts, num_ranks, expert_alignment, recv_capacity, recv_x, cast_fp8,
                              layout=True)
    lib = load()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, H = x.shape
    dev = x.device
    if topk_idx.shape[0] != T or topk_idx.device != dev:
        raise ValueError("topk_idx must be [num_tokens, num_topk] on x's device")
    K = topk_idx.shape[1]
    with torch.cuda.device(dev):
        need = int(lib.cgd_dispatch_capacity(T, K, num_experts, expert_alignment))
        cap = need if recv_capacity is None else int(recv_capacity)
        if recv_x is None:
            recv_x = torch.empty((max(cap, 0), H), dtype=torch.bfloat16, device=dev)
        _dev_tensor(recv_x, "recv_x", torch.bfloat16, 2)
        if recv_x.shape != (cap, H):
            raise ValueError("recv_x must be [recv_capacity, hidden]")
        ntpr = torch.empty(num_ranks, dtype=torch.int32, device=dev)
        ntpe = torch.empty(num_experts, dtype=torch.int32, device=dev)
        itr = torch.empty((T, num_ranks), dtype=torch.bool, device=dev)
        off = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
        nre = torch.empty(num_experts, dtype=torch.int32, device=dev)
        src = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
        dst = torch.empty((T, K), dtype=torch.int32, device=dev)
        ws = _workspace(dev, "dispatch", lib.cgd_dispatch_workspace_bytes(T, K, num_experts, num_ranks))
        _check("cgd_layout_and_dispatch",
               lib.cgd_layout_and_dispatch(_ptr(x), T, H, _ptr(topk_idx), K, num_experts, num_ranks, expert_alignment,
                                           _ptr(recv_x), cap, _ptr(ntpr), _ptr(ntpe), _ptr(itr), _ptr(off),
                                           _ptr(nre), _ptr(src), _ptr(dst), _ptr(ws), ws.numel(), _stream(dev)))
    h = DispatchHandle(off, src, dst, nre, num_experts, num_ranks, expert_alignment, cap)
    return (ntpr, None, ntpe, itr, None), recv_x, nre, h


def layout_and_dispatch_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                                expert_alignment: int = 1, *, recv_x: torch.Tensor, num_tokens_per_rank: torch.Tensor,
                                num_tokens_per_expert: torch.Tensor, is_token_in_rank: torch.Tensor,
                                expert_offset: torch.Tensor, num_recv_tokens_per_expert: torch.Tensor,
                                recv_src_idx: torch.Tensor, dst_row: torch.Tensor) -> None:
    """layout_and_dispatch into the caller's output tensors, with libcgd's
    static scratch as the workspace: nothing is allocated, here or in the
    library (for graph capture and loops that must not allocate). Calls that
    overlap on one GPU share that scratch and race; workspaces above 8 MiB are
    refused (CgdError with the workspace status)."""
    lib = load()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, H = x.shape
    K = topk_idx.shape[1]
    dev = x.device
    cap = recv_x.shape[0] if isinstance(recv_x, torch.Tensor) else -1
    want = (("recv_x", recv_x, torch.bfloat16, (cap, H)), ("topk_idx", topk_idx, torch.int64, (T, K)),
            ("num_tokens_per_rank", num_tokens_per_rank, torch.int32, (num_ranks,)),
            ("num_tokens_per_expert", num_tokens_per_expert, torch.int32, (num_experts,)),
            ("is_token_in_rank", is_token_in_rank, torch.bool, (T, num_ranks)),
            ("expert_offset", expert_offset, torch.int32, (num_experts + 1,)),
            ("num_recv_tokens_per_expert", num_recv_tokens_per_expert, torch.int32, (num_experts,)),
            ("recv_src_idx", recv_src_idx, torch.int32, (cap,)), ("dst_row", dst_row, torch.int32, (T, K)))
    for name, t, dtype, shape in want:
        _dev_tensor(t, name, dtype, len(shape))
        if tuple(t.shape) != shape or t.device != dev:
            raise ValueError(f"{name} must be {list(shape)} on x's device (got {list(t.shape)} on {t.device})")
    with torch.cuda.device(dev):
        _check("cgd_layout_and_dispatch_noalloc",
               lib.cgd_layout_and_dispatch_noalloc(_ptr(x), T, H, _ptr(topk_idx), K, num_experts, num_ranks,
                                                   expert_alignment, _ptr(recv_x), cap, _ptr(num_tokens_per_rank),
                                                   _ptr(num_tokens_per_expert), _ptr(is_token_in_rank),
                                                   _ptr(expert_offset), _ptr(num_recv_tokens_per_expert),
                                                   _ptr(recv_src_idx), _ptr(dst_row), _stream(dev)))


def dispatch_apply(x, plan: DispatchPlan, recv_x=None, cast_fp8: int | None = None):
    """Second step of dispatch: copy rows to the plan's handle (the cached
    dispatch with plan.handle). x: bf16 [T, H] or an FP8 tuple; cast_fp8 (a
    scale format) casts a bf16 x on the way. Returns (recv_x,
    num_recv_tokens_per_expert, handle), recv_x an FP8 tuple for FP8 payloads."""
    T = (x[0] if isinstance(x, tuple) else x).shape[0]
    if T != plan.num_tokens:
        raise ValueError("x has a different number of tokens than the plan")
    return dispatch(x, handle=plan.handle, recv_x=recv_x, cast_fp8=cast_fp8)


def combine(expert_out: torch.Tensor, handle: DispatchHandle, topk_weights: torch.Tensor,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """combined[t] = bf16( sum_k w[t,k] * expert_out[dst_row[t,k]] ), fp32 accumulation."""
    lib = load()
    _dev_tensor(expert_out, "expert_out", torch.bfloat16, 2)
    _dev_tensor(topk_weights, "topk_weights", torch.float32, 2)
    T, K = handle.dst_row.shape
    if topk_weights.shape != (T, K):
        raise ValueError("topk_weights must be [num_tokens, num_topk]")
    rows, H = expert_out.shape
    dev = expert_out.device
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        _dev_tensor(out, "out", torch.bfloat16, 2)
        if out.shape != (T, H):
            raise ValueError("out must be [num_tokens, hidden]")
        _check("cgd_combine",
               lib.cgd_combine(_ptr(expert_out), rows, H, _ptr(handle.dst_row), _ptr(topk_weights), T, K, _ptr(out),
                               _stream(dev)))
    return out


# ---------------------------------------------------------------------------
# Rank-granular ("normal mode") dispatch and combine: one received row per
# (token, flagged rank), the DeepEP normal-mode receive layout.
# ---------------------------------------------------------------------------

def normal_workspace_bytes(num_tokens: int, num_ranks: int) -> int:
    """Bytes of a workspace of its own for normal_dispatch_plan."""
    n = int(load().cgd_normal_workspace_bytes(num_tokens, num_ranks))
    if n == 0:
        raise ValueError("invalid sizes for a workspace")
    return n


def layout_and_normal_workspace_bytes(num_tokens: int, num_topk: int, num_experts: int, num_ranks: int) -> int:
    """Bytes of a workspace of its own for layout_and_normal_dispatch_plan."""
    n = int(load().cgd_layout_and_normal_workspace_bytes(num_tokens, num_topk, num_experts, num_ranks))
    if n == 0:
        raise ValueError("invalid sizes for a workspace")
    return n


def normal_capacity(num_tokens: int, num_topk: int, num_ranks: int) -> int:
    cap = int(load().cgd_normal_capacity(num_tokens, num_topk, num_ranks))
    if cap < 0:
        raise ValueError("invalid sizes for a receive buffer")
    return cap


@dataclass
class NormalHandle:
    """Layout of one normal-mode dispatch, reusable for cached dispatch and combine.

    rank_offset  int32 [R+1]: rows of rank r are [rank_offset[r], rank_offset[r+1]).
    recv_src_idx int32 [recv_capacity]: source token of each row, -1 if none.
    send_row     int32 [T, R]: the token's row on each rank, -1 if not sent.
    """
    rank_offset: torch.Tensor
    recv_src_idx: torch.Tensor
    send_row: torch.Tensor
    num_topk: int
    recv_capacity: int

    @property
    def num_tokens(self) -> int:
        return self.send_row.shape[0]

    @property
    def num_ranks(self) -> int:
        return self.send_row.shape[1]


def normal_dispatch(x: torch.Tensor, is_token_in_rank: torch.Tensor | None = None,
                    num_tokens_per_expert: torch.Tensor | None = None, topk_idx: torch.Tensor | None = None,
                    topk_weights: torch.Tensor | None = None, num_experts: int | None = None,
                    num_topk: int | None = None, expert_alignment: int = 1, handle: NormalHandle | None = None,
                    recv_capacity: int | None = None, recv_x: torch.Tensor | None = None):
    """Send each token once to every rank flagged in is_token_in_rank.

    Non-cached: -> (recv_x, recv_topk_idx | None, recv_topk_weights | None,
    num_recv_tokens_per_expert | None, NormalHandle). num_experts is needed;
    num_topk comes from topk_idx, else must be given (it sizes the capacity).
    Cached (handle given): -> (recv_x, None, None, None, handle).
    """
    lib = load()
    if isinstance(x, tuple):
        q, sc, fmt, st, sb = _fp8_parts(x)
        T, H = q.shape
        dev = q.device
        if handle is None:
            if is_token_in_rank is None or num_experts is None:
                raise ValueError("non-cached normal dispatch needs is_token_in_rank and num_experts")
            plan = normal_dispatch_plan(is_token_in_rank, num_tokens_per_expert, num_experts, expert_alignment)
            return normal_dispatch_apply(x, plan, topk_idx, topk_weights, num_topk, recv_capacity, recv_x)
        if is_token_in_rank is not None or topk_idx is not None:
            raise ValueError("cached normal dispatch takes a handle and no layout")
        if handle.num_tokens != T:
            raise ValueError("x has a different number of tokens than the handle")
        with torch.cuda.device(dev):
            cap = handle.recv_capacity
            recv_x = _recv_fp8(recv_x, cap, H, fmt, dev)
            _check("cgd_normal_dispatch_cached_fp8",
                   lib.cgd_normal_dispatch_cached_fp8(_ptr(q), _ptr(sc), st, sb, fmt, T, H, handle.num_ranks,
                                                      _ptr(handle.send_row), _ptr(recv_x[0]), _ptr(recv_x[1]), cap,
                                                      _stream(dev)))
        return recv_x, None, None, None, handle
    _dev_tensor(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    dev = x.device
    with torch.cuda.device(dev):
        if handle is not None:
            if is_token_in_rank is not None or topk_idx is not None:
                raise ValueError("cached normal dispatch takes a handle and no layout")
            if handle.num_tokens != T:
                raise ValueError("x has a different number of tokens than the handle")
            cap = handle.recv_capacity
            if recv_x is None:
                recv_x = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
            _dev_tensor(recv_x, "recv_x", torch.bfloat16, 2)
            if recv_x.shape != (cap, H):
                raise ValueError("recv_x must be [recv_capacity, hidden]")
            _check("cgd_normal_dispatch_cached",
                   lib.cgd_normal_dispatch_cached(_ptr(x), T, H, handle.num_ranks, _ptr(handle.send_row),
                                                  _ptr(recv_x), cap, _stream(dev)))
            return recv_x, None, None, None, handle

        if is_token_in_rank is None or num_experts is None:
            raise ValueError("non-cached normal dispatch needs is_token_in_rank and num_experts")
        _dev_tensor(is_token_in_rank, "is_token_in_rank", torch.bool, 2)
        if is_token_in_rank.shape[0] != T:
            raise ValueError("is_token_in_rank must be [num_tokens, num_ranks]")
        R = is_token_in_rank.shape[1]
        if (topk_idx is None) != (topk_weights is None):
            raise ValueError("topk_idx and topk_weights go together")
        if topk_idx is not None:
            _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
            _dev_tensor(topk_weights, "topk_weights", torch.float32, 2)
            if topk_idx.shape[0] != T or topk_weights.shape != topk_idx.shape:
                raise ValueError("topk_idx and topk_weights must be [num_tokens, num_topk]")
            K = topk_idx.shape[1]
        elif num_topk is not None:
            K = int(num_topk)
        else:
            raise ValueError("num_topk is needed when dispatching without top-k")
        if num_tokens_per_expert is not None:
            _dev_tensor(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, 1)
            if num_tokens_per_expert.shape[0] != num_experts:
                raise ValueError("num_tokens_per_expert must be [num_experts]")
        need = int(lib.cgd_normal_capacity(T, K, R))
        cap = need if recv_capacity is None else int(recv_capacity)
        if recv_x is None:
            recv_x = torch.empty((max(cap, 0), H), dtype=torch.bfloat16, device=dev)
        _dev_tensor(recv_x, "recv_x", torch.bfloat16, 2)
        if recv_x.shape != (cap, H):
            raise ValueError("recv_x must be [recv_capacity, hidden]")
        off = torch.empty(R + 1, dtype=torch.int32, device=dev)
        src = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
        send = torch.empty((T, R), dtype=torch.int32, device=dev)
        ridx = rw = nre = None
        if topk_idx is not None:
            ridx = torch.empty((max(cap, 0), K), dtype=torch.int64, device=dev)
            rw = torch.empty((max(cap, 0), K), dtype=torch.float32, device=dev)
        if num_tokens_per_expert is not None:
            nre = torch.empty(num_experts, dtype=torch.int32, device=dev)
        nbytes = lib.cgd_normal_workspace_bytes(T, R)
        ws = _workspace(dev, "normal", nbytes)
        _note_plan_write(ws)  # its plan step replaces any plan left there
        _check("cgd_normal_dispatch",
               lib.cgd_normal_dispatch(_ptr(x), T, H, _ptr(is_token_in_rank), _ptr(num_tokens_per_expert),
                                       _ptr(topk_idx), _ptr(topk_weights), K, num_experts, R, expert_alignment,
                                       _ptr(recv_x), cap, _ptr(off), _ptr(src), _ptr(send), _ptr(ridx), _ptr(rw),
                                       _ptr(nre), _ptr(ws), ws.numel(), _stream(dev)))
    return recv_x, ridx, rw, nre, NormalHandle(off, src, send, K, cap)


@dataclass
class NormalPlan:
    """Result of normal_dispatch_plan: rank offsets, aligned per-expert counts
    and the workspace holding the plan's per-token places, which
    normal_dispatch_apply reads. By default that workspace is the one shared by
    the plans on the current stream: apply the plan before making the next one
    there (normal_dispatch_apply raises otherwise), or pass a workspace of the
    plan's own to keep several plans alive."""
    rank_offset: torch.Tensor
    num_recv_tokens_per_expert: torch.Tensor | None
    workspace: torch.Tensor
    num_tokens: int
    num_experts: int
    write: int = 0  # the workspace's plan-write count when this plan wrote it


def _normal_plan_workspace(workspace, nbytes: int, dev, kind: str) -> torch.Tensor:
    if workspace is None:
        return _workspace(dev, kind, nbytes)
    return _caller_workspace(workspace, nbytes, dev)


def normal_dispatch_plan(is_token_in_rank: torch.Tensor, num_tokens_per_expert: torch.Tensor | None = None,
                         num_experts: int | None = None, expert_alignment: int = 1,
                         workspace: torch.Tensor | None = None) -> NormalPlan:
    """First step of normal dispatch: rank offsets from is_token_in_rank alone.
    workspace: None (the stream's shared one), or a zero-filled uint8 device
    tensor of at least normal_workspace_bytes(T, R) bytes that the plan keeps."""
    lib = load()
    _dev_tensor(is_token_in_rank, "is_token_in_rank", torch.bool, 2)
    T, R = is_token_in_rank.shape
    if num_experts is None:
        raise ValueError("num_experts is needed")
    dev = is_token_in_rank.device
    with torch.cuda.device(dev):
        nre = None
        if num_tokens_per_expert is not None:
            _dev_tensor(num_tokens_per_expert, "num_tokens_per_expert", torch.int32, 1)
            if num_tokens_per_expert.shape[0] != num_experts:
                raise ValueError("num_tokens_per_expert must be [num_experts]")
            nre = torch.empty(num_experts, dtype=torch.int32, device=dev)
        off = torch.empty(R + 1, dtype=torch.int32, device=dev)
        ws = _normal_plan_workspace(workspace, lib.cgd_normal_workspace_bytes(T, R), dev, "normal")
        _check("cgd_normal_dispatch_plan",
               lib.cgd_normal_dispatch_plan(_ptr(is_token_in_rank), T, R, _ptr(num_tokens_per_expert), num_experts,
                                            expert_alignment, _ptr(off), _ptr(nre), _ptr(ws), ws.numel(),
                                            _stream(dev)))
    return NormalPlan(off, nre, ws, T, num_experts, _note_plan_write(ws))


def layout_and_normal_dispatch_plan(topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                                    expert_alignment: int = 1, num_recv_tokens_per_expert: bool = True,
                                    workspace: torch.Tensor | None = None):
    """get_dispatch_layout and normal_dispatch_plan in one launch.
    -> ((num_tokens_per_rank, None, num_tokens_per_expert, is_token_in_rank, None), NormalPlan).
    workspace: as normal_dispatch_plan, at least
    layout_and_normal_workspace_bytes(T, K, E, R) bytes."""
    lib = load()
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, K = topk_idx.shape
    dev = topk_idx.device
    with torch.cuda.device(dev):
        ntpr = torch.empty(num_ranks, dtype=torch.int32, device=dev)
        ntpe = torch.empty(num_experts, dtype=torch.int32, device=dev)
        itr = torch.empty((T, num_ranks), dtype=torch.bool, device=dev)
        off = torch.empty(num_ranks + 1, dtype=torch.int32, device=dev)
        nre = torch.empty(num_experts, dtype=torch.int32, device=dev) if num_recv_tokens_per_expert else None
        need = int(lib.cgd_layout_and_normal_workspace_bytes(T, K, num_experts, num_ranks))
        ws = _normal_plan_workspace(workspace, max(need, 1), dev, "layout_normal")
        _check("cgd_layout_and_normal_dispatch_plan",
               lib.cgd_layout_and_normal_dispatch_plan(_ptr(topk_idx), T, K, num_experts, num_ranks,
                                                       expert_alignment, _ptr(ntpr), _ptr(ntpe), _ptr(itr), _ptr(off),
                                                       _ptr(nre), _ptr(ws), ws.numel(), _stream(dev)))
    return (ntpr, None, ntpe, itr, None), NormalPlan(off, nre, ws, T, num_experts, _note_plan_write(ws))


def layout_and_normal_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, topk_weights: torch.Tensor | None,
                               num_experts: int, num_ranks: int, expert_alignment: int = 1,
                               recv_capacity: int | None = None, recv_x=None,
                               workspace: torch.Tensor | None = None, cast_fp8: int | None = None, x_fp8=None):
    """layout_and_normal_dispatch_plan and normal_dispatch_apply (bf16 x) in one
    call; the plan pulls x toward the caches for the apply. topk_weights None:
    no recv_topk_idx / recv_topk_weights. cast_fp8 (a scale format): the plan's
    idle blocks cast x per token (into x_fp8, a (codes [T, H], row-major scales
    [T, H/128]) tuple of the caller's, else a new one) and the apply moves that
    tuple; recv_x is then an FP8 tuple.
    -> ((num_tokens_per_rank, None, num_tokens_per_expert, is_token_in_rank, None), recv_x,
        recv_topk_idx | None, recv_topk_weights | None, num_recv_tokens_per_expert, NormalHandle)."""
    lib = load()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, H = x.shape
    K = topk_idx.shape[1]
    dev = x.device
    if topk_idx.shape[0] != T or topk_idx.device != dev:
        raise ValueError("topk_idx must be [num_tokens, num_topk] on x's device")
    if topk_weights is not None:
        _dev_tensor(topk_weights, "topk_weights", torch.float32, 2)
        if topk_weights.shape != topk_idx.shape:
            raise ValueError("topk_weights must be [num_tokens, num_topk]")
    R = num_ranks
    with torch.cuda.device(dev):
        cap = int(lib.cgd_normal_capacity(T, K, R)) if recv_capacity is None else int(recv_capacity)
        if cast_fp8 is not None:
            recv_x = _recv_fp8(recv_x, max(cap, 0), H, cast_fp8, dev)
            x_fp8 = _recv_fp8(x_fp8, T, H, cast_fp8, dev)
        else:
            if recv_x is None:
                recv_x = torch.empty((max(cap, 0), H), dtype=torch.bfloat16, device=dev)
            _dev_tensor(recv_x, "recv_x", torch.bfloat16, 2)
            if recv_x.shape != (cap, H):
                raise ValueError("recv_x must be [recv_capacity, hidden]")
        ntpr = torch.empty(R, dtype=torch.int32, device=dev)
        ntpe = torch.empty(num_experts, dtype=torch.int32, device=dev)
        itr = torch.empty((T, R), dtype=torch.bool, device=dev)
        off = torch.empty(R + 1, dtype=torch.int32, device=dev)
        nre = torch.empty(num_experts, dtype=torch.int32, device=dev)
        src = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
        send = torch.empty((T, R), dtype=torch.int32, device=dev)
        ridx = rw = None
        if topk_weights is not None:
            ridx = torch.empty((max(cap, 0), K), dtype=torch.int64, device=dev)
            rw = torch.empty((max(cap, 0), K), dtype=torch.float32, device=dev)
        need = int(lib.cgd_layout_and_normal_workspace_bytes(T, K, num_experts, R))
        ws = _normal_plan_workspace(workspace, max(need, 1), dev, "layout_normal")
        if cast_fp8 is not None:
            _check("cgd_layout_and_normal_dispatch_cast_fp8",
                   lib.cgd_layout_and_normal_dispatch_cast_fp8(
                       _ptr(x), T, H, _ptr(topk_idx), _ptr(topk_weights), K, num_experts, R, expert_alignment,
                       cast_fp8, _ptr(x_fp8[0]), _ptr(x_fp8[1]), _ptr(recv_x[0]), _ptr(recv_x[1]), cap, _ptr(ntpr),
                       _ptr(ntpe), _ptr(itr), _ptr(off), _ptr(nre), _ptr(src), _ptr(send), _ptr(ridx), _ptr(rw),
                       _ptr(ws), ws.numel(), _stream(dev)))
        else:
            _check("cgd_layout_and_normal_dispatch",
                   lib.cgd_layout_and_normal_dispatch(_ptr(x), T, H, _ptr(topk_idx), _ptr(topk_weights), K,
                                                      num_experts, R, expert_alignment, _ptr(recv_x), cap,
                                                      _ptr(ntpr), _ptr(ntpe), _ptr(itr), _ptr(off), _ptr(nre),
                                                      _ptr(src), _ptr(send), _ptr(ridx), _ptr(rw), _ptr(ws),
                                                      ws.numel(), _stream(dev)))
        _note_plan_write(ws)
    return (ntpr, None, ntpe, itr, None), recv_x, ridx, rw, nre, NormalHandle(off, src, send, K, cap)


def normal_dispatch_apply(x: torch.Tensor, plan: NormalPlan, topk_idx: torch.Tensor | None = None,
                          topk_weights: torch.Tensor | None = None, num_topk: int | None = None,
                          recv_capacity: int | None = None, recv_x: torch.Tensor | None = None):
    """Second step of normal dispatch: rows and per-row outputs.
    -> (recv_x, recv_topk_idx | None, recv_topk_weights | None, num_recv_tokens_per_expert | None, NormalHandle)."""
    lib = load()
    fp8 = isinstance(x, tuple)
    if fp8:
        q, sc, fmt, st, sb = _fp8_parts(x)
        T, H = q.shape
        dev = q.device
    else:
        _dev_tensor(x, "x", torch.bfloat16, 2)
        T, H = x.shape
        dev = x.device
    if T != plan.num_tokens:
        raise ValueError("x has a different number of tokens than the plan")
    if _plan_writes.get(plan.workspace.data_ptr()) != plan.write:
        raise ValueError("a later plan has overwritten this plan's workspace: apply each plan before the next "
                         "one is made on the stream, or give the plans workspaces of their own")
    R = plan.rank_offset.shape[0] - 1
    if (topk_idx is None) != (topk_weights is None):
        raise ValueError("topk_idx and topk_weights go together")
    if topk_idx is not None:
        _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
        _dev_tensor(topk_weights, "topk_weights", torch.float32, 2)
        if topk_idx.shape[0] != T or topk_weights.shape != topk_idx.shape:
            raise ValueError("topk_idx and topk_weights must be [num_tokens, num_topk]")
        K = topk_idx.shape[1]
    elif num_topk is not None:
        K = int(num_topk)
    else:
        raise ValueError("num_topk is needed when dispatching without top-k")
    with torch.cuda.device(dev):
        cap = int(lib.cgd_normal_capacity(T, K, R)) if recv_capacity is None else int(recv_capacity)
        if fp8:
            recv_x = _recv_fp8(recv_x, max(cap, 0), H, fmt, dev)
        else:
            if recv_x is None:
                recv_x = torch.empty((max(cap, 0), H), dtype=torch.bfloat16, device=dev)
            _dev_tensor(recv_x, "recv_x", torch.bfloat16, 2)
            if recv_x.shape != (cap, H):
                raise ValueError("recv_x must be [recv_capacity, hidden]")
        src = torch.empty(max(cap, 0), dtype=torch.int32, device=dev)
        send = torch.empty((T, R), dtype=torch.int32, device=dev)
        ridx = rw = None
        if topk_idx is not None:
            ridx = torch.empty((max(cap, 0), K), dtype=torch.int64, device=dev)
            rw = torch.empty((max(cap, 0), K), dtype=torch.float32, device=dev)
        if fp8:
            _check("cgd_normal_dispatch_apply_fp8",
                   lib.cgd_normal_dispatch_apply_fp8(_ptr(q), _ptr(sc), st, sb, fmt, T, H, _ptr(topk_idx),
                                                     _ptr(topk_weights), K, plan.num_experts, R, _ptr(recv_x[0]),
                                                     _ptr(recv_x[1]), cap, _ptr(plan.rank_offset), _ptr(src),
                                                     _ptr(send), _ptr(ridx), _ptr(rw), _ptr(plan.workspace),
                                                     plan.workspace.numel(), _stream(dev)))
        else:
            _check("cgd_normal_dispatch_apply",
                   lib.cgd_normal_dispatch_apply(_ptr(x), T, H, _ptr(topk_idx), _ptr(topk_weights), K,
                                                 plan.num_experts, R, _ptr(recv_x), cap, _ptr(plan.rank_offset),
                                                 _ptr(src), _ptr(send), _ptr(ridx), _ptr(rw), _ptr(plan.workspace),
                                                 plan.workspace.numel(), _stream(dev)))
    return recv_x, ridx, rw, plan.num_recv_tokens_per_expert, NormalHandle(plan.rank_offset, src, send, K, cap)


def normal_combine(expert_out: torch.Tensor, handle: NormalHandle, recv_topk_weights: torch.Tensor | None = None,
                   bias=None, out: torch.Tensor | None = None):
    """combined[t] = bf16( sum over t's rows, ascending rank, + bias_0[t] + bias_1[t] ), fp32 sum.

    bias: None, a tensor, or a tuple of up to two bf16 [T, H] tensors.
    -> (combined_x, combined_topk_weights | None)."""
    lib = load()
    _dev_tensor(expert_out, "expert_out", torch.bfloat16, 2)
    rows, H = expert_out.shape
    T, R = handle.send_row.shape
    K = handle.num_topk
    dev = expert_out.device
    if bias is None:
        bias = ()
    elif isinstance(bias, torch.Tensor):
        bias = (bias,)
    bias = tuple(b for b in bias if b is not None)
    if len(bias) > 2:
        raise ValueError("at most two bias tensors")
    for i, b in enumerate(bias):
        _dev_tensor(b, f"bias_{i}", torch.bfloat16, 2)
        if b.shape != (T, H):
            raise ValueError("bias tensors must be [num_tokens, hidden]")
    b0 = bias[0] if len(bias) > 0 else None
    b1 = bias[1] if len(bias) > 1 else None
    with torch.cuda.device(dev):
        cw = None
        if recv_topk_weights is not None:
            _dev_tensor(recv_topk_weights, "recv_topk_weights", torch.float32, 2)
            if recv_topk_weights.shape != (rows, K):
                raise ValueError("recv_topk_weights must be [recv_rows, num_topk]")
            cw = torch.empty((T, K), dtype=torch.float32, device=dev)
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        _dev_tensor(out, "out", torch.bfloat16, 2)
        if out.shape != (T, H):
            raise ValueError("out must be [num_tokens, hidden]")
        _check("cgd_normal_combine",
               lib.cgd_normal_combine(_ptr(expert_out), rows, H, _ptr(handle.send_row), T, R,
                                      _ptr(recv_topk_weights), K, _ptr(b0), _ptr(b1), _ptr(out), _ptr(cw),
                                      _stream(dev)))
    return out, cw


# ---------------------------------------------------------------------------
# Fixed-capacity packed layout (the low-latency dispatch's receive buffers).
# ---------------------------------------------------------------------------

@dataclass
class PackedHandle:
    """recv_src_info int32 [E, cap]: source token of each valid packed row, -1 elsewhere.
    dst_row int32 [T, K]: packed row (e * cap + i) of each slot, -1 if not selected or dropped."""
    recv_src_info: torch.Tensor
    dst_row: torch.Tensor
    num_experts: int
    expert_capacity: int


def _packed_fp8_out(out, E: int, cap: int, H: int, fmt: int, dev):
    """A caller's FP8 packed receive tuple: codes [E*cap, H] or [E, cap, H]
    (float8_e4m3fn or uint8), scales [E*cap, H/128] or [E, cap, H/128] of the
    format's storage type, both contiguous on the device."""
    if not (isinstance(out, tuple) and len(out) == 2):
        raise TypeError("out must be a (codes, scales) tuple with use_fp8")
    q, sc = out
    for t, name in ((q, "codes"), (sc, "scales")):
        if not isinstance(t, torch.Tensor) or t.device != dev or not t.is_contiguous():
            raise ValueError(f"out {name} must be a contiguous tensor on the inputs' device")
    if q.dtype not in (torch.float8_e4m3fn, torch.uint8) or tuple(q.shape) not in ((E * cap, H), (E, cap, H)):
        raise ValueError("out codes must be float8_e4m3fn (or uint8) [E * expert_capacity, hidden] "
                         "or [E, expert_capacity, hidden]")
    if sc.dtype != _scale_dtype(fmt):
        raise TypeError(f"out scales must be {_scale_dtype(fmt)} for scale format {fmt} (got {sc.dtype})")
    if tuple(sc.shape) not in ((E * cap, H // 128), (E, cap, H // 128)):
        raise ValueError("out scales must be [E * expert_capacity, hidden / 128] or [E, expert_capacity, hidden / 128]")
    return q, sc


def low_latency_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                         expert_capacity: int | None = None, use_fp8: bool = False, scale_format: int = SCALE_F32,
                         cumulative_local_expert_recv_stats: torch.Tensor | None = None, out=None):
    """Dispatch into fixed per-expert buffers (no host synchronisation, graph-capturable).

    expert_capacity defaults to num_tokens (enough unless a token repeats an
    expert). Returns (packed_recv_x, packed_recv_count int32 [E], PackedHandle);
    packed_recv_x is bf16 [E, cap, H], or with use_fp8 the tuple
    (codes float8_e4m3fn [E, cap, H], scales [E, cap, H/128])."""
    return _low_latency_dispatch(x, topk_idx, num_experts, num_ranks, expert_capacity, use_fp8, scale_format,
                                 cumulative_local_expert_recv_stats, out, False)


def layout_and_low_latency_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                                    expert_capacity: int | None = None, use_fp8: bool = False,
                                    scale_format: int = SCALE_F32,
                                    cumulative_local_expert_recv_stats: torch.Tensor | None = None, out=None):
    """get_dispatch_layout and low_latency_dispatch in one call (one launch up
    to 256 tokens). -> ((num_tokens_per_rank, None, num_tokens_per_expert,
    is_token_in_rank, None), packed_recv_x, packed_recv_count, PackedHandle)."""
    return _low_latency_dispatch(x, topk_idx, num_experts, num_ranks, expert_capacity, use_fp8, scale_format,
                                 cumulative_local_expert_recv_stats, out, True)


def _low_latency_dispatch(x, topk_idx, num_experts, num_ranks, expert_capacity, use_fp8, scale_format,
                          cumulative_local_expert_recv_stats, out, with_layout):
    lib = load()
    _dev_tensor(x, "x", torch.bfloat16, 2)
    _dev_tensor(topk_idx, "topk_idx", torch.int64, 2)
    T, H = x.shape
    K = topk_idx.shape[1]
    if topk_idx.shape[0] != T:
        raise ValueError("topk_idx must be [num_tokens, num_topk]")
    E = num_experts
    cap = T if expert_capacity is None else int(expert_capacity)
    dev = x.device
    st = cumulative_local_expert_recv_stats
    if st is not None:
        _dev_tensor(st, "cumulative_local_expert_recv_stats", torch.int32, 1)
        if st.shape[0] != E:
            raise ValueError("cumulative_local_expert_recv_stats must be [num_experts]")
    with torch.cuda.device(dev):
        count = torch.empty(E, dtype=torch.int32, device=dev)
        info = torch.empty((E, max(cap, 0)), dtype=torch.int32, device=dev)
        dst = torch.empty((T, K), dtype=torch.int32, device=dev)
        if with_layout:
            R = num_ranks
            ntpr = torch.empty(R, dtype=torch.int32, device=dev)
            ntpe = torch.empty(E, dtype=torch.int32, device=dev)
            itr = torch.empty((T, R), dtype=torch.bool, device=dev)
            ws = _workspace(dev, "dispatch", lib.cgd_dispatch_workspace_bytes(T, K, E, R))
        else:
            ws = _workspace(dev, "dispatch", lib.cgd_packed_workspace_bytes(T, K, E))
        if use_fp8:
            if out is None:
                q, sc = _fp8_empty(E * cap, H, scale_format, dev)
            else:
                q, sc = _packed_fp8_out(out, E, cap, H, scale_format, dev)
            if with_layout:
                _check("cgd_layout_and_dispatch_packed_cast_fp8",
                       lib.cgd_layout_and_dispatch_packed_cast_fp8(
                           _ptr(x), T, H, _ptr(topk_idx), K, E, num_ranks, cap, scale_format, _ptr(q), _ptr(sc),
                           _ptr(count), _ptr(info), _ptr(dst), _ptr(st), _ptr(ntpr), _ptr(ntpe), _ptr(itr), _ptr(ws),
                           ws.numel(), _stream(dev)))
            else:
                _check("cgd_dispatch_packed_cast_fp8",
                       lib.cgd_dispatch_packed_cast_fp8(_ptr(x), T, H, _ptr(topk_idx), K, E, num_ranks, cap,
                                                        scale_format, _ptr(q), _ptr(sc), _ptr(count), _ptr(info),
                                                        _ptr(dst), _ptr(st), _ptr(ws), ws.numel(), _stream(dev)))
            recv = (q.view(E, cap, H), sc.view(E, cap, H // 128))
        else:
            recv = torch.empty((E, cap, H), dtype=torch.bfloat16, device=dev) if out is None else out
            _dev_tensor(recv, "out", torch.bfloat16, 3)
            if recv.shape != (E, cap, H):
                raise ValueError("out must be [num_experts, expert_capacity, hidden]")
            if with_layout:
                _check("cgd_layout_and_dispatch_packed",
                       lib.cgd_layout_and_dispatch_packed(_ptr(x), T, H, _ptr(topk_idx), K, E, num_ranks, cap,
                                                          _ptr(recv), _ptr(count), _ptr(info), _ptr(dst), _ptr(st),
                                                          _ptr(ntpr), _ptr(ntpe), _ptr(itr), _ptr(ws), ws.numel(),
                                                          _stream(dev)))
            else:
                _check("cgd_dispatch_packed",
                       lib.cgd_dispatch_packed(_ptr(x), T, H, _ptr(topk_idx), K, E, num_ranks, cap, _ptr(recv),
                                               _ptr(count), _ptr(info), _ptr(dst), _ptr(st), _ptr(ws), ws.numel(),
                                               _stream(dev)))
    if with_layout:
        return (ntpr, None, ntpe, itr, None), recv, count, PackedHandle(info, dst, E, cap)
    return recv, count, PackedHandle(info, dst, E, cap)


def low_latency_combine(expert_out: torch.Tensor, topk_weights: torch.Tensor, handle: PackedHandle,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """combined[t] = bf16( sum_k w[t,k] * expert_out[packed row of (t, k)] ), fp32 accumulation;
    expert_out is bf16 [E, cap, H] (the packed layout)."""
    lib = load()
    _dev_tensor(expert_out, "expert_out", torch.bfloat16, 3)
    _dev_tensor(topk_weights, "topk_weights", torch.float32, 2)
    E, cap, H = expert_out.shape
    if (E, cap) != (handle.num_experts, handle.expert_capacity):
        raise ValueError("expert_out must be [num_experts, expert_capacity, hidden] of the handle")
    T, K = handle.dst_row.shape
    if topk_weights.shape != (T, K):
        raise ValueError("topk_weights must be [num_tokens, num_topk]")
    dev = expert_out.device
    with torch.cuda.device(dev):
        if out is None:
            out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        _dev_tensor(out, "out", torch.bfloat16, 2)
        _check("cgd_combine",
               lib.cgd_combine(_ptr(expert_out), E * cap, H, _ptr(handle.dst_row), _ptr(topk_weights), T, K,
                               _ptr(out), _stream(dev)))
    return out
