"""ctypes wrapper of the plain C oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. Every function here
takes and returns numpy arrays on the host; bf16 values travel as their uint16
bit patterns. It shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, EINVAL, ECAPACITY = 0, -1, -2


def build() -> str:
    """Compile liboracle.so with gcc (single-threaded, IEEE arithmetic)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        lib.oracle_layout.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
        lib.oracle_layout.restype = i32
        lib.oracle_capacity.argtypes = [i64, i32, i32, i32]
        lib.oracle_capacity.restype = i64
        lib.oracle_dispatch.argtypes = [vp, i64, i64, vp, i32, i32, i32, i32, vp, vp, vp, i64, vp]
        lib.oracle_dispatch.restype = i32
        lib.oracle_bf16_round.argtypes = [ctypes.c_double]
        lib.oracle_bf16_round.restype = ctypes.c_uint16
        lib.oracle_combine.argtypes = [vp, i64, i64, vp, vp, i64, i32, vp]
        lib.oracle_combine.restype = i32
        _lib = lib
    return _lib


class OracleError(ValueError):
    def __init__(self, rc: int):
        super().__init__({EINVAL: "invalid argument", ECAPACITY: "capacity too small"}.get(rc, str(rc)))
        self.rc = rc


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a) -> int | None:
    return None if a is None else a.ctypes.data


def layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int):
    """-> (num_tokens_per_rank int32 [R], num_tokens_per_expert int32 [E], is_token_in_rank bool [T,R])."""
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    ntpr = np.zeros(num_ranks, np.int32)
    ntpe = np.zeros(num_experts, np.int32)
    itr = np.zeros((T, num_ranks), np.uint8)
    rc = _load().oracle_layout(_p(idx), T, K, num_experts, num_ranks, _p(ntpr), _p(ntpe), _p(itr))
    if rc:
        raise OracleError(rc)
    return ntpr, ntpe, itr.astype(bool)


def capacity(T: int, K: int, E: int, align: int = 1) -> int:
    return int(_load().oracle_capacity(T, K, E, align))


def dispatch(x: np.ndarray | None, topk_idx: np.ndarray, num_experts: int, num_ranks: int,
             align: int = 1, cap: int | None = None, hidden: int | None = None, with_rows: bool = True):
    """-> dict(expert_offset [E+1], dst_row [T,K], recv_src_idx [cap], recv_x [cap,H] uint16 or None).

    With ``with_rows=False`` only the positions are computed (x may be None)."""
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    if cap is None:
        cap = capacity(T, K, num_experts, align)
    H = hidden if x is None else x.shape[1]
    H = 0 if H is None else H
    xs = None if x is None else _c(x, np.uint16)
    off = np.zeros(num_experts + 1, np.int32)
    dst = np.zeros((T, K), np.int32)
    src = np.zeros(max(cap, 0), np.int32)
    recv = None
    if with_rows:
        if xs is None:
            raise ValueError("x is required for rows")
        recv = np.zeros((max(cap, 0), H), np.uint16)
    rc = _load().oracle_dispatch(_p(xs), T, H, _p(idx), K, num_experts, num_ranks, align,
                                 _p(off), _p(dst), _p(src), cap, _p(recv))
    if rc:
        raise OracleError(rc)
    return {"expert_offset": off, "dst_row": dst, "recv_src_idx": src, "recv_x": recv}


def bf16_round(v: float) -> int:
    return int(_load().oracle_bf16_round(float(v)))


def combine(y: np.ndarray, dst_row: np.ndarray, topk_weights: np.ndarray) -> np.ndarray:
    """-> combined rows, bf16 bits uint16 [T, H]."""
    ys = _c(y, np.uint16)
    dst = _c(dst_row, np.int32)
    w = _c(topk_weights, np.float32)
    T, K = dst.shape
    rows, H = ys.shape
    out = np.zeros((T, H), np.uint16)
    rc = _load().oracle_combine(_p(ys), rows, H, _p(dst), _p(w), T, K, _p(out))
    if rc:
        raise OracleError(rc)
    return out
