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
        path = os.environ.get("CGD_ORACLE_LIBRARY")  # another build (e.g. with sanitizers); must exist
        if not path:
            path = _LIB
            if not os.path.exists(path):
                build()
        lib = ctypes.CDLL(path)
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
        lib.oracle_normal_capacity.argtypes = [i64, i32, i32]
        lib.oracle_normal_capacity.restype = i64
        lib.oracle_dispatch_normal.argtypes = [vp, i64, i64, vp, vp, vp, vp, i32, i32, i32, i32, i64,
                                               vp, vp, vp, vp, vp, vp, vp]
        lib.oracle_dispatch_normal.restype = i32
        lib.oracle_combine_normal.argtypes = [vp, i64, i64, vp, vp, vp, vp, i64, i32, i32, vp, vp]
        lib.oracle_combine_normal.restype = i32
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        lib.oracle_e4m3_encode.restype = ctypes.c_uint8
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_decode.restype = ctypes.c_float
        lib.oracle_cast_to_fp8.argtypes = [vp, i64, i64, i32, vp, vp]
        lib.oracle_cast_to_fp8.restype = i32
        lib.oracle_cast_back.argtypes = [vp, vp, i64, i64, i32, vp]
        lib.oracle_cast_back.restype = i32
        lib.oracle_dispatch_packed.argtypes = [vp, i64, i64, vp, i32, i32, i32, i64, vp, vp, vp, vp, vp]
        lib.oracle_dispatch_packed.restype = i32
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


def normal_capacity(T: int, K: int, R: int) -> int:
    return int(_load().oracle_normal_capacity(T, K, R))


def dispatch_normal(x: np.ndarray | None, is_token_in_rank: np.ndarray, num_experts: int, num_topk: int,
                    num_tokens_per_expert: np.ndarray | None = None, topk_idx: np.ndarray | None = None,
                    topk_weights: np.ndarray | None = None, align: int = 1, cap: int | None = None,
                    hidden: int = 0):
    """Rank-granular dispatch. -> dict(rank_offset [R+1], send_row [T,R], recv_src_idx [cap],
    recv_topk_idx [cap,K] int64 | None, recv_topk_weights [cap,K] f32 | None,
    num_recv_tokens_per_expert [E] | None, recv_x [cap,H] uint16 | None)."""
    itr = _c(is_token_in_rank, np.uint8)
    T, R = itr.shape
    K = num_topk
    if cap is None:
        cap = normal_capacity(T, K, R)
    xs = None if x is None else _c(x, np.uint16)
    H = hidden if xs is None else xs.shape[1]
    ntpe = None if num_tokens_per_expert is None else _c(num_tokens_per_expert, np.int32)
    idx = None if topk_idx is None else _c(topk_idx, np.int64)
    w = None if topk_weights is None else _c(topk_weights, np.float32)
    if (idx is None) != (w is None):
        raise ValueError("topk_idx and topk_weights go together")
    off = np.zeros(R + 1, np.int32)
    send = np.zeros((T, R), np.int32)
    src = np.zeros(max(cap, 0), np.int32)
    ridx = None if idx is None else np.zeros((max(cap, 0), K), np.int64)
    rw = None if idx is None else np.zeros((max(cap, 0), K), np.float32)
    nre = None if ntpe is None else np.zeros(num_experts, np.int32)
    recv = None if xs is None else np.zeros((max(cap, 0), H), np.uint16)
    rc = _load().oracle_dispatch_normal(_p(xs), T, H, _p(itr), _p(ntpe), _p(idx), _p(w), K, num_experts, R,
                                        align, cap, _p(off), _p(send), _p(src), _p(ridx), _p(rw), _p(nre),
                                        _p(recv))
    if rc:
        raise OracleError(rc)
    return {"rank_offset": off, "send_row": send, "recv_src_idx": src, "recv_topk_idx": ridx,
            "recv_topk_weights": rw, "num_recv_tokens_per_expert": nre, "recv_x": recv}


def combine_normal(y: np.ndarray, send_row: np.ndarray, recv_topk_weights: np.ndarray | None = None,
                   bias_0: np.ndarray | None = None, bias_1: np.ndarray | None = None, num_topk: int = 1):
    """Rank-granular combine. -> (combined_x uint16 [T,H], combined_topk_weights f32 [T,K] | None)."""
    ys = _c(y, np.uint16)
    send = _c(send_row, np.int32)
    T, R = send.shape
    rows, H = ys.shape
    rw = None if recv_topk_weights is None else _c(recv_topk_weights, np.float32)
    K = num_topk if rw is None else rw.shape[1]
    b0 = None if bias_0 is None else _c(bias_0, np.uint16)
    b1 = None if bias_1 is None else _c(bias_1, np.uint16)
    out = np.zeros((T, H), np.uint16)
    cw = np.zeros((T, K), np.float32)
    zero_w = np.zeros((max(rows, 1), K), np.float32)
    rc = _load().oracle_combine_normal(_p(ys), rows, H, _p(send), _p(rw if rw is not None else zero_w), _p(b0),
                                       _p(b1), T, K, R, _p(out), _p(cw))
    if rc:
        raise OracleError(rc)
    return out, (None if rw is None else cw)


SCALE_F32, SCALE_POW2, SCALE_UE8M0 = 0, 1, 2


def e4m3_encode(v: float) -> int:
    return int(_load().oracle_e4m3_encode(float(v)))


def e4m3_decode(c: int) -> float:
    return float(_load().oracle_e4m3_decode(int(c)))


def cast_to_fp8(x: np.ndarray, scale_format: int = SCALE_F32):
    """Per-token FP8 cast. x: bf16 bits uint16 [T, H], H % 128 == 0.
    -> (codes uint8 [T, H], scales float32 [T, H/128] or uint8 exponent bytes for UE8M0)."""
    xs = _c(x, np.uint16)
    T, H = xs.shape
    q = np.zeros((T, H), np.uint8)
    sc = np.zeros((T, H // 128), np.uint8 if scale_format == SCALE_UE8M0 else np.float32)
    rc = _load().oracle_cast_to_fp8(_p(xs), T, H, scale_format, _p(q), _p(sc))
    if rc:
        raise OracleError(rc)
    return q, sc


def cast_back(q: np.ndarray, scales: np.ndarray, scale_format: int = SCALE_F32) -> np.ndarray:
    """-> bf16 bits uint16 [T, H]."""
    qs = _c(q, np.uint8)
    T, H = qs.shape
    sc = _c(scales, np.uint8 if scale_format == SCALE_UE8M0 else np.float32)
    out = np.zeros((T, H), np.uint16)
    rc = _load().oracle_cast_back(_p(qs), _p(sc), T, H, scale_format, _p(out))
    if rc:
        raise OracleError(rc)
    return out


def dispatch_packed(x: np.ndarray | None, topk_idx: np.ndarray, num_experts: int, num_ranks: int, cap: int,
                    hidden: int = 0, stats: np.ndarray | None = None):
    """Fixed-capacity packed layout. -> dict(packed_recv_count [E], recv_src_info [E, cap], dst_row [T, K],
    packed_recv_x [E, cap, H] uint16 | None, cumulative_recv_stats (the updated copy of stats) | None)."""
    idx = _c(topk_idx, np.int64)
    T, K = idx.shape
    xs = None if x is None else _c(x, np.uint16)
    H = hidden if xs is None else xs.shape[1]
    cnt = np.zeros(num_experts, np.int32)
    info = np.zeros((num_experts, max(cap, 0)), np.int32)
    dst = np.zeros((T, K), np.int32)
    st = None if stats is None else _c(stats, np.int32).copy()
    recv = None if xs is None else np.zeros((num_experts, max(cap, 0), H), np.uint16)
    rc = _load().oracle_dispatch_packed(_p(xs), T, H, _p(idx), K, num_experts, num_ranks, cap, _p(cnt), _p(info),
                                        _p(dst), _p(st), _p(recv))
    if rc:
        raise OracleError(rc)
    return {"packed_recv_count": cnt, "recv_src_info": info, "dst_row": dst, "packed_recv_x": recv,
            "cumulative_recv_stats": st}
