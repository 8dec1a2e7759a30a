"""Seeded synthetic inputs for the MoE layout / dispatch / combine path.

This module only draws random inputs: routing (``topk_idx``), routing weights,
token activations ``x`` and expert outputs. It holds none of the method's
arithmetic. The CPU oracle and the GPU path both take their inputs from here,
and from nowhere else they share.

The five workloads below are the shapes of a DeepEP-style expert-parallel MoE
layer: a prefill batch (4096 tokens, hidden 7168, top-8 of 256 experts), a
decode batch (128 tokens), Zipf-skewed routing, an upper-range stress shape at
the limits the NPU ``get_dispatch_layout`` API page lists under "Parameters"
and "Notes" (top-k up to 16, up to 512 experts), and a tiny case.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")

# Stream ids: each tensor of a workload has its own counter-addressed stream.
STREAM_X = 1
STREAM_TOPK = 2
STREAM_LOGITS = 3
STREAM_PERM = 4
STREAM_EXPERT_OUT = 5


def build() -> str:
    """Compile libsynth.so (plain C, OpenMP) in place; returns its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", _LIB + ".tmp", _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("CGD_SYNTH_LIBRARY")  # another build (e.g. with sanitizers); must exist
        if not path:
            path = _LIB
            if not os.path.exists(path):
                build()
        lib = ctypes.CDLL(path)
        u64, i64, i32 = ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
        vp = ctypes.c_void_p
        lib.synth_splitmix64.argtypes = [u64, u64]
        lib.synth_splitmix64.restype = u64
        lib.synth_stream_key.argtypes = [u64, u64, u64]
        lib.synth_stream_key.restype = u64
        lib.synth_normal_f64.argtypes = [u64, i64, i64, vp]
        lib.synth_normal_f64.restype = None
        lib.synth_normal_bf16.argtypes = [u64, i64, i64, vp]
        lib.synth_normal_bf16.restype = None
        lib.synth_topk_uniform.argtypes = [u64, i64, i32, i32, vp]
        lib.synth_topk_uniform.restype = i32
        lib.synth_permutation.argtypes = [u64, i32, vp]
        lib.synth_permutation.restype = i32
        lib.synth_topk_zipf.argtypes = [u64, u64, i64, i32, i32, ctypes.c_double, vp]
        lib.synth_topk_zipf.restype = i32
        lib.synth_softmax_weights.argtypes = [u64, i64, i32, vp]
        lib.synth_softmax_weights.restype = None
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


def salt_of(name: str) -> int:
    """FNV-1a 64-bit hash of a workload name, used to separate streams."""
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def splitmix64(key: int, i: int) -> int:
    return int(_load().synth_splitmix64(key, i))


def stream_key(seed: int, salt: int, stream: int) -> int:
    return int(_load().synth_stream_key(seed, salt, stream))


def normal_f64(key: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    _load().synth_normal_f64(key, offset, n, _ptr(out))
    return out


def normal_bf16(key: int, n: int, offset: int = 0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) draws, elements offset..offset+n."""
    out = np.empty(n, dtype=np.uint16)
    _load().synth_normal_bf16(key, offset, n, _ptr(out))
    return out


def topk_uniform(key: int, T: int, K: int, E: int) -> np.ndarray:
    out = np.empty((T, K), dtype=np.int64)
    if _load().synth_topk_uniform(key, T, K, E, _ptr(out)) != 0:
        raise ValueError("bad topk_uniform arguments")
    return out


def permutation(key: int, E: int) -> np.ndarray:
    out = np.empty(E, dtype=np.int32)
    if _load().synth_permutation(key, E, _ptr(out)) != 0:
        raise ValueError("bad permutation arguments")
    return out


def topk_zipf(key_perm: int, key_draw: int, T: int, K: int, E: int, s: float) -> np.ndarray:
    out = np.empty((T, K), dtype=np.int64)
    if _load().synth_topk_zipf(key_perm, key_draw, T, K, E, s, _ptr(out)) != 0:
        raise ValueError("bad topk_zipf arguments")
    return out


def softmax_weights(key: int, T: int, K: int) -> np.ndarray:
    out = np.empty((T, K), dtype=np.float32)
    _load().synth_softmax_weights(key, T, K, _ptr(out))
    return out


@dataclass(frozen=True)
class Workload:
    name: str
    T: int  # num_tokens
    H: int  # hidden
    K: int  # num_topk
    E: int  # num_experts
    R: int  # logical ranks (partitions of the expert set)
    routing: str = "uniform"  # "uniform" | "zipf"
    zipf_s: float = 1.2
    align: int = 1  # expert_alignment

    @property
    def L(self) -> int:
        return self.E // self.R

    def replace(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "tiny": Workload("tiny", T=128, H=256, K=2, E=8, R=2),
    "prefill": Workload("prefill", T=4096, H=7168, K=8, E=256, R=8),
    "decode": Workload("decode", T=128, H=7168, K=8, E=256, R=16),
    "skewed": Workload("skewed", T=8192, H=7168, K=8, E=256, R=32, routing="zipf", zipf_s=1.2),
    "stress": Workload("stress", T=32768, H=4096, K=16, E=512, R=64),
}


def make_topk_idx(w: Workload, seed: int = 0) -> np.ndarray:
    salt = salt_of(w.name)
    if w.routing == "uniform":
        return topk_uniform(stream_key(seed, salt, STREAM_TOPK), w.T, w.K, w.E)
    if w.routing == "zipf":
        return topk_zipf(stream_key(seed, salt, STREAM_PERM), stream_key(seed, salt, STREAM_TOPK),
                         w.T, w.K, w.E, w.zipf_s)
    raise ValueError(w.routing)


def make_weights(w: Workload, seed: int = 0) -> np.ndarray:
    return softmax_weights(stream_key(seed, salt_of(w.name), STREAM_LOGITS), w.T, w.K)


def make_x(w: Workload, seed: int = 0) -> np.ndarray:
    """x as bf16 bit patterns, shape [T, H]."""
    return normal_bf16(stream_key(seed, salt_of(w.name), STREAM_X), w.T * w.H).reshape(w.T, w.H)


def make_expert_out(w: Workload, rows: int, seed: int = 0, row_offset: int = 0) -> np.ndarray:
    """Independent N(0,1) expert outputs as bf16 bits, rows row_offset..row_offset+rows of [*, H]."""
    key = stream_key(seed, salt_of(w.name), STREAM_EXPERT_OUT)
    return normal_bf16(key, rows * w.H, offset=row_offset * w.H).reshape(rows, w.H)


def make_inputs(w: Workload, seed: int = 0) -> dict:
    return {"topk_idx": make_topk_idx(w, seed), "topk_weights": make_weights(w, seed), "x": make_x(w, seed)}
