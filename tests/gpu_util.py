"""Helpers shared by the GPU tests: host<->device moves of generator arrays
and the combine tolerance check. No arithmetic of the method lives here."""
from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def dev_i64(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int64)).to(DEV)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bf16 device tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_combine(got_bits: np.ndarray, exp_bits: np.ndarray, term_mag: np.ndarray, tol: float = 1e-2):
    """Tolerance of the weighted combine (bf16 output, fp32 accumulation):
    |g - o| <= tol * sum_k |w_k y_k| + 2^-133 elementwise, and
    ||g - o|| <= tol * ||o|| per token row and overall. Returns the fraction of
    bit-identical values (+0 == -0)."""
    g = bf16_to_f64(got_bits)
    o = bf16_to_f64(exp_bits)
    assert np.isfinite(g).all()
    err = np.abs(g - o)
    bound = tol * term_mag + 2.0 ** -133
    bad = err > bound
    assert not bad.any(), f"{bad.sum()} values out of tolerance; worst err {err.max()}"
    num = np.sqrt((err ** 2).sum(axis=-1))
    den = np.sqrt((o ** 2).sum(axis=-1))
    assert (num <= tol * den + 1e-30).all()
    assert np.sqrt((err ** 2).sum()) <= tol * np.sqrt((o ** 2).sum()) + 1e-30
    same = (got_bits == exp_bits) | (((got_bits & 0x7FFF) == 0) & ((exp_bits & 0x7FFF) == 0))
    return float(same.mean())


def term_magnitude(y_bits: np.ndarray, dst: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum over selected k of |w[t,k] * y[dst[t,k]]| per element, in double."""
    T, K = dst.shape
    H = y_bits.shape[1]
    out = np.zeros((T, H))
    for k in range(K):
        sel = dst[:, k] >= 0
        if sel.any():
            out[sel] += np.abs(w[sel, k].astype(np.float64)[:, None] * bf16_to_f64(y_bits[dst[sel, k]]))
    return out
