"""Pins of the oracle's rank-granular ("normal mode") dispatch and combine:
the hand-worked fixture, an independent column-wise formulation, a
reduction to the pinned expert-granular dispatch, closed forms of the
pages' own checks, exact rational sums and the capacity bound."""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _bf16_bits(vals) -> np.ndarray:
    import torch
    return torch.from_numpy(np.asarray(vals, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_f32(bits) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _routing(rng, T, K, E, p_neg=0.0, dup=False):
    if dup:
        idx = rng.integers(0, E, size=(T, K))
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]) if T else np.zeros((0, K), np.int64)
    return np.where(rng.random((T, K)) < p_neg, -1, idx).astype(np.int64)


def _columnwise(itr, idx, w, E, cap):
    """Independent formulation: rank r's rows are np.flatnonzero of column r
    of is_token_in_rank, laid out rank after rank; a slot survives in a row
    of rank r exactly when its expert divided by L equals r."""
    T, R = itr.shape
    L = E // R
    counts = itr.sum(axis=0).astype(np.int64)
    off = np.concatenate([[0], np.cumsum(counts)])
    send = np.full((T, R), -1, np.int64)
    src = np.full(cap, -1, np.int64)
    K = idx.shape[1]
    ridx = np.full((cap, K), -1, np.int64)
    rw = np.zeros((cap, K), np.float32)
    for r in range(R):
        toks = np.flatnonzero(itr[:, r])
        rows = off[r] + np.arange(len(toks))
        send[toks, r] = rows
        src[rows] = toks
        sel = (idx[toks] >= 0) & (idx[toks] // L == r)
        ridx[rows] = np.where(sel, idx[toks] - r * L, -1)
        rw[rows] = np.where(sel, w[toks], 0.0)
    return off, send, src, ridx, rw


def test_golden_normal_dispatch():
    g = json.load(open(GOLDEN))
    n = g["normal"]
    idx = np.array(g["topk_idx"], np.int64)
    itr = np.array(g["is_token_in_rank"], np.uint8)
    ntpe = np.array(g["num_tokens_per_expert"], np.int32)
    w = np.array(g["combine_identity"]["topk_weights"], np.float32)
    x = _bf16_bits(g["combine_identity"]["x"])
    for align, key in ((1, "num_recv_tokens_per_expert_align1"), (4, "num_recv_tokens_per_expert_align4")):
        assert oracle.normal_capacity(g["T"], g["K"], g["R"]) == n["capacity"]
        o = oracle.dispatch_normal(x, itr, g["E"], g["K"], ntpe, idx, w, align=align)
        assert o["rank_offset"].tolist() == n["rank_offset"]
        assert o["recv_src_idx"].tolist() == n["recv_src_idx"]
        assert o["send_row"].tolist() == n["send_row"]
        rows = n["rank_offset"][-1]
        assert o["recv_topk_idx"][:rows].tolist() == n["recv_topk_idx"]
        assert (o["recv_topk_idx"][rows:] == -1).all()
        assert o["recv_topk_weights"][:rows].tolist() == n["recv_topk_weights"]
        assert (o["recv_topk_weights"][rows:] == 0).all()
        assert o["num_recv_tokens_per_expert"].tolist() == n[key]
        src = np.array(n["recv_src_idx"][:rows])
        assert (o["recv_x"][:rows] == x[src]).all()


def test_golden_normal_combine():
    g = json.load(open(GOLDEN))
    n = g["normal"]
    x = _bf16_bits(g["combine_identity"]["x"])
    send = np.array(n["send_row"], np.int32)
    src = np.array(n["recv_src_idx"])
    y = np.zeros((n["capacity"], 2), np.uint16)
    y[src >= 0] = x[src[src >= 0]]
    rw = np.zeros((n["capacity"], g["K"]), np.float32)
    rw[: len(n["recv_topk_weights"])] = n["recv_topk_weights"]
    out, cw = oracle.combine_normal(y, send, rw, _bf16_bits(n["bias_0"]), _bf16_bits(n["bias_1"]))
    assert _bf16_f32(out).tolist() == n["combined_x"]
    assert cw.tolist() == n["combined_topk_weights"]


@pytest.mark.parametrize("T,K,E,R,p_neg,dup", [
    (0, 4, 16, 4, 0.0, False), (1, 1, 1, 1, 0.0, False), (77, 8, 256, 8, 0.0, False), (77, 8, 256, 8, 0.3, False),
    (50, 3, 12, 12, 0.1, True), (64, 16, 512, 64, 0.05, False), (40, 2, 384, 384, 0.0, False),
    (33, 6, 30, 3, 0.2, True),
])
def test_normal_dispatch_matches_columnwise(T, K, E, R, p_neg, dup):
    rng = np.random.default_rng(T * 7 + K * 3 + R)
    idx = _routing(rng, T, K, E, p_neg, dup)
    w = rng.standard_normal((T, K)).astype(np.float32)
    ntpr, ntpe, itr = oracle.layout(idx, E, R)
    cap = oracle.normal_capacity(T, K, R)
    o = oracle.dispatch_normal(None, itr, E, K, ntpe, idx, w, align=1)
    off, send, src, ridx, rw = _columnwise(itr, idx, w, E, cap)
    assert (o["rank_offset"] == off).all()
    assert (np.diff(o["rank_offset"]) == ntpr).all()
    assert (o["send_row"] == send).all()
    assert (o["recv_src_idx"] == src).all()
    assert (o["recv_topk_idx"] == ridx).all()
    assert (o["recv_topk_weights"] == rw).all()


def test_normal_dispatch_reduces_to_expert_dispatch():
    """One expert per rank (E == R), no repeated experts, alignment 1: every
    selected slot is its own rank row, so the rank-granular permutation is
    the pinned expert-granular one."""
    rng = np.random.default_rng(5)
    T, K, E = 200, 4, 16
    idx = _routing(rng, T, K, E, p_neg=0.2)
    w = rng.random((T, K)).astype(np.float32)
    _, ntpe, itr = oracle.layout(idx, E, E)
    n = oracle.dispatch_normal(None, itr, E, K, ntpe, idx, w)
    d = oracle.dispatch(None, idx, E, E, align=1, with_rows=False)
    assert (n["rank_offset"] == d["expert_offset"]).all()
    rows = d["expert_offset"][-1]
    assert (n["recv_src_idx"][:rows] == d["recv_src_idx"][:rows]).all()
    for t in range(T):
        for k in range(K):
            if idx[t, k] >= 0:
                assert n["send_row"][t, idx[t, k]] == d["dst_row"][t, k]
                assert n["recv_topk_idx"][d["dst_row"][t, k], k] == 0  # local id of the rank's only expert
    assert (n["num_recv_tokens_per_expert"] == ntpe).all()


def test_normal_dispatch_without_topk_and_flags_beyond_experts():
    """Dispatch without top-k (the pages' with_topk=False calls) moves rows by
    is_token_in_rank alone, even for a flag with no expert behind it."""
    rng = np.random.default_rng(9)
    T, H, R = 20, 16, 4
    itr = (rng.random((T, R)) < 0.5).astype(np.uint8)
    x = _bf16_bits(rng.standard_normal((T, H)))
    o = oracle.dispatch_normal(x, itr, 8, 4)
    assert o["recv_topk_idx"] is None and o["num_recv_tokens_per_expert"] is None
    for r in range(R):
        toks = np.flatnonzero(itr[:, r])
        seg = slice(o["rank_offset"][r], o["rank_offset"][r + 1])
        assert (o["recv_src_idx"][seg] == toks).all()
        assert (o["recv_x"][seg] == x[toks]).all()


def test_normal_aligned_expert_counts():
    rng = np.random.default_rng(2)
    idx = _routing(rng, 150, 8, 64, p_neg=0.1)
    _, ntpe, itr = oracle.layout(idx, 64, 8)
    cnt = np.bincount(idx[idx >= 0], minlength=64)
    for A in (1, 7, 16, 128):
        o = oracle.dispatch_normal(None, itr, 64, 8, ntpe, idx, np.ones_like(idx, np.float32), align=A)
        assert (o["num_recv_tokens_per_expert"] == -(-cnt // A) * A).all()


def test_normal_capacity_bound_is_tight():
    # each token on min(K, R) distinct ranks fills the bound exactly
    T, K, E, R = 12, 3, 20, 5
    idx = np.array([[(t + j) % R * (E // R) for j in range(K)] for t in range(T)], np.int64)
    _, ntpe, itr = oracle.layout(idx, E, R)
    cap = oracle.normal_capacity(T, K, R)
    assert cap == T * 3 and itr.sum() == cap
    oracle.dispatch_normal(None, itr, E, K, ntpe, idx, np.ones((T, K), np.float32), cap=cap)
    with pytest.raises(oracle.OracleError):
        oracle.dispatch_normal(None, itr, E, K, ntpe, idx, np.ones((T, K), np.float32), cap=cap - 1)
    assert oracle.normal_capacity(T, 8, 5) == T * 5


def test_normal_rejects_bad_routing():
    itr = np.ones((2, 2), np.uint8)
    with pytest.raises(oracle.OracleError):
        oracle.dispatch_normal(None, itr, 4, 2, None, np.array([[0, 4], [1, 2]]), np.ones((2, 2), np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.dispatch_normal(None, np.ones((2, 3), np.uint8), 4, 2)  # E % R != 0


def _exact_nearest_bf16(v: Fraction) -> float:
    """Nearest bf16 value of an exact rational, ties to the even pattern."""
    if v == 0:
        return 0.0
    a = abs(v)
    b = struct.unpack("<I", struct.pack("<f", np.float32(float(a))))[0] >> 16
    best = None
    for p in range(max(b - 2, 0), min(b + 3, 0x7F80)):
        val = struct.unpack("<f", struct.pack("<I", p << 16))[0]
        d = abs(Fraction(val) - a)
        if best is None or d < best[0] or (d == best[0] and p % 2 == 0):
            best = (d, val)
    return best[1] if v > 0 else -best[1]


@pytest.mark.parametrize("bias", [0, 1, 2])
def test_normal_combine_matches_exact_rational_sum(bias):
    rng = np.random.default_rng(11 + bias)
    T, R, H, rows = 7, 6, 12, 30
    y = _bf16_bits(rng.standard_normal((rows, H)) * rng.choice([1e-2, 1, 30], size=(rows, 1)))
    send = np.where(rng.random((T, R)) < 0.5, rng.integers(0, rows, size=(T, R)), -1).astype(np.int32)
    b0 = _bf16_bits(rng.standard_normal((T, H))) if bias >= 1 else None
    b1 = _bf16_bits(rng.standard_normal((T, H)) * 4) if bias >= 2 else None
    out, _ = oracle.combine_normal(y, send, None, b0, b1)
    for t in range(T):
        for h in range(H):
            s = sum((Fraction(float(_bf16_f32(y[row, h]))) for row in send[t] if row >= 0), Fraction(0))
            for b in (b0, b1):
                if b is not None:
                    s += Fraction(float(_bf16_f32(b[t, h])))
            assert float(_bf16_f32(out[t, h])) == _exact_nearest_bf16(s)


def test_normal_combine_recovers_x_through_the_pages_check():
    """Identity experts with small-integer rows: (combined_x - bias_0 - bias_1)
    divided by the number of ranks of the token gives x back exactly, and the
    summed weights give the masked top-k weights (normal-mode combine check)."""
    rng = np.random.default_rng(4)
    T, K, E, R, H = 60, 6, 48, 6, 24
    idx = _routing(rng, T, K, E, p_neg=0.15)
    w = (rng.integers(-8, 9, size=(T, K)) / 8).astype(np.float32)
    # |x * ranks + bias_0 + bias_1| <= 67.5 on a 0.5 grid: exact in bf16
    x = _bf16_bits(rng.integers(-10, 11, size=(T, H)))
    b0 = _bf16_bits(rng.integers(-5, 6, size=(T, H)))
    b1 = _bf16_bits(rng.integers(-5, 6, size=(T, H)) / 2)
    _, ntpe, itr = oracle.layout(idx, E, R)
    d = oracle.dispatch_normal(x, itr, E, K, ntpe, idx, w)
    out, cw = oracle.combine_normal(d["recv_x"], d["send_row"], d["recv_topk_weights"], b0, b1)
    n = itr.sum(axis=1).astype(np.float32)
    back = (_bf16_f32(out) - _bf16_f32(b0) - _bf16_f32(b1))
    has = n > 0
    assert (back[has] / n[has, None] == _bf16_f32(x)[has]).all()
    assert (back[~has] == 0).all()
    assert (cw == np.where(idx >= 0, w, 0)).all()
