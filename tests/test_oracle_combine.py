"""Pins of the oracle's weighted combine: exact rational arithmetic with an
independent nearest-even bf16 rounding, closed forms and special cases."""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _to_bf16_bits(vals: np.ndarray) -> np.ndarray:
    import torch
    return torch.from_numpy(np.asarray(vals, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _nearest_bf16_exact(v: Fraction) -> int:
    """Nearest bf16 pattern to an exact rational, ties to the even pattern,
    found by comparing exact distances to the neighbouring bf16 values."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    approx = float(a)
    b = struct.unpack("<I", struct.pack("<f", np.float32(approx)))[0] >> 16  # truncation: at or below
    best = None
    for p in range(max(b - 2, 0), min(b + 3, 0x7F80)):
        d = abs(Fraction(_bf16_value(p)) - a)
        if best is None or d < best[0] or (d == best[0] and p % 2 == 0):
            best = (d, p)
    return sign | best[1]


def _exact_combine(y, dst, w):
    T, K = dst.shape
    H = y.shape[1]
    out = np.zeros((T, H), np.uint16)
    for t in range(T):
        for h in range(H):
            s = Fraction(0)
            for k in range(K):
                if dst[t, k] >= 0:
                    s += Fraction(float(w[t, k])) * Fraction(_bf16_value(y[dst[t, k], h]))
            out[t, h] = _nearest_bf16_exact(s)
    return out


def _same_values(a, b):
    """bf16 bit arrays equal as values (+0 == -0)."""
    za = (a & 0x7FFF) == 0
    zb = (b & 0x7FFF) == 0
    return bool(((a == b) | (za & zb)).all())


@pytest.mark.parametrize("T,K,H,rows,p_neg", [(6, 4, 12, 30, 0.2), (5, 16, 8, 90, 0.3), (9, 1, 16, 9, 0.0)])
def test_combine_matches_exact_rational_sum(T, K, H, rows, p_neg):
    rng = np.random.default_rng(T * K)
    y = _to_bf16_bits(rng.standard_normal((rows, H)) * rng.choice([1e-3, 1, 50], size=(rows, 1)))
    dst = rng.integers(0, rows, size=(T, K)).astype(np.int32)
    dst[rng.random((T, K)) < p_neg] = -1
    w = (rng.standard_normal((T, K))).astype(np.float32)
    got = oracle.combine(y, dst, w)
    assert _same_values(got, _exact_combine(y, dst, w))


def test_combine_cancellation_and_rounding_edges():
    # rows built so exact sums land on ties and just off them
    one = 0x3F80
    y = np.array([[one, one, one, one]], np.uint16)
    dst = np.array([[0, 0], [0, 0], [0, 0], [0, 0], [0, 0]], np.int32)
    w = np.array([[1.0, 2 ** -8], [1.0, 2 ** -8 + 2 ** -20], [1.0, 3 * 2 ** -8], [1.0, -1.0], [-1.0, 2 ** -8]],
                 np.float32)
    got = oracle.combine(y, dst, w)
    exp = _exact_combine(y, dst, w)
    assert _same_values(got, exp)
    assert got[:, 0].tolist()[:3] == [0x3F80, 0x3F81, 0x3F82]
    assert (got[3] & 0x7FFF == 0).all()


def test_identity_round_trip_returns_x():
    # I8: identity experts and softmax weights -> combine(dispatch(x)) == x
    for name in ("tiny", "decode"):
        w = synth.WORKLOADS[name]
        inp = synth.make_inputs(w)
        d = oracle.dispatch(inp["x"], inp["topk_idx"], w.E, w.R)
        out = oracle.combine(d["recv_x"], d["dst_row"], inp["topk_weights"])
        np.testing.assert_array_equal(out, inp["x"])


def test_one_hot_weights_select_one_expert_row_exactly():
    rng = np.random.default_rng(11)
    w = synth.WORKLOADS["tiny"].replace(T=64, H=32, K=4, E=16, R=4)
    idx = np.stack([rng.permutation(w.E)[:w.K] for _ in range(w.T)]).astype(np.int64)
    y = _to_bf16_bits(rng.standard_normal((w.T * w.K, w.H)))
    d = oracle.dispatch(None, idx, w.E, w.R, with_rows=False)
    hot = rng.integers(0, w.K, size=w.T)
    wt = np.zeros((w.T, w.K), np.float32)
    wt[np.arange(w.T), hot] = 1.0
    out = oracle.combine(y, d["dst_row"], wt)
    np.testing.assert_array_equal(out, y[d["dst_row"][np.arange(w.T), hot]])


def test_k1_unit_weight_is_inverse_gather():
    rng = np.random.default_rng(5)
    T, E, H = 200, 8, 24
    idx = rng.integers(0, E, size=(T, 1)).astype(np.int64)
    x = _to_bf16_bits(rng.standard_normal((T, H)))
    d = oracle.dispatch(x, idx, E, 2)
    y = d["recv_x"][::-1].copy()  # any expert output; here reversed rows
    dst_rev = (T - 1 - d["dst_row"]).astype(np.int32)
    out = oracle.combine(y, dst_rev, np.ones((T, 1), np.float32))
    np.testing.assert_array_equal(out, x)


def test_per_expert_scalar_outputs_closed_form():
    # expert e outputs c_e * x (c_e a power of two, exact in bf16), so
    # out[t] = bf16( x[t] * sum_k w[t,k] c_{e_k} ), computed exactly here
    rng = np.random.default_rng(23)
    T, K, E, R, H = 40, 6, 24, 6, 10
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx[rng.random((T, K)) < 0.15] = -1
    x = _to_bf16_bits(rng.standard_normal((T, H)))
    c = 2.0 ** rng.integers(-3, 4, size=E)
    wt = rng.random((T, K)).astype(np.float32)
    d = oracle.dispatch(x, idx, E, R)
    src = d["recv_src_idx"]
    y = d["recv_x"].copy()
    n = int(d["expert_offset"][-1])
    seg_e = np.repeat(np.arange(E), np.diff(d["expert_offset"]))
    assert (src[:n] >= 0).all() and (src[n:] == -1).all()
    y[:n] = _to_bf16_bits(_bf16_to_f32(y[:n]) * c[seg_e][:, None])
    out = oracle.combine(y, d["dst_row"], wt)
    for t in range(T):
        scale = sum(Fraction(float(wt[t, k])) * Fraction(float(c[idx[t, k]])) for k in range(K) if idx[t, k] >= 0)
        for h in range(H):
            exp = _nearest_bf16_exact(Fraction(_bf16_value(x[t, h])) * scale)
            assert _same_values(np.array([out[t, h]]), np.array([exp]))


def _bf16_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def test_unselected_slots_contribute_nothing_and_empty_token_is_zero():
    y = _to_bf16_bits(np.array([[1.5, -2.0], [4.0, 8.0]]))
    dst = np.array([[0, -1], [-1, -1], [-1, 1]], np.int32)
    w = np.array([[2.0, 1e9], [3.0, 3.0], [1e9, 0.5]], np.float32)
    out = oracle.combine(y, dst, w)
    np.testing.assert_array_equal(_bf16_to_f32(out), np.array([[3.0, -4.0], [0.0, 0.0], [2.0, 4.0]], np.float32))
    assert out[1].tolist() == [0, 0]  # +0


def test_combine_golden_identity_example():
    g = json.load(open(GOLDEN))
    idx = np.array(g["topk_idx"], np.int64)
    c = g["combine_identity"]
    x = _to_bf16_bits(np.array(c["x"]))
    d = oracle.dispatch(x, idx, g["E"], g["R"])
    out = oracle.combine(d["recv_x"], d["dst_row"], np.array(c["topk_weights"], np.float32))
    np.testing.assert_array_equal(_bf16_to_f32(out), np.array(c["combined_x"], np.float32))


def test_combine_rejects_rows_out_of_range():
    y = np.zeros((2, 4), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.combine(y, np.array([[2]], np.int32), np.ones((1, 1), np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.combine(y, np.array([[-2]], np.int32), np.ones((1, 1), np.float32))
