"""Pins of the oracle's dispatch permutation: stable counting sort via a
library routine, invariants, brute force, special cases, the worked fixture."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _numpy_positions(idx, E, A):
    """Independent formulation: the received rows of one expert are the slots
    that selected it in (token, slot) order -> a stable argsort of the
    flattened routing; segments are the aligned counts laid end to end."""
    flat = idx.ravel()
    cnt = np.bincount(flat[flat >= 0], minlength=E)
    seg = (cnt + A - 1) // A * A
    off = np.concatenate([[0], np.cumsum(seg)]).astype(np.int64)
    dst = np.full(flat.shape, -1, np.int64)
    order = np.argsort(np.where(flat >= 0, flat, E), kind="stable")
    order = order[: (flat >= 0).sum()]
    # position inside the segment = index among equal keys in stable order
    e_sorted = flat[order]
    first = np.searchsorted(e_sorted, e_sorted, side="left")
    dst[order] = off[e_sorted] + (np.arange(len(order)) - first)
    return off, dst.reshape(idx.shape)


def _rowcode_x(T, H):
    """Rows that name their token: x[t,0] = t & 0xFF, x[t,1] = t >> 8, as
    exact small bf16 integers; the rest is noise."""
    import torch
    rng = np.random.default_rng(T)
    f = rng.standard_normal((T, H)).astype(np.float32)
    f[:, 0] = np.arange(T) & 0xFF
    f[:, 1] = np.arange(T) >> 8
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_to_f32(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("T,K,E,R,A,dup,p_neg", [
    (1, 1, 1, 1, 1, False, 0.0), (37, 3, 12, 4, 1, False, 0.2), (300, 8, 256, 8, 1, False, 0.0),
    (300, 8, 256, 8, 16, False, 0.1), (129, 16, 512, 64, 32, False, 0.05), (90, 5, 7, 7, 3, True, 0.2),
    (64, 4, 4, 2, 1, True, 0.0),
])
def test_dispatch_positions_match_stable_argsort(T, K, E, R, A, dup, p_neg):
    rng = np.random.default_rng(T + 17 * K + A)
    if dup:
        idx = rng.integers(0, E, size=(T, K))
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)])
    idx = np.where(rng.random((T, K)) < p_neg, -1, idx).astype(np.int64)
    H = 16
    x = _rowcode_x(T, H)
    d = oracle.dispatch(x, idx, E, R, align=A)
    off, dst = _numpy_positions(idx, E, A)
    np.testing.assert_array_equal(d["expert_offset"], off)
    np.testing.assert_array_equal(d["dst_row"], dst)
    src = d["recv_src_idx"]
    cap = oracle.capacity(T, K, E, A)
    assert src.shape == (cap,)
    sel = idx >= 0
    # I6: recv_src_idx inverts dst_row; dst_row is a bijection onto data rows
    tt = np.broadcast_to(np.arange(T)[:, None], idx.shape)
    np.testing.assert_array_equal(src[dst[sel]], tt[sel])
    assert len(np.unique(dst[sel])) == sel.sum()
    data_rows = np.zeros(cap, bool)
    data_rows[dst[sel]] = True
    assert (src[~data_rows] == -1).all()
    # rows inside each segment come from non-decreasing tokens
    for e in range(E):
        seg = src[off[e]: off[e + 1]]
        seg = seg[seg >= 0]
        assert (np.diff(seg) >= 0).all()
        if not dup:
            assert (np.diff(seg) > 0).all()
        # segment sizes are multiples of the alignment
        assert (off[e + 1] - off[e]) % A == 0
    # I7: each received row is its token's row, bit for bit; the row code names it
    recv = d["recv_x"]
    np.testing.assert_array_equal(recv[dst[sel]], np.repeat(x, sel.sum(1), axis=0))
    code = _bf16_to_f32(recv[dst[sel]][:, :2]).astype(np.int64)
    np.testing.assert_array_equal(code[:, 0] + 256 * code[:, 1], tt[sel])


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_dispatch_invariants_on_workloads(name):
    w = synth.WORKLOADS[name]
    idx = synth.make_topk_idx(w)
    d = oracle.dispatch(None, idx, w.E, w.R, with_rows=False)
    off = d["expert_offset"].astype(np.int64)
    _, ntpe, _ = oracle.layout(idx, w.E, w.R)
    # I5: alignment 1 -> rows per rank are the sums of that rank's expert counts
    rows_per_rank = off[np.arange(1, w.R + 1) * w.L] - off[np.arange(w.R) * w.L]
    np.testing.assert_array_equal(rows_per_rank, ntpe.reshape(w.R, w.L).sum(1))
    assert off[-1] == w.T * w.K
    assert (np.diff(off) >= 0).all()
    off2, dst2 = _numpy_positions(idx, w.E, 1)
    np.testing.assert_array_equal(d["dst_row"], dst2)


def test_dispatch_k1_is_stable_sort_of_rows():
    rng = np.random.default_rng(3)
    T, E, H = 500, 32, 8
    idx = rng.integers(0, E, size=(T, 1)).astype(np.int64)
    x = _rowcode_x(T, H)
    d = oracle.dispatch(x, idx, E, 4)
    np.testing.assert_array_equal(d["recv_x"][:T], x[np.argsort(idx[:, 0], kind="stable")])


def test_dispatch_brute_force_all_small_routings():
    E, T, K = 4, 3, 2
    rows = [(a, b) for a in range(-1, E) for b in range(-1, E) if a < 0 or b < 0 or a != b]
    for R in (1, 2, 4):
        for combo in itertools.product(rows, repeat=T):
            idx = np.array(combo, dtype=np.int64)
            d = oracle.dispatch(None, idx, E, R, with_rows=False)
            # list-based definition: segment of e lists its (t,k) in order
            segs = {e: [(t, k) for t in range(T) for k in range(K) if combo[t][k] == e] for e in range(E)}
            start, exp_dst = 0, {}
            exp_off = [0]
            for e in range(E):
                for j, tk in enumerate(segs[e]):
                    exp_dst[tk] = start + j
                start += len(segs[e])
                exp_off.append(start)
            assert d["expert_offset"].tolist() == exp_off
            for t in range(T):
                for k in range(K):
                    assert d["dst_row"][t, k] == exp_dst.get((t, k), -1)


def test_dispatch_golden_worked_example():
    g = json.load(open(GOLDEN))
    idx = np.array(g["topk_idx"], dtype=np.int64)
    d1 = oracle.dispatch(None, idx, g["E"], g["R"], align=1, with_rows=False)
    assert d1["expert_offset"].tolist() == g["align1"]["expert_offset"]
    assert d1["dst_row"].tolist() == g["align1"]["dst_row"]
    assert d1["recv_src_idx"].tolist()[:11] == g["align1"]["recv_src_idx"]
    d4 = oracle.dispatch(None, idx, g["E"], g["R"], align=4, with_rows=False)
    assert oracle.capacity(g["T"], g["K"], g["E"], 4) == g["align4"]["capacity"]
    assert d4["expert_offset"].tolist() == g["align4"]["expert_offset"]
    assert d4["dst_row"].tolist() == g["align4"]["dst_row"]


def test_dispatch_duplicate_expert_in_token_takes_two_rows_in_slot_order():
    idx = np.array([[2, 2], [2, -1], [0, 2]], np.int64)
    d = oracle.dispatch(None, idx, 4, 2, with_rows=False)
    assert d["expert_offset"].tolist() == [0, 1, 1, 5, 5]
    assert d["dst_row"].tolist() == [[1, 2], [3, -1], [0, 4]]


def test_dispatch_capacity_and_argument_errors():
    idx = np.array([[0, 1]], np.int64)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.dispatch(None, idx, 4, 2, align=2, cap=4, with_rows=False)
    assert ei.value.rc == oracle.ECAPACITY
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(None, idx, 4, 2, align=0, with_rows=False)
    with pytest.raises(oracle.OracleError):
        oracle.dispatch(None, np.array([[4, 1]], np.int64), 4, 2, with_rows=False)


def test_dispatch_zero_tokens():
    d = oracle.dispatch(np.zeros((0, 8), np.uint16), np.zeros((0, 2), np.int64), 8, 2)
    assert d["expert_offset"].tolist() == [0] * 9
    assert d["recv_src_idx"].shape == (0,)
