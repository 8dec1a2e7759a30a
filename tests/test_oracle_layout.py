"""Pins of the oracle's get_dispatch_layout: independent formulations,
invariants, brute force and a hand-worked fixture."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _numpy_layout(idx, E, R):
    """Independent formulation with library routines: bincount and any()."""
    L = E // R
    sel = idx[idx >= 0]
    ntpe = np.bincount(sel, minlength=E).astype(np.int32)
    ranks = np.where(idx >= 0, idx // L, -1)
    itr = np.stack([(ranks == r).any(axis=1) for r in range(R)], axis=1) if len(idx) else np.zeros((0, R), bool)
    ntpr = itr.sum(axis=0).astype(np.int32)
    return ntpr, ntpe, itr


def _random_routing(rng, T, K, E, p_neg=0.1, dup=False):
    if dup:
        idx = rng.integers(0, E, size=(T, K))
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]) if T else np.zeros((0, K), np.int64)
    mask = rng.random((T, K)) < p_neg
    return np.where(mask, -1, idx).astype(np.int64)


@pytest.mark.parametrize("T,K,E,R,dup", [
    (1, 1, 1, 1, False), (7, 3, 12, 4, False), (300, 8, 256, 8, False), (513, 16, 512, 64, False),
    (200, 6, 96, 96, False), (100, 16, 16, 1, True), (64, 4, 384, 384, True), (257, 2, 10, 5, True),
])
def test_layout_matches_numpy_formulation(T, K, E, R, dup):
    rng = np.random.default_rng(T * 1000 + K)
    idx = _random_routing(rng, T, K, E, dup=dup)
    got = oracle.layout(idx, E, R)
    ref = _numpy_layout(idx, E, R)
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_layout_invariants_on_workloads(name):
    w = synth.WORKLOADS[name]
    idx = synth.make_topk_idx(w)
    ntpr, ntpe, itr = oracle.layout(idx, w.E, w.R)
    # I1: every selected slot is counted once
    assert ntpe.sum() == (idx >= 0).sum() == w.T * w.K
    # I2: tokens per rank = column sums of is_token_in_rank
    np.testing.assert_array_equal(ntpr, itr.sum(0))
    # I3: max expert count <= distinct tokens per rank <= min(T, sum of its experts' counts)
    per_rank_slots = ntpe.reshape(w.R, w.L).sum(1)
    assert (ntpe.reshape(w.R, w.L).max(1) <= ntpr).all()
    assert (ntpr <= np.minimum(w.T, per_rank_slots)).all()
    # with distinct experts per token, equality on the right iff each rank has one expert
    if w.L == 1:
        np.testing.assert_array_equal(ntpr, per_rank_slots)
    # I4: a token with any selection sits on 1..min(K,R) ranks
    fan = itr.sum(1)
    assert (fan >= 1).all() and (fan <= min(w.K, w.R)).all()


def test_layout_brute_force_all_small_routings():
    # every routing of 3 tokens, 2 slots, 4 experts with -1 allowed and no
    # repeated expert in a token: 21 choices per token, 9261 routings per R
    E, T, K = 4, 3, 2
    rows = [(a, b) for a in range(-1, E) for b in range(-1, E) if a < 0 or b < 0 or a != b]
    assert len(rows) == 21
    for R in (1, 2, 4):
        L = E // R
        for combo in itertools.product(rows, repeat=T):
            idx = np.array(combo, dtype=np.int64)
            ntpr, ntpe, itr = oracle.layout(idx, E, R)
            # set-based definition
            exp_ntpe = [sum(1 for row in combo for e in row if e == x) for x in range(E)]
            exp_sets = [{e // L for e in row if e >= 0} for row in combo]
            exp_itr = [[r in s for r in range(R)] for s in exp_sets]
            exp_ntpr = [sum(1 for s in exp_sets if r in s) for r in range(R)]
            assert ntpe.tolist() == exp_ntpe
            assert itr.tolist() == exp_itr
            assert ntpr.tolist() == exp_ntpr


def test_layout_golden_worked_example():
    g = json.load(open(GOLDEN))
    idx = np.array(g["topk_idx"], dtype=np.int64)
    ntpr, ntpe, itr = oracle.layout(idx, g["E"], g["R"])
    assert ntpe.tolist() == g["num_tokens_per_expert"]
    assert ntpr.tolist() == g["num_tokens_per_rank"]
    assert itr.astype(int).tolist() == g["is_token_in_rank"]


def test_layout_expected_rank_counts_uniform():
    # sanity against the closed form E[tokens on rank r] = T (1 - C(E-L,K)/C(E,K))
    from math import comb
    w = synth.WORKLOADS["prefill"]
    ntpr, _, _ = oracle.layout(synth.make_topk_idx(w), w.E, w.R)
    expect = w.T * (1 - comb(w.E - w.L, w.K) / comb(w.E, w.K))
    assert abs(ntpr.mean() - expect) < 0.02 * expect


def test_layout_zero_tokens():
    ntpr, ntpe, itr = oracle.layout(np.zeros((0, 4), np.int64), 16, 4)
    assert ntpr.tolist() == [0] * 4 and ntpe.tolist() == [0] * 16 and itr.shape == (0, 4)


@pytest.mark.parametrize("K,E,R,bad", [
    (17, 16, 4, None), (0, 16, 4, None), (2, 513, 1, None), (2, 0, 1, None),
    (2, 770, 385, None), (2, 16, 3, None), (2, 16, 4, 16), (2, 16, 4, -2),
])
def test_layout_rejects_out_of_range(K, E, R, bad):
    idx = np.zeros((3, max(K, 1)), np.int64)
    if bad is not None:
        idx[1, 0] = bad
    with pytest.raises(oracle.OracleError):
        oracle.layout(idx[:, :K] if K else idx[:, :0], E, R)
