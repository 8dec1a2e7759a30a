"""The seeded generator: its published definitions and the workload recipes."""
import math

import numpy as np
import pytest

import synth

M64 = (1 << 64) - 1


def _splitmix64_py(state: int) -> int:
    # Steele, Lea & Flood 2014: advance by the golden gamma, then mix.
    state = (state + 0x9E3779B97F4A7C15) & M64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31), state


def test_splitmix64_matches_sequential_definition():
    for seed in (0, 1, 0x1234567, M64):
        state = seed
        for i in range(20):
            z, state = _splitmix64_py(state)
            assert synth.splitmix64(seed, i) == z


def test_splitmix64_seed0_first_output():
    # widely quoted first output of SplitMix64 from state 0
    assert synth.splitmix64(0, 0) == 0xE220A8397B1DCDAF


def test_normal_moments_and_offsets():
    key = synth.stream_key(0, 1, synth.STREAM_X)
    v = synth.normal_f64(key, 400_000)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    # counter-addressed: any sub-range equals the slice of the whole
    np.testing.assert_array_equal(synth.normal_f64(key, 1001, offset=777), v[777:1778])
    b = synth.normal_bf16(key, 1001, offset=777)
    np.testing.assert_array_equal(b, synth.normal_bf16(key, 2000)[777:1778])


def test_normal_bf16_is_nearest_of_fp32():
    import torch
    key = synth.stream_key(3, 4, 5)
    f = synth.normal_f64(key, 50_000).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.normal_bf16(key, 50_000), ref)


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_routing_is_valid(name):
    w = synth.WORKLOADS[name]
    idx = synth.make_topk_idx(w)
    assert idx.shape == (w.T, w.K) and idx.dtype == np.int64
    assert idx.min() >= 0 and idx.max() < w.E
    s = np.sort(idx, axis=1)
    assert (np.diff(s, axis=1) > 0).all(), "experts of a token must be distinct"
    wt = synth.make_weights(w)
    assert wt.dtype == np.float32 and (wt > 0).all()
    assert np.abs(wt.astype(np.float64).sum(1) - 1).max() < 1e-6
    # deterministic
    np.testing.assert_array_equal(idx, synth.make_topk_idx(w))


def test_uniform_routing_is_uniform():
    w = synth.WORKLOADS["prefill"]
    c = np.bincount(synth.make_topk_idx(w).ravel(), minlength=w.E)
    mean = w.T * w.K / w.E  # 128
    # chi-square with E-1 dof: mean 255, sd ~22.6
    chi2 = ((c - mean) ** 2 / mean).sum()
    assert 150 < chi2 < 400


def test_zipf_routing_follows_popularity():
    w = synth.WORKLOADS["skewed"]
    idx = synth.make_topk_idx(w)
    c = np.bincount(idx.ravel(), minlength=w.E)
    perm = synth.permutation(synth.stream_key(0, synth.salt_of(w.name), synth.STREAM_PERM), w.E)
    by_rank = c[perm]
    # the most popular expert is picked by nearly every token under s=1.2, K=8
    assert by_rank[0] > 0.85 * w.T
    # counts fall with popularity rank (allow noise between neighbours)
    assert by_rank[:8].mean() > by_rank[8:32].mean() > by_rank[32:].mean()
    # slots are in descending-key order: slot 0 holds a popular expert far more often
    rank_of = np.empty(w.E, np.int64)
    rank_of[perm] = np.arange(w.E)
    assert np.median(rank_of[idx[:, 0]]) < np.median(rank_of[idx[:, -1]])


def test_zipf_single_draw_distribution():
    # K=1: the first key-ordered pick is one draw from p itself
    E, T, s = 16, 200_000, 1.2
    idx = synth.topk_zipf(synth.stream_key(9, 9, 1), synth.stream_key(9, 9, 2), T, 1, E, s)
    perm = synth.permutation(synth.stream_key(9, 9, 1), E)
    p = np.array([i ** -s for i in range(1, E + 1)])
    p /= p.sum()
    freq = np.bincount(idx[:, 0], minlength=E)[perm] / T
    assert np.abs(freq - p).max() < 0.005


def test_permutation_is_permutation():
    p = synth.permutation(12345, 512)
    assert sorted(p.tolist()) == list(range(512))
