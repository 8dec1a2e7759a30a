"""Routing values outside [-1, num_experts) mean "not selected" in every kernel.

The C ABI documents that an out-of-range topk_idx entry is treated as -1 and
never indexes memory. Each path that reads topk_idx (layout alone, the
expert-major dispatch, layout and dispatch in one call, the fused plan, the
packed layout and the rank-granular dispatch with its top-k metadata) gets a
routing that mixes in values just past the range, far past it, negative
values other than -1 and int64 values whose low 32 bits are a valid expert.
Its outputs must equal, bit for bit, the oracle's on the same routing with
those entries replaced by -1. Routing widths of 8 (routing read straight
from HBM in the layout kernels) and 16 (staged through LDS) are both used."""
import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import oracle
import synth
from gpu_util import DEV, dev_bf16, dev_f32, dev_i64, host_bits, say

pytestmark = pytest.mark.gpu

I64 = np.iinfo(np.int64)


def _routing(T, K, E, seed, p_bad=0.15):
    """(routing with bad entries, the same routing with them as -1)."""
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    bad = np.array([E, E + 1, 2 * E, (1 << 31) - 1, 1 << 31, (1 << 32) + 3, (1 << 40) + 1, I64.max,
                    -2, -E, -(1 << 31), -(1 << 32) + 5, I64.min], dtype=np.int64)
    where = rng.random((T, K)) < p_bad
    idx_bad = idx.copy()
    idx_bad[where] = rng.choice(bad, size=int(where.sum()))
    # every kind of bad value appears at least once
    flat = np.flatnonzero(where)
    if len(flat) >= len(bad):
        idx_bad.reshape(-1)[flat[:len(bad)]] = bad
    clean = idx.copy()
    clean[where] = -1
    return idx_bad, clean


CASES = [(3000, 8, 256, 16), (700, 16, 512, 64), (100, 3, 8, 2), (200, 8, 256, 16), (2100, 8, 256, 8)]


@pytest.mark.parametrize("T,K,E,R", CASES)
def test_out_of_range_routing_in_layout_and_dispatch(T, K, E, R):
    idx_bad, clean = _routing(T, K, E, seed=T + K)
    H = 64
    x = synth.normal_bf16(synth.stream_key(T, 77, 1), T * H).reshape(T, H)
    say(f"[routing range] T={T} K={K} E={E} R={R}")
    idx_dev = dev_i64(idx_bad)
    ol = oracle.layout(clean, E, R)
    od = oracle.dispatch(x, clean, E, R)
    data = od["recv_src_idx"] >= 0

    ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx_dev, E, R)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])

    def check_handle(h, recv_x):
        np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), od["expert_offset"])
        np.testing.assert_array_equal(h.dst_row.cpu().numpy(), od["dst_row"])
        np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), od["recv_src_idx"])
        np.testing.assert_array_equal(host_bits(recv_x)[data], od["recv_x"][data])

    recv_x, _, h = cgd.dispatch(dev_bf16(x), idx_dev, E, R)
    torch.cuda.synchronize()
    check_handle(h, recv_x)
    say(f"[routing range] T={T}: layout and dispatch ok")

    (l_ntpr, _, l_ntpe, l_itr, _), recv_x, _, h = cgd.layout_and_dispatch(dev_bf16(x), idx_dev, E, R)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(l_ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(l_ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(l_itr.cpu().numpy(), ol[2])
    check_handle(h, recv_x)

    (p_ntpr, _, p_ntpe, p_itr, _), plan = cgd.layout_and_dispatch_plan(idx_dev, E, R)
    recv_x, _, h = cgd.dispatch_apply(dev_bf16(x), plan)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(p_ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(p_ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(p_itr.cpu().numpy(), ol[2])
    check_handle(h, recv_x)
    say(f"[routing range] T={T}: fused layout paths ok")

    recv, count, ph = cgd.low_latency_dispatch(dev_bf16(x), idx_dev, E, R, expert_capacity=T)
    torch.cuda.synchronize()
    op = oracle.dispatch_packed(None, clean, E, R, T)
    np.testing.assert_array_equal(ph.dst_row.cpu().numpy(), op["dst_row"])
    np.testing.assert_array_equal(count.cpu().numpy(), op["packed_recv_count"])
    np.testing.assert_array_equal(ph.recv_src_info.cpu().numpy(), op["recv_src_info"])
    flat = host_bits(recv).reshape(E * T, H)
    sel_t, sel_k = np.nonzero(op["dst_row"] >= 0)
    np.testing.assert_array_equal(flat[op["dst_row"][sel_t, sel_k]], x[sel_t])
    say(f"[routing range] T={T}: packed layout ok")


@pytest.mark.parametrize("T,K,E,R", CASES[:4])
def test_out_of_range_routing_in_rank_granular_dispatch(T, K, E, R):
    idx_bad, clean = _routing(T, K, E, seed=3 * T + K)
    H = 64
    x = synth.normal_bf16(synth.stream_key(T, 78, 1), T * H).reshape(T, H)
    wts = synth.softmax_weights(synth.stream_key(T, 78, 3), T, K)
    say(f"[routing range, normal] T={T} K={K} E={E} R={R}")
    idx_dev = dev_i64(idx_bad)
    ol = oracle.layout(clean, E, R)
    o = oracle.dispatch_normal(x, ol[2], E, K, ol[1], clean, wts, hidden=H)
    data = o["recv_src_idx"] >= 0

    def check(plan_off, nre, h, recv_x, ridx, rw):
        np.testing.assert_array_equal(plan_off.cpu().numpy(), o["rank_offset"])
        np.testing.assert_array_equal(nre.cpu().numpy(), o["num_recv_tokens_per_expert"])
        np.testing.assert_array_equal(h.send_row.cpu().numpy(), o["send_row"])
        np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
        np.testing.assert_array_equal(ridx.cpu().numpy(), o["recv_topk_idx"])
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), o["recv_topk_weights"].view(np.uint32))
        np.testing.assert_array_equal(host_bits(recv_x)[data], o["recv_x"][data])

    _, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx_dev, E, R)
    recv_x, ridx, rw, nre, h = cgd.normal_dispatch(dev_bf16(x), itr, ntpe, idx_dev, dev_f32(wts), num_experts=E)
    torch.cuda.synchronize()
    check(h.rank_offset, nre, h, recv_x, ridx, rw)

    (ntpr, _, ntpe, itr, _), plan = cgd.layout_and_normal_dispatch_plan(idx_dev, E, R)
    recv_x, ridx, rw, nre, h = cgd.normal_dispatch_apply(dev_bf16(x), plan, idx_dev, dev_f32(wts))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])
    check(plan.rank_offset, nre, h, recv_x, ridx, rw)

    # layout, plan and rows in one call (one launch for a batch of one tile)
    (ntpr, _, ntpe, itr, _), recv_x, ridx, rw, nre, h = cgd.layout_and_normal_dispatch(dev_bf16(x), idx_dev,
                                                                                       dev_f32(wts), E, R)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])
    check(h.rank_offset, nre, h, recv_x, ridx, rw)
    say(f"[routing range, normal] T={T}: ok")
