"""Parity of the fixed-capacity packed layout (low-latency dispatch) with the
CPU oracle, its FP8 form, the combine over packed rows, and replay of the
whole decode step from a captured HIP graph.

dst_row, packed_recv_count, recv_src_info, the statistics and every valid
row must be bit-exact; the combine is checked as elsewhere (1e-2 of the
term magnitudes, > 99 % bit-identical)."""
import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import oracle
import synth
from gpu_util import DEV, check_combine, dev_bf16, dev_f32, dev_i64, host_bits, say, term_magnitude

pytestmark = pytest.mark.gpu


def _check_packed_rows(recv, x_dev, dst_np):
    """packed row of every placed slot == x[t], compared on the device."""
    E, cap, H = recv.shape
    flat = recv.view(E * cap, H).view(torch.int16)
    sel_t, sel_k = np.nonzero(dst_np >= 0)
    rows = dst_np[sel_t, sel_k]
    step = 1 << 16
    for i in range(0, len(rows), step):
        r = torch.from_numpy(rows[i:i + step].astype(np.int64)).to(DEV)
        t = torch.from_numpy(sel_t[i:i + step].astype(np.int64)).to(DEV)
        assert torch.equal(flat.index_select(0, r), x_dev.view(torch.int16).index_select(0, t))


def _packed_and_check(x_np, idx_np, E, R, cap, stats=None):
    x_dev = dev_bf16(x_np)
    st_dev = None if stats is None else torch.from_numpy(stats.copy()).to(DEV)
    recv, count, h = cgd.low_latency_dispatch(x_dev, dev_i64(idx_np), E, R, expert_capacity=cap,
                                              cumulative_local_expert_recv_stats=st_dev)
    torch.cuda.synchronize()
    o = oracle.dispatch_packed(None, idx_np, E, R, cap, stats=stats)
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    np.testing.assert_array_equal(count.cpu().numpy(), o["packed_recv_count"])
    np.testing.assert_array_equal(h.recv_src_info.cpu().numpy(), o["recv_src_info"])
    if stats is not None:
        np.testing.assert_array_equal(st_dev.cpu().numpy(), o["cumulative_recv_stats"])
    _check_packed_rows(recv, x_dev, o["dst_row"])
    return x_dev, recv, count, h, o


@pytest.mark.parametrize("name,cap", [("decode", None), ("tiny", None), ("prefill", 300), ("skewed", 2000),
                                      ("stress", 2048)])
def test_packed_workload_parity(name, cap):
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w, seed=0)
    idx = inp["topk_idx"]
    cnt = np.bincount(idx[idx >= 0], minlength=w.E)
    cap = w.T if cap is None else cap
    say(f"[packed] {name}: T={w.T} E={w.E} cap={cap} max count={cnt.max()} dropped={np.maximum(cnt - cap, 0).sum()}")
    stats = np.arange(w.E, dtype=np.int32)
    x_dev, recv, count, h, o = _packed_and_check(inp["x"], idx, w.E, w.R, cap, stats=stats)
    # low-latency combine over the packed rows: identity experts give x times
    # the sum of the placed slots' weights; check against the oracle
    wt = inp["topk_weights"]
    out = cgd.low_latency_combine(recv, dev_f32(wt), h)
    torch.cuda.synchronize()
    tok = np.arange(w.T) if w.T * w.H <= 40_000_000 else np.unique(np.random.default_rng(2).integers(0, w.T, 512))
    y = host_bits(recv.view(-1, w.H)) if w.E * cap * w.H <= 600_000_000 else None
    if y is not None:
        exp = oracle.combine(y, o["dst_row"][tok], wt[tok])
        frac = check_combine(host_bits(out)[tok], exp, term_magnitude(y, o["dst_row"][tok], wt[tok]))
        assert frac > 0.99
    say(f"[packed] {name}: ok")


@pytest.mark.parametrize("T,H", [(128, 7168), (2500, 1024), (1, 7168), (256, 512)])
def test_packed_fp8_cast(T, H):
    w = synth.WORKLOADS["decode"].replace(T=T, H=H)
    inp = synth.make_inputs(w, seed=1)
    for fmt in (cgd.SCALE_F32, cgd.SCALE_UE8M0):
        (q, sc), count, h = cgd.low_latency_dispatch(dev_bf16(inp["x"]), dev_i64(inp["topk_idx"]), w.E, w.R,
                                                     use_fp8=True, scale_format=fmt)
        torch.cuda.synchronize()
        o = oracle.dispatch_packed(None, inp["topk_idx"], w.E, w.R, w.T)
        np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
        np.testing.assert_array_equal(count.cpu().numpy(), o["packed_recv_count"])
        oq, osc = oracle.cast_to_fp8(inp["x"], fmt)
        sel_t, sel_k = np.nonzero(o["dst_row"] >= 0)
        rows = o["dst_row"][sel_t, sel_k]
        np.testing.assert_array_equal(q.view(torch.uint8).reshape(-1, w.H).cpu().numpy()[rows], oq[sel_t])
        np.testing.assert_array_equal(sc.reshape(-1, w.H // 128).cpu().numpy()[rows].view(np.uint8),
                                      osc[sel_t].view(np.uint8))


def test_packed_overflow_duplicates_and_zero_capacity():
    rng = np.random.default_rng(4)
    T, K, E, R, H = 500, 6, 12, 4, 64
    idx = rng.integers(0, E, (T, K)).astype(np.int64)  # repeats allowed
    idx[rng.random((T, K)) < 0.2] = -1
    x = synth.normal_bf16(synth.stream_key(4, 97, 1), T * H).reshape(T, H)
    _packed_and_check(x, idx, E, R, cap=100)
    _packed_and_check(x, idx, E, R, cap=0)
    _packed_and_check(x[:1], idx[:1], E, R, cap=3)
    # one-tile batches (plan and copy in one launch), with and without overflow
    _packed_and_check(x[:200], idx[:200], E, R, cap=10, stats=np.arange(E, dtype=np.int32))
    _packed_and_check(x[:200], idx[:200], E, R, cap=200)
    _packed_and_check(x[:256], idx[:256], E, R, cap=0)


def _decode_step(x, idx, wt, E, R, cap):
    ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx, E, R)
    recv, count, h = cgd.low_latency_dispatch(x, idx, E, R, expert_capacity=cap)
    out = cgd.low_latency_combine(recv, wt, h)
    return ntpr, ntpe, itr, recv, count, h.recv_src_info, h.dst_row, out


def test_decode_step_replays_from_a_captured_graph():
    """layout + packed dispatch + combine captured once, replayed with new
    inputs; every replay equals an eager step on the same inputs."""
    w = synth.WORKLOADS["decode"]
    cap = w.T
    inputs = [synth.make_inputs(w, seed=s) for s in range(6)]
    sx = dev_bf16(inputs[0]["x"])
    sidx = dev_i64(inputs[0]["topk_idx"])
    swt = dev_f32(inputs[0]["topk_weights"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):  # warm-up on the capture stream: its workspaces exist before capture
            _decode_step(sx, sidx, swt, w.E, w.R, cap)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        static_out = _decode_step(sx, sidx, swt, w.E, w.R, cap)
    torch.cuda.synchronize()
    for i, inp in enumerate(inputs[1:]):
        sx.copy_(dev_bf16(inp["x"]))
        sidx.copy_(dev_i64(inp["topk_idx"]))
        swt.copy_(dev_f32(inp["topk_weights"]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = _decode_step(dev_bf16(inp["x"]), dev_i64(inp["topk_idx"]), dev_f32(inp["topk_weights"]), w.E, w.R,
                             cap)
        torch.cuda.synchronize()
        for a, b in zip(static_out, eager):
            if a.dtype == torch.bfloat16 and a.dim() == 3:  # packed rows: valid rows only
                continue
            assert torch.equal(a, b), f"replay {i} differs"
        valid = eager[5] >= 0
        assert torch.equal(static_out[3][valid].view(torch.int16), eager[3][valid].view(torch.int16))
        o = oracle.dispatch_packed(None, inp["topk_idx"], w.E, w.R, cap)
        np.testing.assert_array_equal(static_out[6].cpu().numpy(), o["dst_row"])
    say("[packed] graph replays ok")


@pytest.mark.parametrize("name,T,H,cap,fp8,dup", [("decode", None, None, None, None, False),
                                                  ("decode", None, None, None, cgd.SCALE_UE8M0, False),
                                                  ("tiny", None, None, None, None, False),
                                                  ("prefill", 2500, 1024, 300, None, False),
                                                  ("prefill", 2500, 1024, 300, cgd.SCALE_F32, False),
                                                  ("edge", 200, 256, 30, cgd.SCALE_POW2, True),
                                                  ("edge", 700, 128, 40, None, True)])
def test_layout_and_packed_dispatch(name, T, H, cap, fp8, dup):
    """layout_and_low_latency_dispatch: the layout outputs equal the oracle's
    get_dispatch_layout, the packed handle and rows (or FP8 codes and scales)
    the oracle's packed dispatch (one launch up to 256 tokens; repeated
    experts overflow the capacity in the edge cases)."""
    if name == "edge":
        rng = np.random.default_rng(T)
        E, R, K = 16, 4, 6
        idx = rng.integers(0, E, (T, K)).astype(np.int64) if dup else \
            np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
        idx[rng.random((T, K)) < 0.1] = -1
        x = synth.normal_bf16(synth.stream_key(T, 96, 1), T * H).reshape(T, H)
    else:
        w = synth.WORKLOADS[name]
        w = w.replace(T=T or w.T, H=H or w.H)
        inp = synth.make_inputs(w, seed=2)
        idx, x, E, R = inp["topk_idx"], inp["x"], w.E, w.R
        T, H = w.T, w.H
    cap = cap or T
    say(f"[packed] layout + packed dispatch {name} T={T} H={H} cap={cap} fp8={fp8}")
    x_dev = dev_bf16(x)
    if fp8 is None:
        lay, recv, count, h = cgd.layout_and_low_latency_dispatch(x_dev, dev_i64(idx), E, R, expert_capacity=cap)
    else:
        lay, recv, count, h = cgd.layout_and_low_latency_dispatch(x_dev, dev_i64(idx), E, R, expert_capacity=cap,
                                                                  use_fp8=True, scale_format=fp8)
    torch.cuda.synchronize()
    ntpr, _, ntpe, itr, _ = lay
    ol = oracle.layout(idx, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])
    o = oracle.dispatch_packed(None, idx, E, R, cap)
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    np.testing.assert_array_equal(count.cpu().numpy(), o["packed_recv_count"])
    np.testing.assert_array_equal(h.recv_src_info.cpu().numpy(), o["recv_src_info"])
    if fp8 is None:
        _check_packed_rows(recv, x_dev, o["dst_row"])
    else:
        q, sc = recv
        oq, osc = oracle.cast_to_fp8(x, fp8)
        sel_t, sel_k = np.nonzero(o["dst_row"] >= 0)
        rows = o["dst_row"][sel_t, sel_k]
        np.testing.assert_array_equal(q.view(torch.uint8).reshape(-1, H).cpu().numpy()[rows], oq[sel_t])
        np.testing.assert_array_equal(sc.reshape(-1, H // 128).cpu().numpy()[rows].view(np.uint8),
                                      osc[sel_t].view(np.uint8))
