"""The binding's own bookkeeping around the C ABI, on device tensors:

* a rank-granular plan leaves each token's place in a workspace that the
  apply reads, so an apply must never read another plan's words: with the
  stream's shared workspace the binding refuses an overwritten plan, and plans
  given workspaces of their own stay valid side by side (checked against the
  oracle bit for bit);
* caller-supplied FP8 receive buffers must hold the scale format the kernel
  writes (1-byte UE8M0 or 4-byte fp32 scales), checked before any launch;
* a workspace that a larger call outgrows stays alive, so a HIP graph
  captured on it keeps replaying correctly."""
import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import oracle
import synth
from gpu_util import DEV, dev_bf16, dev_f32, dev_i64, host_bits, say

pytestmark = pytest.mark.gpu


def _normal_inputs(seed, T=700, H=256):
    w = synth.WORKLOADS["prefill"].replace(T=T, H=H)
    base = synth.WORKLOADS["prefill"]
    idx = synth.make_topk_idx(base, seed=seed)[:T]
    wts = synth.make_weights(base, seed=seed)[:T]
    x = synth.make_x(w, seed=seed)
    return w, idx, wts, x


def _check_normal(w, idx, wts, x, out):
    recv_x, ridx, rw, _, h = out
    torch.cuda.synchronize()
    itr = oracle.layout(idx, w.E, w.R)[2]
    o = oracle.dispatch_normal(x, itr, w.E, w.K, None, idx, wts)
    for got, key in ((h.rank_offset, "rank_offset"), (h.send_row, "send_row"), (h.recv_src_idx, "recv_src_idx"),
                     (ridx, "recv_topk_idx"), (rw, "recv_topk_weights")):
        np.testing.assert_array_equal(got.cpu().numpy(), o[key], err_msg=key)
    data = o["recv_src_idx"] >= 0
    np.testing.assert_array_equal(host_bits(recv_x)[data], o["recv_x"][data])


def test_overwritten_shared_plan_workspace_is_refused():
    say("shared normal-plan workspace: a second plan invalidates the first")
    w, idx_a, wts_a, x_a = _normal_inputs(1)
    _, idx_b, wts_b, x_b = _normal_inputs(2)
    _, plan_a = cgd.layout_and_normal_dispatch_plan(dev_i64(idx_a), w.E, w.R)
    _, plan_b = cgd.layout_and_normal_dispatch_plan(dev_i64(idx_b), w.E, w.R)
    assert plan_a.workspace.data_ptr() == plan_b.workspace.data_ptr()
    with pytest.raises(ValueError, match="overwritten"):
        cgd.normal_dispatch_apply(dev_bf16(x_a), plan_a, dev_i64(idx_a), dev_f32(wts_a))
    # the latest plan is still good, and may be applied more than once
    for _ in range(2):
        out = cgd.normal_dispatch_apply(dev_bf16(x_b), plan_b, dev_i64(idx_b), dev_f32(wts_b))
        _check_normal(w, idx_b, wts_b, x_b, out)
    # the same holds for the plan from is_token_in_rank alone
    itr_a = cgd.get_dispatch_layout(dev_i64(idx_a), w.E, w.R)[3]
    itr_b = cgd.get_dispatch_layout(dev_i64(idx_b), w.E, w.R)[3]
    pa = cgd.normal_dispatch_plan(itr_a, num_experts=w.E)
    pb = cgd.normal_dispatch_plan(itr_b, num_experts=w.E)
    with pytest.raises(ValueError, match="overwritten"):
        cgd.normal_dispatch_apply(dev_bf16(x_a), pa, dev_i64(idx_a), dev_f32(wts_a))
    _check_normal(w, idx_b, wts_b, x_b, cgd.normal_dispatch_apply(dev_bf16(x_b), pb, dev_i64(idx_b), dev_f32(wts_b)))


def test_plans_with_workspaces_of_their_own_apply_in_any_order():
    say("normal plans with own workspaces, applied after both were made")
    w, idx_a, wts_a, x_a = _normal_inputs(3)
    _, idx_b, wts_b, x_b = _normal_inputs(4)
    n = cgd.layout_and_normal_workspace_bytes(w.T, w.K, w.E, w.R)
    ws_a = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ws_b = torch.zeros(n, dtype=torch.uint8, device=DEV)
    _, plan_a = cgd.layout_and_normal_dispatch_plan(dev_i64(idx_a), w.E, w.R, workspace=ws_a)
    _, plan_b = cgd.layout_and_normal_dispatch_plan(dev_i64(idx_b), w.E, w.R, workspace=ws_b)
    assert plan_a.workspace is ws_a and plan_b.workspace is ws_b
    out_b = cgd.normal_dispatch_apply(dev_bf16(x_b), plan_b, dev_i64(idx_b), dev_f32(wts_b))
    out_a = cgd.normal_dispatch_apply(dev_bf16(x_a), plan_a, dev_i64(idx_a), dev_f32(wts_a))
    _check_normal(w, idx_a, wts_a, x_a, out_a)
    _check_normal(w, idx_b, wts_b, x_b, out_b)
    # plans from is_token_in_rank alone, each with its own workspace
    m = cgd.normal_workspace_bytes(w.T, w.R)
    itr_a = cgd.get_dispatch_layout(dev_i64(idx_a), w.E, w.R)[3]
    itr_b = cgd.get_dispatch_layout(dev_i64(idx_b), w.E, w.R)[3]
    pa = cgd.normal_dispatch_plan(itr_a, num_experts=w.E, workspace=torch.zeros(m, dtype=torch.uint8, device=DEV))
    pb = cgd.normal_dispatch_plan(itr_b, num_experts=w.E, workspace=torch.zeros(m, dtype=torch.uint8, device=DEV))
    _check_normal(w, idx_a, wts_a, x_a, cgd.normal_dispatch_apply(dev_bf16(x_a), pa, dev_i64(idx_a), dev_f32(wts_a)))
    _check_normal(w, idx_b, wts_b, x_b, cgd.normal_dispatch_apply(dev_bf16(x_b), pb, dev_i64(idx_b), dev_f32(wts_b)))
    with pytest.raises(ValueError, match="needs"):
        cgd.normal_dispatch_plan(itr_a, num_experts=w.E, workspace=torch.zeros(16, dtype=torch.uint8, device=DEV))


def test_fp8_receive_buffers_must_hold_the_written_scale_format():
    say("FP8 receive buffers: scale storage checked against the format")
    T, H, E, R = 64, 256, 16, 4
    idx = dev_i64(synth.make_topk_idx(synth.WORKLOADS["tiny"].replace(T=T, K=2, E=E, R=R), seed=0))
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    cap = cgd.dispatch_capacity(T, 2, E)
    q = torch.empty((cap, H), dtype=torch.uint8, device=DEV)
    s8 = torch.empty((cap, H // 128), dtype=torch.uint8, device=DEV)
    s32 = torch.empty((cap, H // 128), dtype=torch.float32, device=DEV)
    for fmt, bad in ((cgd.SCALE_F32, s8), (cgd.SCALE_POW2, s8), (cgd.SCALE_UE8M0, s32)):
        with pytest.raises(TypeError, match="scales"):
            cgd.dispatch(x, idx, E, R, cast_fp8=fmt, recv_x=(q, bad))
    # a tuple dispatch keeps the scale storage of its input
    xq, xs = cgd.per_token_cast_to_fp8(x, cgd.SCALE_F32)
    with pytest.raises(TypeError, match="scales"):
        cgd.dispatch((xq, xs), idx, E, R, recv_x=(q, s8))
    with pytest.raises(TypeError, match="scales"):
        cgd.per_token_cast_back((xq, xs), scale_format=cgd.SCALE_UE8M0)
    # the packed FP8 receive tuple: shape, storage and format
    ecap = 32
    good_q = torch.empty((E * ecap, H), dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    with pytest.raises(TypeError, match="scales"):
        cgd.low_latency_dispatch(x, idx, E, R, expert_capacity=ecap, use_fp8=True, scale_format=cgd.SCALE_UE8M0,
                                 out=(good_q, torch.empty((E * ecap, H // 128), dtype=torch.float32, device=DEV)))
    with pytest.raises(ValueError, match="codes"):
        cgd.low_latency_dispatch(x, idx, E, R, expert_capacity=ecap, use_fp8=True,
                                 out=(good_q[: E * ecap - 1], torch.empty((E * ecap, H // 128), device=DEV)))
    with pytest.raises(ValueError, match="scales"):
        cgd.low_latency_dispatch(x, idx, E, R, expert_capacity=ecap, use_fp8=True,
                                 out=(good_q, torch.empty((E * ecap, 1), device=DEV)))
    with pytest.raises(ValueError, match="contiguous"):
        cgd.low_latency_dispatch(x, idx, E, R, expert_capacity=ecap, use_fp8=True,
                                 out=(good_q, torch.empty((H // 128, E * ecap), device=DEV).t()))
    # a well-formed 3-D tuple works and equals the packed dispatch's own buffers
    q3 = torch.empty((E, ecap, H), dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
    s3 = torch.empty((E, ecap, H // 128), dtype=torch.float32, device=DEV)
    (gq, gs), count, _ = cgd.low_latency_dispatch(x, idx, E, R, expert_capacity=ecap, use_fp8=True, out=(q3, s3))
    (rq, rs), count2, _ = cgd.low_latency_dispatch(x, idx, E, R, expert_capacity=ecap, use_fp8=True)
    torch.cuda.synchronize()
    assert torch.equal(count, count2)
    n = count.cpu().numpy()
    for e in range(E):
        assert torch.equal(gq[e, : n[e]].view(torch.uint8), rq[e, : n[e]].view(torch.uint8))
        assert torch.equal(gs[e, : n[e]], rs[e, : n[e]])


def test_outgrown_workspace_stays_valid_for_a_captured_graph():
    say("graph captured on a workspace, then a larger eager call outgrows it")
    w = synth.WORKLOADS["prefill"].replace(T=600, H=128)
    base = synth.WORKLOADS["prefill"]
    idx_np = synth.make_topk_idx(base, seed=11)[: w.T]
    idx = dev_i64(idx_np)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            _, plan = cgd.layout_and_dispatch_plan(idx, w.E, w.R)
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            _, plan = cgd.layout_and_dispatch_plan(idx, w.E, w.R)
        ws_captured = plan.workspace
        # a larger eager call on the same stream replaces the stream's workspace
        big = dev_i64(synth.make_topk_idx(synth.WORKLOADS["stress"], seed=1))
        _, big_plan = cgd.layout_and_dispatch_plan(big, 512, 64)
        s.synchronize()
    assert big_plan.workspace.data_ptr() != ws_captured.data_ptr()
    want = oracle.dispatch(None, idx_np, w.E, w.R, hidden=8, with_rows=False)
    for _ in range(4):
        plan.handle.dst_row.fill_(-7)
        plan.handle.expert_offset.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(plan.handle.dst_row.cpu().numpy(), want["dst_row"])
        np.testing.assert_array_equal(plan.handle.expert_offset.cpu().numpy(), want["expert_offset"])
        np.testing.assert_array_equal(plan.handle.recv_src_idx.cpu().numpy(), want["recv_src_idx"])


def test_init_loads_the_code_ahead_of_the_first_call():
    say("cgd_init twice, then a layout against the oracle")
    cgd.init(DEV)
    cgd.init(DEV)
    w = synth.WORKLOADS["tiny"]
    idx_np = synth.make_topk_idx(w, seed=4)
    ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(dev_i64(idx_np), w.E, w.R)
    torch.cuda.synchronize()
    o_ntpr, o_ntpe, o_itr = oracle.layout(idx_np, w.E, w.R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), o_ntpr)
    np.testing.assert_array_equal(ntpe.cpu().numpy(), o_ntpe)
    np.testing.assert_array_equal(itr.cpu().numpy(), o_itr)
