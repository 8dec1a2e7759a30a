"""The steps bench.py times, captured once in a HIP graph and replayed with
new inputs: every replay must equal the same step run eagerly on those inputs
(expert-granular step with the final rows in the plan and the row-copy
apply; the one-launch small-batch dispatch, with and without the layout
outputs; rank-granular step with the fused layout + plan; the one-call
layout + dispatch of larger batches, bf16, rank-granular and with the FP8
cast, whose plans pull x toward the caches; the one-launch FP8 forms of
small batches, packed included)."""
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import synth
from gpu_util import dev_bf16, dev_f32, dev_i64, say

pytestmark = pytest.mark.gpu


def _expert_step(x, idx, wt, w, out):
    lay, plan = cgd.layout_and_dispatch_plan(idx, w.E, w.R)
    recv, _, h = cgd.dispatch_apply(x, plan)
    cgd.combine(recv, h, wt, out=out)
    return list(lay[0::2][:2]) + [lay[3], h.expert_offset, h.dst_row, h.recv_src_idx, out]


def _small_step(x, idx, wt, w, out):
    recv, _, h = cgd.dispatch(x, idx, w.E, w.R)
    cgd.combine(recv, h, wt, out=out)
    return [h.expert_offset, h.dst_row, h.recv_src_idx, out]


def _small_layout_step(x, idx, wt, w, out):
    (ntpr, _, ntpe, itr, _), recv, _, h = cgd.layout_and_dispatch(x, idx, w.E, w.R)
    cgd.combine(recv, h, wt, out=out)
    return [ntpr, ntpe, itr, h.expert_offset, h.dst_row, h.recv_src_idx, out]


def _normal_step(x, idx, wt, w, out):
    (ntpr, _, ntpe, itr, _), plan = cgd.layout_and_normal_dispatch_plan(idx, w.E, w.R)
    recv, ridx, rw, _, h = cgd.normal_dispatch_apply(x, plan, idx, wt)
    cgd.normal_combine(recv, h, rw, out=out)
    return [ntpr, ntpe, itr, plan.rank_offset, h.send_row, h.recv_src_idx, ridx, out]


def _layout_step(x, idx, wt, w, out):
    (ntpr, _, ntpe, itr, _), recv, nre, h = cgd.layout_and_dispatch(x, idx, w.E, w.R)
    cgd.combine(recv, h, wt, out=out)
    return [ntpr, ntpe, itr, h.expert_offset, h.dst_row, h.recv_src_idx, nre, out]


def _normal_whole_step(x, idx, wt, w, out):
    (ntpr, _, ntpe, itr, _), recv, ridx, rw, nre, h = cgd.layout_and_normal_dispatch(x, idx, wt, w.E, w.R)
    cgd.normal_combine(recv, h, rw, out=out)
    return [ntpr, ntpe, itr, h.rank_offset, h.send_row, h.recv_src_idx, ridx, nre, out]


def _fp8_step(x, idx, wt, w, out):
    (ntpr, _, ntpe, itr, _), (q, sc), nre, h = cgd.layout_and_dispatch(x, idx, w.E, w.R, cast_fp8=cgd.SCALE_F32)
    return [ntpr, ntpe, itr, h.expert_offset, h.dst_row, h.recv_src_idx, nre, q.view(torch.uint8), sc]


def _normal_fp8_step(x, idx, wt, w, out):
    (ntpr, _, ntpe, itr, _), (q, sc), ridx, rw, nre, h = cgd.layout_and_normal_dispatch(x, idx, wt, w.E, w.R,
                                                                                        cast_fp8=cgd.SCALE_F32)
    data = (h.recv_src_idx >= 0).unsqueeze(1)  # rows past the data are not written: compare them as zero
    return [ntpr, ntpe, itr, h.rank_offset, h.send_row, h.recv_src_idx, ridx, nre,
            q.view(torch.uint8) * data.to(torch.uint8), torch.where(data, sc, torch.zeros_like(sc))]


def _packed_fp8_step(x, idx, wt, w, out):
    (q, sc), count, h = cgd.low_latency_dispatch(x, idx, w.E, w.R, expert_capacity=64, use_fp8=True,
                                                 scale_format=cgd.SCALE_UE8M0)
    data = (h.recv_src_info.reshape(-1) >= 0).unsqueeze(1)  # rows past each count are not written
    return [count, h.recv_src_info, h.dst_row, q.view(torch.uint8).reshape(data.shape[0], -1) * data.to(torch.uint8),
            sc.reshape(data.shape[0], -1) * data.to(torch.uint8)]


@pytest.mark.parametrize("kind,T", [("expert", 2500), ("small", 200), ("small_layout", 128), ("normal", 2500),
                                    ("normal", 100), ("layout", 2500), ("normal_whole", 2500), ("normal_whole", 200),
                                    ("fp8_cast", 2500), ("fp8_cast", 200), ("normal_fp8", 2500), ("normal_fp8", 200),
                                    ("packed_fp8", 128)])
def test_step_replays_from_a_captured_graph(kind, T):
    w = synth.WORKLOADS["prefill"].replace(T=T, H=1024)
    step = {"expert": _expert_step, "small": _small_step, "small_layout": _small_layout_step,
            "normal": _normal_step, "layout": _layout_step, "normal_whole": _normal_whole_step,
            "fp8_cast": _fp8_step, "normal_fp8": _normal_fp8_step, "packed_fp8": _packed_fp8_step}[kind]
    inputs = [synth.make_inputs(w, seed=s) for s in range(5)]
    sx = dev_bf16(inputs[0]["x"])
    sidx = dev_i64(inputs[0]["topk_idx"])
    swt = dev_f32(inputs[0]["topk_weights"])
    sout = torch.empty_like(sx)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):  # warm-up on the capture stream: its workspaces exist before capture
            step(sx, sidx, swt, w, sout)
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        static = step(sx, sidx, swt, w, sout)
    torch.cuda.synchronize()
    for i, inp in enumerate(inputs[1:]):
        sx.copy_(dev_bf16(inp["x"]))
        sidx.copy_(dev_i64(inp["topk_idx"]))
        swt.copy_(dev_f32(inp["topk_weights"]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eout = torch.empty_like(sx)
        eager = step(dev_bf16(inp["x"]), dev_i64(inp["topk_idx"]), dev_f32(inp["topk_weights"]), w, eout)
        torch.cuda.synchronize()
        for a, b in zip(static, eager):
            assert torch.equal(a, b), f"{kind} replay {i} differs"
    say(f"[graphs] {kind} T={T}: 4 replays equal eager steps")
