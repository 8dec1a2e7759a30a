"""Concurrent calls from two streams: each stream gets its own workspace (the
binding keys workspaces by stream) and every call leaves it zeroed, so
interleaved layout / dispatch / combine on two streams give exactly what the
same calls give one after another on one stream."""
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import synth
from gpu_util import dev_bf16, dev_f32, dev_i64, say

pytestmark = pytest.mark.gpu


def _step(x, idx, wt, E, R):
    ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx, E, R)
    recv_x, _, h = cgd.dispatch(x, idx, E, R)
    out = cgd.combine(recv_x, h, wt)
    _, ridx, rw, _, nh = cgd.normal_dispatch(x, itr, ntpe, idx, wt, num_experts=E)
    nout, _ = cgd.normal_combine(cgd.normal_dispatch(x, handle=nh)[0], nh, rw)
    return [ntpr, ntpe, itr, h.dst_row, h.recv_src_idx, out, nh.send_row, ridx, nout]


def test_two_streams_interleaved_equal_serial():
    wa = synth.WORKLOADS["prefill"].replace(T=1500, H=1024)
    wb = synth.WORKLOADS["skewed"].replace(T=1000, H=512)
    ins = []
    for w, seed in ((wa, 1), (wb, 2)):
        inp = synth.make_inputs(w, seed=seed)
        ins.append((w, dev_bf16(inp["x"]), dev_i64(inp["topk_idx"]), dev_f32(inp["topk_weights"])))
    serial = [_step(x, idx, wt, w.E, w.R) for (w, x, idx, wt) in ins]
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    results = [None, None]
    for _ in range(5):  # interleaved issue; later rounds overwrite earlier ones
        for i, (w, x, idx, wt) in enumerate(ins):
            with torch.cuda.stream(streams[i]):
                results[i] = _step(x, idx, wt, w.E, w.R)
    torch.cuda.synchronize()
    say("[streams] 5 interleaved rounds on 2 streams")
    for i in range(2):
        for a, b in zip(results[i], serial[i]):
            assert torch.equal(a, b), f"stream {i} differs"
