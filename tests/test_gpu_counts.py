"""num_recv_tokens_per_expert, the dispatch output holding each expert's
receive row count rounded up to expert_alignment ("4 Python接口", section
"Dispatch API", outputs), written on the device by every expert-granular
dispatch entry point, against the oracle's segment sizes (the differences of
its prefix-summed segment offsets) on every workload at three alignments.

The counts depend only on the routing, so the entry points that also move
rows run here with 64-channel rows (the full-width rows are covered by the
parity tests)."""
import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import oracle
import synth
from gpu_util import DEV, dev_bf16, dev_i64, say

pytestmark = pytest.mark.gpu

WORKLOADS = ["tiny", "prefill", "decode", "skewed", "stress"]
H_SMALL = 64


def _oracle_sizes(idx_np, E, R, align):
    o = oracle.dispatch(None, idx_np, E, R, align=align, hidden=8, with_rows=False)
    sizes = np.diff(o["expert_offset"]).astype(np.int32)
    # the same sizes from their definition: slot counts rounded up to the alignment
    cnt = np.bincount(idx_np[idx_np >= 0], minlength=E)
    np.testing.assert_array_equal(sizes, -(-cnt // align) * align)
    return sizes, o["expert_offset"]


@pytest.mark.parametrize("align", [1, 16, 32])
@pytest.mark.parametrize("name", WORKLOADS)
def test_num_recv_tokens_per_expert(name, align):
    w = synth.WORKLOADS[name]
    say(f"num_recv_tokens_per_expert: {name} align={align}")
    idx_np = synth.make_topk_idx(w, seed=0)
    want, want_off = _oracle_sizes(idx_np, w.E, w.R, align)
    idx = dev_i64(idx_np)
    x = dev_bf16(synth.normal_bf16(synth.stream_key(0, synth.salt_of(name), 99), w.T * H_SMALL).reshape(w.T, H_SMALL))

    got = {}
    plan = cgd.dispatch_plan(idx, w.E, w.R, expert_alignment=align)
    got["dispatch_plan"] = plan.handle
    _, plan2 = cgd.layout_and_dispatch_plan(idx, w.E, w.R, expert_alignment=align)
    got["layout_and_dispatch_plan"] = plan2.handle
    _, nre, h = cgd.dispatch(x, idx, w.E, w.R, expert_alignment=align)
    assert nre is h.num_recv_tokens_per_expert
    got["dispatch"] = h
    _, _, nre2, h2 = cgd.layout_and_dispatch(x, idx, w.E, w.R, expert_alignment=align)
    assert nre2 is h2.num_recv_tokens_per_expert
    got["layout_and_dispatch"] = h2
    # the apply and the cached dispatch hand back the handle's counts
    _, nre3, h3 = cgd.dispatch_apply(x, plan)
    assert nre3 is plan.handle.num_recv_tokens_per_expert and h3 is plan.handle
    torch.cuda.synchronize()
    for entry, hd in got.items():
        c = hd.num_recv_tokens_per_expert
        assert c.dtype == torch.int32 and c.device.type == "cuda" and tuple(c.shape) == (w.E,)
        np.testing.assert_array_equal(c.cpu().numpy(), want, err_msg=entry)
        np.testing.assert_array_equal(hd.expert_offset.cpu().numpy(), want_off, err_msg=entry)
        assert hd.num_recv_tokens_per_expert_list() == want.tolist()


def test_counts_of_an_empty_batch_and_of_unselected_slots():
    E, R = 16, 4
    idx = torch.full((5, 3), -1, dtype=torch.int64, device=DEV)
    idx[2, 1] = 7
    x = torch.zeros((5, 8), dtype=torch.bfloat16, device=DEV)
    _, nre, _ = cgd.dispatch(x, idx, E, R, expert_alignment=4)
    want = np.zeros(E, np.int32)
    want[7] = 4
    np.testing.assert_array_equal(nre.cpu().numpy(), want)
    _, nre0, _ = cgd.dispatch(torch.empty((0, 8), dtype=torch.bfloat16, device=DEV),
                              torch.empty((0, 3), dtype=torch.int64, device=DEV), E, R, expert_alignment=4)
    np.testing.assert_array_equal(nre0.cpu().numpy(), np.zeros(E, np.int32))


def test_layout_workspace_returns_to_zero():
    """get_dispatch_layout combines its blocks' counts in accumulators in the
    workspace, which every call must leave at zero (include/cgd.h, the
    workspace rules): calls of several sizes in a row on one caller-owned
    workspace each match the oracle, and the workspace is all zero after
    them."""
    import ctypes
    lib = cgd.load()
    E, R = 256, 8
    sizes = [4096, 700, 1, 9000, 513, 4096]
    base = synth.WORKLOADS["prefill"]
    nbytes = max(lib.cgd_layout_workspace_bytes(T, base.K, E, R) for T in sizes)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for i, T in enumerate(sizes):
        say(f"layout workspace: call {i}, T={T}")
        idx_np = synth.make_topk_idx(base.replace(T=T), seed=20 + i)[:T].copy()
        idx_np[np.random.default_rng(i).random(idx_np.shape) < 0.1] = -1
        idx = dev_i64(idx_np)
        ntpr = torch.full((R,), -7, dtype=torch.int32, device=DEV)
        ntpe = torch.full((E,), -7, dtype=torch.int32, device=DEV)
        itr = torch.empty((T, R), dtype=torch.bool, device=DEV)
        rc = lib.cgd_get_dispatch_layout(ctypes.c_void_p(idx.data_ptr()), T, base.K, E, R,
                                         ctypes.c_void_p(ntpr.data_ptr()), ctypes.c_void_p(ntpe.data_ptr()),
                                         ctypes.c_void_p(itr.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                                         ctypes.c_size_t(ws.numel()), stream)
        assert rc == 0, cgd.load().cgd_last_error()
        torch.cuda.synchronize()
        o_ntpr, o_ntpe, o_itr = oracle.layout(idx_np, E, R)
        np.testing.assert_array_equal(ntpr.cpu().numpy(), o_ntpr)
        np.testing.assert_array_equal(ntpe.cpu().numpy(), o_ntpe)
        np.testing.assert_array_equal(itr.cpu().numpy(), o_itr)
        assert int(ws.count_nonzero()) == 0, f"workspace words left non-zero after call {i}"
