"""cgd_layout_and_dispatch_noalloc, the entry point for callers that cannot
allocate (its workspace a static device array inside libcgd), against
cgd_layout_and_dispatch (the same work with a workspace of the binding's),
through the C ABI: several calls in a row on one GPU, each later one smaller
than the first, every output equal bit for bit (received rows compared where
they hold data). Outputs start as sentinel values, so nothing left unwritten
can pass."""
import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import synth
from gpu_util import DEV, dev_bf16, dev_i64, say

pytestmark = pytest.mark.gpu


def _case(name, T, align, seed):
    w = synth.WORKLOADS[name]
    idx = synth.make_topk_idx(w, seed=seed)[:T]
    x = synth.make_x(w.replace(T=T), seed=seed)
    return w, idx, x, align


def _noalloc(w, idx_np, x_np, align):
    T, K, E, R, H = idx_np.shape[0], idx_np.shape[1], w.E, w.R, x_np.shape[1]
    cap = cgd.dispatch_capacity(T, K, E, align)
    out = dict(
        recv_x=torch.full((cap, H), -7.0, dtype=torch.bfloat16, device=DEV),
        num_tokens_per_rank=torch.full((R,), -7, dtype=torch.int32, device=DEV),
        num_tokens_per_expert=torch.full((E,), -7, dtype=torch.int32, device=DEV),
        is_token_in_rank=torch.ones((T, R), dtype=torch.bool, device=DEV),
        expert_offset=torch.full((E + 1,), -7, dtype=torch.int32, device=DEV),
        num_recv_tokens_per_expert=torch.full((E,), -7, dtype=torch.int32, device=DEV),
        recv_src_idx=torch.full((cap,), -7, dtype=torch.int32, device=DEV),
        dst_row=torch.full((T, K), -7, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    cgd.layout_and_dispatch_noalloc(dev_bf16(x_np), dev_i64(idx_np), E, R, align, **out)
    return out


def _reference(w, idx_np, x_np, align):
    (ntpr, _, ntpe, itr, _), recv_x, nre, h = cgd.layout_and_dispatch(dev_bf16(x_np), dev_i64(idx_np), w.E, w.R,
                                                                      expert_alignment=align)
    return dict(recv_x=recv_x, num_tokens_per_rank=ntpr, num_tokens_per_expert=ntpe, is_token_in_rank=itr,
                expert_offset=h.expert_offset, num_recv_tokens_per_expert=nre, recv_src_idx=h.recv_src_idx,
                dst_row=h.dst_row)


def test_noalloc_equals_the_workspace_entry_point_on_calls_in_a_row():
    # the first call is the largest; the later ones are smaller and take both
    # paths (several plan tiles with the row copy, one tile in one launch)
    cases = [("prefill", 4096, 1, 0), ("decode", 128, 4, 1), ("skewed", 1000, 16, 2), ("tiny", 37, 1, 3)]
    for name, T, align, seed in cases:
        say(f"no-alloc dispatch: {name} T={T} align={align}")
        w, idx_np, x_np, align = _case(name, T, align, seed)
        got = _noalloc(w, idx_np, x_np, align)
        want = _reference(w, idx_np, x_np, align)
        torch.cuda.synchronize()
        for key in ("num_tokens_per_rank", "num_tokens_per_expert", "is_token_in_rank", "expert_offset",
                    "num_recv_tokens_per_expert", "recv_src_idx", "dst_row"):
            np.testing.assert_array_equal(got[key].cpu().numpy(), want[key].cpu().numpy(), err_msg=f"{name} {key}")
        data = torch.from_numpy(np.flatnonzero(want["recv_src_idx"].cpu().numpy() >= 0)).to(DEV)
        a = got["recv_x"].view(torch.int16).index_select(0, data)
        b = want["recv_x"].view(torch.int16).index_select(0, data)
        assert torch.equal(a, b), f"{name}: received rows differ"
        # the rows hold their source tokens (an independent check of both)
        src = want["recv_src_idx"].cpu().numpy()
        rows = np.flatnonzero(src >= 0)
        np.testing.assert_array_equal(got["recv_x"].view(torch.int16).cpu().numpy()[rows],
                                      x_np.view(np.int16)[src[rows]])


def test_noalloc_refuses_work_beyond_its_scratch():
    # workspace of 1 << 20 tokens x top-4 exceeds the static 8 MiB: refused on
    # the host, nothing enqueued (the outputs keep their sentinels)
    T, K, E, R, H = 1 << 20, 4, 64, 8, 8
    x = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((T, K), dtype=torch.int64, device=DEV)
    cap = T * K
    out = dict(recv_x=torch.empty((cap, H), dtype=torch.bfloat16, device=DEV),
               num_tokens_per_rank=torch.full((R,), -7, dtype=torch.int32, device=DEV),
               num_tokens_per_expert=torch.empty((E,), dtype=torch.int32, device=DEV),
               is_token_in_rank=torch.empty((T, R), dtype=torch.bool, device=DEV),
               expert_offset=torch.empty((E + 1,), dtype=torch.int32, device=DEV),
               num_recv_tokens_per_expert=torch.empty((E,), dtype=torch.int32, device=DEV),
               recv_src_idx=torch.empty((cap,), dtype=torch.int32, device=DEV),
               dst_row=torch.empty((T, K), dtype=torch.int32, device=DEV))
    with pytest.raises(cgd.CgdError, match="workspace"):
        cgd.layout_and_dispatch_noalloc(x, idx, E, R, **out)
    torch.cuda.synchronize()
    assert (out["num_tokens_per_rank"].cpu().numpy() == -7).all()
