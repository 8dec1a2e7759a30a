"""Every routing of 3 tokens with top-2 of 4 experts, on the GPU.

Each slot holds an expert or -1 and the experts of a token are distinct: 21
choices per token, 9261 routings. For 1, 2 and 4 ranks every routing goes
through get_dispatch_layout, the one-launch dispatch, the plan followed by
the apply, and the combine. Each result is compared with the oracle's:
bit for bit for the layout, the handle and the rows, within the combine
tolerance for the combine (which the oracle pins by brute force on the CPU
as well). The launches of one rank count are issued back to back, and the
stream is synchronised once before the comparison."""
import itertools

import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import oracle
from gpu_util import DEV, check_combine, dev_bf16, dev_f32, dev_i64, host_bits, say, term_magnitude

pytestmark = pytest.mark.gpu

E, T, K, H = 4, 3, 2, 8
ROWS = [(a, b) for a in range(-1, E) for b in range(-1, E) if a < 0 or b < 0 or a != b]


def _stack(ts):
    t = torch.stack(ts)
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy()


@pytest.mark.parametrize("R", [1, 2, 4])
def test_all_small_routings(R):
    cases = np.array(list(itertools.product(ROWS, repeat=T)), dtype=np.int64)  # [9261, T, K]
    assert len(cases) == 21 ** 3
    rng = np.random.default_rng(R)
    x_bits = (rng.integers(0, 2, (T, H)) << 15 | rng.integers(0x3C00, 0x4100, (T, H))).astype(np.uint16)
    w_np = rng.random((T, K)).astype(np.float32)
    idx_all = dev_i64(cases)
    x, w = dev_bf16(x_bits), dev_f32(w_np)
    say(f"[brute force] R={R}: {len(cases)} routings")
    lay, one, two, comb = [], [], [], []
    for c in range(len(cases)):
        idx = idx_all[c]
        ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx, E, R)
        lay.append((ntpr, ntpe, itr))
        recv, _, h = cgd.dispatch(x, idx, E, R)
        one.append((recv, h.expert_offset, h.dst_row, h.recv_src_idx))
        (ntpr2, _, ntpe2, itr2, _), plan = cgd.layout_and_dispatch_plan(idx, E, R)
        recv2, _, h2 = cgd.dispatch_apply(x, plan)
        two.append((ntpr2, ntpe2, itr2, recv2, h2.expert_offset, h2.dst_row, h2.recv_src_idx))
        comb.append(cgd.combine(recv, h, w))
    torch.cuda.synchronize()

    ntpr, ntpe, itr = (_stack([l[i] for l in lay]) for i in range(3))
    recv, off, dst, src = (_stack([o[i] for o in one]) for i in range(4))
    ntpr2, ntpe2, itr2, recv2, off2, dst2, src2 = (_stack([o[i] for o in two]) for i in range(7))
    recv = recv.view(np.uint16)
    recv2 = recv2.view(np.uint16)
    out = _stack(comb).view(np.uint16)
    for c, idx in enumerate(cases):
        o_ntpr, o_ntpe, o_itr = oracle.layout(idx, E, R)
        for g_ntpr, g_ntpe, g_itr in ((ntpr[c], ntpe[c], itr[c]), (ntpr2[c], ntpe2[c], itr2[c])):
            np.testing.assert_array_equal(g_ntpr, o_ntpr, err_msg=f"case {c}")
            np.testing.assert_array_equal(g_ntpe, o_ntpe, err_msg=f"case {c}")
            np.testing.assert_array_equal(g_itr, o_itr, err_msg=f"case {c}")
        d = oracle.dispatch(x_bits, idx, E, R)
        data = d["recv_src_idx"] >= 0
        for g_recv, g_off, g_dst, g_src in ((recv[c], off[c], dst[c], src[c]), (recv2[c], off2[c], dst2[c], src2[c])):
            np.testing.assert_array_equal(g_off, d["expert_offset"], err_msg=f"case {c}")
            np.testing.assert_array_equal(g_dst, d["dst_row"], err_msg=f"case {c}")
            np.testing.assert_array_equal(g_src, d["recv_src_idx"], err_msg=f"case {c}")
            np.testing.assert_array_equal(g_recv[data], d["recv_x"][data], err_msg=f"case {c}")
        exp = oracle.combine(d["recv_x"], d["dst_row"], w_np)
        check_combine(out[c], exp, term_magnitude(d["recv_x"], d["dst_row"], w_np))


@pytest.mark.parametrize("R", [1, 2, 4])
def test_all_small_routings_rank_granular(R):
    """The same routings through the rank-granular path: layout + plan in one
    launch, the apply (rows, send_row, rank-local top-k ids and weights) and
    the combine of identity experts (x times the token's rank count, exact),
    and the one-call layout + dispatch (one launch at this size), all bit for
    bit."""
    cases = np.array(list(itertools.product(ROWS, repeat=T)), dtype=np.int64)
    rng = np.random.default_rng(10 + R)
    x_bits = (rng.integers(0, 2, (T, H)) << 15 | rng.integers(0x3C00, 0x4100, (T, H))).astype(np.uint16)
    w_np = rng.random((T, K)).astype(np.float32)
    idx_all = dev_i64(cases)
    x, w = dev_bf16(x_bits), dev_f32(w_np)
    say(f"[brute force, rank-granular] R={R}: {len(cases)} routings")
    res = []
    for c in range(len(cases)):
        idx = idx_all[c]
        (ntpr, _, ntpe, itr, _), plan = cgd.layout_and_normal_dispatch_plan(idx, E, R)
        recv, ridx, rw, _, h = cgd.normal_dispatch_apply(x, plan, idx, w)
        out, cw = cgd.normal_combine(recv, h, rw)
        (ntpr2, _, ntpe2, itr2, _), recv2, ridx2, rw2, nre2, h2 = cgd.layout_and_normal_dispatch(x, idx, w, E, R)
        res.append((ntpr, ntpe, itr, plan.rank_offset, plan.num_recv_tokens_per_expert, h.send_row,
                    h.recv_src_idx, ridx, rw.view(torch.int32), recv, out, cw.view(torch.int32),
                    ntpr2, ntpe2, itr2, h2.rank_offset, nre2, h2.send_row, h2.recv_src_idx, ridx2,
                    rw2.view(torch.int32), recv2))
    torch.cuda.synchronize()
    (ntpr, ntpe, itr, off, nre, send, src, ridx, rw, recv, out, cw,
     ntpr2, ntpe2, itr2, off2, nre2, send2, src2, ridx2, rw2, recv2) = (_stack([r[i] for r in res])
                                                                        for i in range(22))
    recv, out, recv2 = recv.view(np.uint16), out.view(np.uint16), recv2.view(np.uint16)
    for c, idx in enumerate(cases):
        o_ntpr, o_ntpe, o_itr = oracle.layout(idx, E, R)
        np.testing.assert_array_equal(ntpr[c], o_ntpr, err_msg=f"case {c}")
        np.testing.assert_array_equal(ntpe[c], o_ntpe, err_msg=f"case {c}")
        np.testing.assert_array_equal(itr[c], o_itr, err_msg=f"case {c}")
        o = oracle.dispatch_normal(x_bits, o_itr, E, K, o_ntpe, idx, w_np)
        np.testing.assert_array_equal(off[c], o["rank_offset"], err_msg=f"case {c}")
        np.testing.assert_array_equal(nre[c], o["num_recv_tokens_per_expert"], err_msg=f"case {c}")
        np.testing.assert_array_equal(send[c], o["send_row"], err_msg=f"case {c}")
        np.testing.assert_array_equal(src[c], o["recv_src_idx"], err_msg=f"case {c}")
        np.testing.assert_array_equal(ridx[c], o["recv_topk_idx"], err_msg=f"case {c}")
        np.testing.assert_array_equal(rw[c], o["recv_topk_weights"].view(np.int32), err_msg=f"case {c}")
        data = o["recv_src_idx"] >= 0
        np.testing.assert_array_equal(recv[c][data], o["recv_x"][data], err_msg=f"case {c}")
        o_out, o_cw = oracle.combine_normal(o["recv_x"], o["send_row"], o["recv_topk_weights"])
        np.testing.assert_array_equal(out[c], o_out, err_msg=f"case {c}")
        np.testing.assert_array_equal(cw[c], o_cw.view(np.int32), err_msg=f"case {c}")
        for got, want in ((ntpr2, o_ntpr), (ntpe2, o_ntpe), (itr2, o_itr), (off2, o["rank_offset"]),
                          (nre2, o["num_recv_tokens_per_expert"]), (send2, o["send_row"]),
                          (src2, o["recv_src_idx"]), (ridx2, o["recv_topk_idx"]),
                          (rw2, o["recv_topk_weights"].view(np.int32))):
            np.testing.assert_array_equal(got[c], want, err_msg=f"one call, case {c}")
        np.testing.assert_array_equal(recv2[c][data], o["recv_x"][data], err_msg=f"one call, case {c}")


@pytest.mark.parametrize("R", [1, 2, 4])
def test_all_small_routings_packed(R):
    """The same routings through the fixed-capacity packed layout with room
    for 2 rows per expert (a third token of an expert is dropped) and its
    combine."""
    cap = 2
    cases = np.array(list(itertools.product(ROWS, repeat=T)), dtype=np.int64)
    rng = np.random.default_rng(20 + R)
    x_bits = (rng.integers(0, 2, (T, H)) << 15 | rng.integers(0x3C00, 0x4100, (T, H))).astype(np.uint16)
    w_np = rng.random((T, K)).astype(np.float32)
    idx_all = dev_i64(cases)
    x, w = dev_bf16(x_bits), dev_f32(w_np)
    say(f"[brute force, packed] R={R}: {len(cases)} routings")
    res = []
    for c in range(len(cases)):
        recv, count, h = cgd.low_latency_dispatch(x, idx_all[c], E, R, expert_capacity=cap)
        out = cgd.low_latency_combine(recv, w, h)
        res.append((count, h.recv_src_info, h.dst_row, recv, out))
    torch.cuda.synchronize()
    count, info, dst, recv, out = (_stack([r[i] for r in res]) for i in range(5))
    recv, out = recv.view(np.uint16), out.view(np.uint16)
    for c, idx in enumerate(cases):
        o = oracle.dispatch_packed(x_bits, idx, E, R, cap)
        np.testing.assert_array_equal(count[c], o["packed_recv_count"], err_msg=f"case {c}")
        np.testing.assert_array_equal(info[c], o["recv_src_info"], err_msg=f"case {c}")
        np.testing.assert_array_equal(dst[c], o["dst_row"], err_msg=f"case {c}")
        valid = o["recv_src_info"] >= 0
        np.testing.assert_array_equal(recv[c][valid], o["packed_recv_x"][valid], err_msg=f"case {c}")
        y = o["packed_recv_x"].reshape(E * cap, H)
        check_combine(out[c], oracle.combine(y, o["dst_row"], w_np), term_magnitude(y, o["dst_row"], w_np))
