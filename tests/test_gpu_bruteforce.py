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
        recv, h = cgd.dispatch(x, idx, E, R)
        one.append((recv, h.expert_offset, h.dst_row, h.recv_src_idx))
        (ntpr2, _, ntpe2, itr2, _), plan = cgd.layout_and_dispatch_plan(idx, E, R)
        recv2, h2 = cgd.dispatch_apply(x, plan)
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
