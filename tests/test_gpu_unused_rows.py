"""Rows without data are neither read by the combines nor written by the
dispatches.

A receive buffer has rows without data: alignment padding, spare capacity
past the last segment, the unused tail of each fixed-capacity packed segment
and the rank-granular buffer's spare rows (recv_src_idx / recv_src_info < 0
marks them). The combine tests fill exactly those rows with a bf16 NaN and
check that the combine output is bit-identical to the combine of the
untouched buffer: a NaN in any row that is read, even one weighted by 0,
would reach the output. The dispatch tests hand the dispatch a receive
buffer that is the head of a larger sentinel-filled allocation and check
that only the rows with data changed, each to its source row."""
import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import synth
from gpu_util import DEV, dev_bf16, dev_f32, dev_i64, say

pytestmark = pytest.mark.gpu

NAN_BITS = 0x7FC0  # bf16 quiet NaN


def _inputs(T, K, E, H, seed, p_neg=0.2):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx[rng.random((T, K)) < p_neg] = -1
    x = synth.normal_bf16(synth.stream_key(seed, 97, 1), T * H).reshape(T, H)
    w = synth.softmax_weights(synth.stream_key(seed, 97, 3), T, K)
    return idx, x, w


def _poisoned(buf, no_data):
    """A copy of buf whose rows flagged in no_data (one flag per row) are NaN."""
    assert no_data.any(), "the case must have rows without data"
    y = buf.clone()
    rows = y.view(torch.int16).view(-1, buf.shape[-1])
    assert rows.shape[0] == no_data.size
    rows[torch.from_numpy(no_data.reshape(-1)).to(DEV)] = NAN_BITS
    return y


def _same_bits(a, b):
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.isnan(b.float()).any()


@pytest.mark.parametrize("T,K,E,R,H,align,extra", [(300, 4, 64, 8, 64, 16, 500), (2100, 8, 32, 4, 136, 8, 3000),
                                                   (128, 8, 256, 16, 256, 32, 0)])
def test_expert_combine_reads_only_rows_with_data(T, K, E, R, H, align, extra):
    idx, x, w = _inputs(T, K, E, H, seed=T)
    cap = cgd.dispatch_capacity(T, K, E, align) + extra
    say(f"[unused rows, expert] T={T} K={K} E={E} align={align} cap={cap}")
    recv, _, h = cgd.dispatch(dev_bf16(x), dev_i64(idx), E, R, expert_alignment=align, recv_capacity=cap)
    wd = dev_f32(w)
    clean = cgd.combine(recv, h, wd)
    torch.cuda.synchronize()
    no_data = h.recv_src_idx.cpu().numpy() < 0
    _same_bits(clean, cgd.combine(_poisoned(recv, no_data), h, wd))


@pytest.mark.parametrize("T,K,E,R,H,cap", [(128, 8, 64, 8, 64, 40), (3000, 8, 32, 4, 72, 900),
                                           (2000, 4, 16, 4, 64, 400)])
def test_packed_combine_reads_only_rows_with_data(T, K, E, R, H, cap):
    """The last case overflows some experts' capacity and leaves others
    with spare rows: the dropped slots are not read either."""
    idx, x, w = _inputs(T, K, E, H, seed=T + 1)
    counts = np.bincount(idx[idx >= 0], minlength=E)
    say(f"[unused rows, packed] T={T} K={K} E={E} cap={cap} counts {counts.min()}..{counts.max()}")
    if cap == 400:
        assert counts.max() > cap > counts.min()
    recv, _, h = cgd.low_latency_dispatch(dev_bf16(x), dev_i64(idx), E, R, expert_capacity=cap)
    wd = dev_f32(w)
    clean = cgd.low_latency_combine(recv, wd, h)
    torch.cuda.synchronize()
    no_data = h.recv_src_info.cpu().numpy() < 0
    _same_bits(clean, cgd.low_latency_combine(_poisoned(recv, no_data), wd, h))


@pytest.mark.parametrize("T,K,E,R,H,align,extra", [(300, 4, 32, 4, 40, 4, 999), (2000, 8, 64, 8, 64, 8, 100)])
def test_normal_combine_reads_only_rows_with_data(T, K, E, R, H, align, extra):
    idx, x, w = _inputs(T, K, E, H, seed=T + 2)
    idx_d = dev_i64(idx)
    _, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx_d, E, R)
    cap = cgd.normal_capacity(T, K, R) + extra
    say(f"[unused rows, rank-granular] T={T} K={K} E={E} R={R} cap={cap}")
    recv, _, rw, _, h = cgd.normal_dispatch(dev_bf16(x), itr, num_tokens_per_expert=ntpe, topk_idx=idx_d,
                                            topk_weights=dev_f32(w), num_experts=E, expert_alignment=align,
                                            recv_capacity=cap)
    clean, cw = cgd.normal_combine(recv, h, rw)
    torch.cuda.synchronize()
    no_data = h.recv_src_idx.cpu().numpy() < 0
    bad, cw2 = cgd.normal_combine(_poisoned(recv, no_data), h, rw)
    _same_bits(clean, bad)
    assert torch.equal(cw.view(torch.int32), cw2.view(torch.int32))


# ---- the dispatches write only rows that receive data ----
SENTINEL = 0x5A5A  # a finite bf16 bit pattern
GUARD = 64         # rows past the receive buffer, inside the same allocation


def _guarded(rows, H):
    """A receive buffer of `rows` rows, the first rows of a sentinel-filled
    allocation GUARD rows longer, and that allocation."""
    big = torch.full((rows + GUARD, H), SENTINEL, dtype=torch.int16, device=DEV)
    return big[:rows].view(torch.bfloat16), big


def _check_writes(big, rows, src, x):
    """Rows with src >= 0 hold x[src], every other row and the guard rows
    still hold the sentinel."""
    torch.cuda.synchronize()
    g = big.cpu().numpy()
    assert (g[rows:] == SENTINEL).all(), "write past the receive buffer"
    src = src.reshape(-1)
    assert (g[:rows][src < 0] == SENTINEL).all(), "write to a row without data"
    np.testing.assert_array_equal(g[:rows][src >= 0], x.view(np.int16)[src[src >= 0]])


@pytest.mark.parametrize("T,K,E,R,H,align,extra", [(300, 4, 64, 8, 64, 16, 500), (2100, 8, 32, 4, 136, 8, 3000),
                                                   (128, 8, 256, 16, 256, 32, 0), (1100, 16, 64, 8, 64, 4, 77)])
def test_expert_dispatch_writes_only_rows_with_data(T, K, E, R, H, align, extra):
    """The broadcast apply, the row copy, the one-launch dispatch and the
    top-16 apply."""
    idx, x, _ = _inputs(T, K, E, H, seed=T + 3)
    cap = cgd.dispatch_capacity(T, K, E, align) + extra
    say(f"[writes, expert] T={T} K={K} E={E} align={align} cap={cap}")
    recv, big = _guarded(cap, H)
    _, _, h = cgd.dispatch(dev_bf16(x), dev_i64(idx), E, R, expert_alignment=align, recv_capacity=cap, recv_x=recv)
    torch.cuda.synchronize()
    _check_writes(big, cap, h.recv_src_idx.cpu().numpy(), x)


@pytest.mark.parametrize("T,K,E,R,H,cap", [(128, 8, 64, 8, 64, 40), (2000, 4, 16, 4, 64, 400)])
def test_packed_dispatch_writes_only_rows_with_data(T, K, E, R, H, cap):
    idx, x, _ = _inputs(T, K, E, H, seed=T + 4)
    say(f"[writes, packed] T={T} K={K} E={E} cap={cap}")
    recv, big = _guarded(E * cap, H)
    _, _, h = cgd.low_latency_dispatch(dev_bf16(x), dev_i64(idx), E, R, expert_capacity=cap,
                                       out=recv.view(E, cap, H))
    torch.cuda.synchronize()
    _check_writes(big, E * cap, h.recv_src_info.cpu().numpy(), x)


@pytest.mark.parametrize("T,K,E,R,H,align,extra", [(300, 4, 32, 4, 40, 4, 999), (2000, 8, 64, 8, 64, 8, 100)])
def test_normal_dispatch_writes_only_rows_with_data(T, K, E, R, H, align, extra):
    idx, x, w = _inputs(T, K, E, H, seed=T + 5)
    idx_d = dev_i64(idx)
    _, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx_d, E, R)
    cap = cgd.normal_capacity(T, K, R) + extra
    say(f"[writes, rank-granular] T={T} K={K} E={E} R={R} cap={cap}")
    recv, big = _guarded(cap, H)
    _, _, _, _, h = cgd.normal_dispatch(dev_bf16(x), itr, num_tokens_per_expert=ntpe, topk_idx=idx_d,
                                        topk_weights=dev_f32(w), num_experts=E, expert_alignment=align,
                                        recv_capacity=cap, recv_x=recv)
    torch.cuda.synchronize()
    _check_writes(big, cap, h.recv_src_idx.cpu().numpy(), x)


@pytest.mark.parametrize("T,K,E,R,H", [(300, 4, 64, 8, 64), (2100, 8, 32, 4, 136), (100, 16, 64, 8, 256)])
def test_combines_write_only_their_output(T, K, E, R, H):
    """Each combine writes its [T, H] output and nothing past it."""
    idx, x, w = _inputs(T, K, E, H, seed=T + 6)
    x_d, idx_d, w_d = dev_bf16(x), dev_i64(idx), dev_f32(w)
    say(f"[writes, combine outputs] T={T} K={K} E={E} R={R} H={H}")
    recv, _, h = cgd.dispatch(x_d, idx_d, E, R)
    out, big = _guarded(T, H)
    cgd.combine(recv, h, w_d, out=out)
    precv, _, ph = cgd.low_latency_dispatch(x_d, idx_d, E, R, expert_capacity=T)
    pout, pbig = _guarded(T, H)
    cgd.low_latency_combine(precv, w_d, ph, out=pout)
    _, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx_d, E, R)
    nrecv, _, rw, _, nh = cgd.normal_dispatch(x_d, itr, num_tokens_per_expert=ntpe, topk_idx=idx_d, topk_weights=w_d,
                                              num_experts=E)
    nout, nbig = _guarded(T, H)
    cgd.normal_combine(nrecv, nh, rw, out=nout)
    torch.cuda.synchronize()
    for b in (big, pbig, nbig):
        assert (b[T:].cpu().numpy() == SENTINEL).all(), "write past the combine output"
        assert not (b[:T].cpu().numpy() == SENTINEL).all(axis=1).any(), "an output row was not written"


@pytest.mark.parametrize("T,K,E,R,H,align,extra,cast", [(2100, 8, 32, 4, 256, 8, 3000, True),
                                                         (300, 4, 64, 8, 384, 16, 500, False),
                                                         (128, 8, 256, 16, 256, 1, 40, True)])
def test_fp8_dispatch_writes_only_rows_with_data(T, K, E, R, H, align, extra, cast):
    """FP8 rows (codes and fp32 block scales), cast on dispatch or dispatched
    as an FP8 tuple: only the rows with data change, each to its source
    token's codes and scales from the standalone cast."""
    idx, x, _ = _inputs(T, K, E, H, seed=T + 7)
    fmt = cgd.SCALE_F32
    cap = cgd.dispatch_capacity(T, K, E, align) + extra
    nb = H // 128
    say(f"[writes, fp8] T={T} K={K} E={E} H={H} cap={cap} cast_on_dispatch={cast}")
    qbig = torch.full((cap + GUARD, H), 0x5A, dtype=torch.uint8, device=DEV)
    sbig = torch.full((cap + GUARD, nb), 12345.0, dtype=torch.float32, device=DEV)
    recv = (qbig[:cap].view(torch.float8_e4m3fn), sbig[:cap])
    x_d = dev_bf16(x)
    q_ref, s_ref = cgd.per_token_cast_to_fp8(x_d, fmt)
    if cast:
        _, _, h = cgd.dispatch(x_d, dev_i64(idx), E, R, expert_alignment=align, recv_capacity=cap, recv_x=recv,
                            cast_fp8=fmt)
    else:
        _, _, h = cgd.dispatch((q_ref, s_ref), dev_i64(idx), E, R, expert_alignment=align, recv_capacity=cap,
                            recv_x=recv)
    torch.cuda.synchronize()
    src = h.recv_src_idx.cpu().numpy()
    data = src >= 0
    q, s = qbig.cpu().numpy(), sbig.cpu().numpy()
    assert (q[cap:] == 0x5A).all() and (s[cap:] == 12345.0).all(), "write past the receive buffer"
    assert (q[:cap][~data] == 0x5A).all() and (s[:cap][~data] == 12345.0).all(), "write to a row without data"
    qr = q_ref.view(torch.uint8).cpu().numpy()
    sr = s_ref.contiguous().cpu().numpy()
    np.testing.assert_array_equal(q[:cap][data], qr[src[data]])
    np.testing.assert_array_equal(s[:cap][data].view(np.int32), sr[src[data]].view(np.int32))
