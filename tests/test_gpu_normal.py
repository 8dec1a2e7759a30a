"""Parity of the rank-granular ("normal mode") HIP path with the CPU oracle.

rank_offset, send_row, recv_src_idx, recv_topk_idx, recv_topk_weights, the
aligned per-expert counts and the received rows must be bit-exact. The
combine is bit-exact where the fp32 sum is exact (identity experts without
bias: n copies of one bf16 row) and within 1e-2 of the summed term magnitudes
otherwise. Inputs come from the seeded generator, expected values from the
oracle; is_token_in_rank comes from the GPU layout, itself checked against
the oracle."""
import hashlib

import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import oracle
import synth
from gpu_util import DEV, bf16_to_f64, check_combine, dev_bf16, dev_f32, dev_i64, host_bits, say

pytestmark = pytest.mark.gpu

FULL_ORACLE_ROWS = 40_000_000  # recv_x elements up to which the oracle copies every row


def _layout(idx_np, E, R):
    ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(dev_i64(idx_np), E, R)
    o = oracle.layout(idx_np, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), o[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), o[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), o[2])
    return ntpr, ntpe, itr


def _check_rows_on_device(recv_x, x_dev, send_np):
    """recv_x[send_row[t,r]] == x[t] bit for bit for every sent row (chunked)."""
    sel_t, sel_r = np.nonzero(send_np >= 0)
    rows = send_np[sel_t, sel_r]
    step = 1 << 16
    for i in range(0, len(rows), step):
        r = torch.from_numpy(rows[i:i + step].astype(np.int64)).to(DEV)
        t = torch.from_numpy(sel_t[i:i + step].astype(np.int64)).to(DEV)
        assert torch.equal(recv_x.view(torch.int16).index_select(0, r),
                           x_dev.view(torch.int16).index_select(0, t)), f"row mismatch in rows {i}..{i + step}"


def _normal_and_check(x_np, idx_np, wts_np, E, R, align=1, cap=None, with_topk=True, with_counts=True, itr=None,
                      ntpe=None):
    T, K = idx_np.shape
    H = x_np.shape[1]
    if itr is None:
        _, ntpe, itr = _layout(idx_np, E, R)
    x_dev = dev_bf16(x_np)
    args = dict(num_tokens_per_expert=ntpe if with_counts else None, num_experts=E, num_topk=K,
                expert_alignment=align, recv_capacity=cap)
    if with_topk:
        args.update(topk_idx=dev_i64(idx_np), topk_weights=dev_f32(wts_np))
    recv_x, ridx, rw, nre, h = cgd.normal_dispatch(x_dev, itr, **args)
    torch.cuda.synchronize()
    itr_np = itr.cpu().numpy()
    want_rows = T * H * min(K, R) <= FULL_ORACLE_ROWS
    o = oracle.dispatch_normal(x_np if want_rows else None, itr_np, E, K,
                               ntpe.cpu().numpy() if with_counts else None,
                               idx_np if with_topk else None, wts_np if with_topk else None,
                               align=align, cap=h.recv_capacity, hidden=H)
    np.testing.assert_array_equal(h.rank_offset.cpu().numpy(), o["rank_offset"])
    np.testing.assert_array_equal(h.send_row.cpu().numpy(), o["send_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    if with_topk:
        np.testing.assert_array_equal(ridx.cpu().numpy(), o["recv_topk_idx"])
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), o["recv_topk_weights"].view(np.uint32))
    else:
        assert ridx is None and rw is None
    if with_counts:
        np.testing.assert_array_equal(nre.cpu().numpy(), o["num_recv_tokens_per_expert"])
    if want_rows:
        data = o["recv_src_idx"] >= 0
        np.testing.assert_array_equal(host_bits(recv_x)[data], o["recv_x"][data])
    else:
        _check_rows_on_device(recv_x, x_dev, o["send_row"])
    return x_dev, recv_x, rw, h, o, itr_np


def _term_mag(y_bits, send, b0=None, b1=None):
    """sum of |terms| of the normal combine per element, in double."""
    T, R = send.shape
    out = np.zeros((T, y_bits.shape[1]))
    for r in range(R):
        sel = send[:, r] >= 0
        if sel.any():
            out[sel] += np.abs(bf16_to_f64(y_bits[send[sel, r]]))
    for b in (b0, b1):
        if b is not None:
            out += np.abs(bf16_to_f64(b))
    return out


def _combine_and_check(y_np, h, send_np, rw_dev, rw_np, b0=None, b1=None, tok=None):
    bias = tuple(dev_bf16(b) for b in (b0, b1) if b is not None)
    out, cw = cgd.normal_combine(dev_bf16(y_np), h, rw_dev, bias=bias or None)
    torch.cuda.synchronize()
    T = send_np.shape[0]
    tok = np.arange(T) if tok is None else tok
    sb0 = None if b0 is None else b0[tok]
    sb1 = None if b1 is None else b1[tok]
    exp, ecw = oracle.combine_normal(y_np, send_np[tok], rw_np, sb0, sb1, num_topk=h.num_topk)
    got = host_bits(out)[tok]
    frac = check_combine(got, exp, _term_mag(y_np, send_np[tok], sb0, sb1))
    if rw_dev is not None:
        np.testing.assert_allclose(cw.cpu().numpy()[tok], ecw, rtol=2.0 ** -20, atol=0)
    return out, cw, frac


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_normal_workload_parity(name):
    w = synth.WORKLOADS[name]
    say(f"[normal] {name}: T={w.T} H={w.H} K={w.K} E={w.E} R={w.R} routing={w.routing}")
    inp = synth.make_inputs(w, seed=0)
    idx, wts = inp["topk_idx"], inp["topk_weights"]
    x_dev, recv_x, rw, h, o, itr = _normal_and_check(inp["x"], idx, wts, w.E, w.R, align=w.align)
    say(f"[normal] {name}: dispatch ok, {int(o['rank_offset'][-1])} rows of {h.recv_capacity}")

    # identity experts, no bias: n copies of one bf16 row sum exactly in fp32,
    # so the result is the oracle's bit for bit; the summed weights are the
    # input weights with unselected slots at 0
    out, cw = cgd.normal_combine(recv_x, h, rw)
    torch.cuda.synchronize()
    n = itr.sum(axis=1)
    if w.T * w.H <= 40_000_000:
        exp, _ = oracle.combine_normal(host_bits(recv_x), o["send_row"])
        np.testing.assert_array_equal(host_bits(out), exp)
    else:
        for c in np.unique(n):
            sel = torch.from_numpy(np.flatnonzero(n == c)).to(DEV)
            want = (x_dev.index_select(0, sel).float() * float(c)).to(torch.bfloat16)
            assert torch.equal(out.index_select(0, sel).view(torch.int16), want.view(torch.int16))
    np.testing.assert_array_equal(cw.cpu().numpy(), np.where(idx >= 0, wts, 0).astype(np.float32))
    say(f"[normal] {name}: identity combine ok")

    # independent expert outputs and two biases
    cap = h.recv_capacity
    y = synth.make_expert_out(w, cap, seed=0)
    b0 = synth.normal_bf16(synth.stream_key(0, synth.salt_of(w.name + "/bias0"), 1), w.T * w.H).reshape(w.T, w.H)
    b1 = synth.normal_bf16(synth.stream_key(0, synth.salt_of(w.name + "/bias1"), 1), w.T * w.H).reshape(w.T, w.H)
    rw_np = rw.cpu().numpy()
    tok = None if w.T * w.H * w.K <= 300_000_000 else np.unique(np.random.default_rng(1).integers(0, w.T, 512))
    _, _, frac = _combine_and_check(y, h, o["send_row"], rw, rw_np, b0, b1, tok=tok)
    say(f"[normal] {name}: combine ok, bit-identical fraction {frac:.6f}")
    assert frac > 0.99


def _edge(T, K, E, R, H, seed=0, p_neg=0.0, dup=False):
    rng = np.random.default_rng(seed)
    if dup:
        idx = rng.integers(0, E, size=(T, K)).astype(np.int64)
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64) if T else \
            np.zeros((0, K), np.int64)
    if p_neg:
        idx[rng.random((T, K)) < p_neg] = -1
    x = synth.normal_bf16(synth.stream_key(seed, 98, 1), T * H).reshape(T, H)
    wts = synth.softmax_weights(synth.stream_key(seed, 98, 3), T, K)
    return idx, x, wts


NORMAL_EDGE = {
    "T=1": dict(T=1, K=8, E=256, R=8, H=7168),
    "ragged_T=300": dict(T=300, K=8, E=256, R=8, H=512),
    "ragged_T=1025_neg": dict(T=1025, K=6, E=96, R=12, H=136, p_neg=0.3),
    "all_minus_one_rows": dict(T=257, K=4, E=16, R=4, H=64, p_neg=0.9),
    "duplicates": dict(T=513, K=8, E=8, R=2, H=64, dup=True),
    "K=1": dict(T=777, K=1, E=32, R=4, H=8),
    "K=16_E=512_R=64": dict(T=700, K=16, E=512, R=64, H=256),
    "R=1": dict(T=300, K=4, E=64, R=1, H=64),
    "R>64_R=E=384": dict(T=600, K=9, E=384, R=384, H=64),
    "R>64_K=2_R=128": dict(T=400, K=2, E=256, R=128, H=40),
    "R>K_R=64_K=4": dict(T=333, K=4, E=64, R=64, H=24),
    "H=8": dict(T=513, K=2, E=4, R=2, H=8),
    "align16": dict(T=1000, K=8, E=256, R=8, H=64, align=16),
}


@pytest.mark.parametrize("case", list(NORMAL_EDGE))
def test_normal_edge_case_parity(case):
    spec = dict(NORMAL_EDGE[case])
    align = spec.pop("align", 1)
    say(f"[normal-edge] {case}")
    idx, x, wts = _edge(**spec)
    E, R, T, H = spec["E"], spec["R"], spec["T"], spec["H"]
    x_dev, recv_x, rw, h, o, itr = _normal_and_check(x, idx, wts, E, R, align=align)
    y = synth.normal_bf16(synth.stream_key(7, 98, 5), h.recv_capacity * H).reshape(h.recv_capacity, H)
    b0 = synth.normal_bf16(synth.stream_key(7, 98, 6), T * H).reshape(T, H)
    for bias in ((), (b0,), (b0, b0 ^ np.uint16(0x8000))):  # none, one, two (cancelling) bias tensors
        bb = list(bias) + [None] * (2 - len(bias))
        out, cw, frac = _combine_and_check(y, h, o["send_row"], rw, rw.cpu().numpy(), bb[0], bb[1])
        assert frac > 0.99
        if not bias:
            # tokens sent nowhere combine to +0
            assert (host_bits(out)[itr.sum(axis=1) == 0] == 0).all()


ONE_TILE_EDGE = {
    "one_tile_duplicates": dict(T=200, K=8, E=8, R=2, H=64, dup=True),
    "one_tile_neg_T=256": dict(T=256, K=6, E=96, R=12, H=136, p_neg=0.3),
    "one_tile_all_minus_one": dict(T=100, K=4, E=16, R=4, H=64, p_neg=0.9),
    "one_tile_R=1": dict(T=100, K=4, E=64, R=1, H=64),
    "one_tile_H=8": dict(T=64, K=2, E=4, R=2, H=8),
    "one_tile_R>64": dict(T=250, K=9, E=384, R=384, H=64, dup=True),
    "one_tile_align16": dict(T=130, K=8, E=256, R=8, H=64, align=16),
}


@pytest.mark.parametrize("case", list(NORMAL_EDGE) + list(ONE_TILE_EDGE))
def test_normal_edge_case_one_call(case):
    """The edge cases through layout_and_normal_dispatch (layout, plan and
    rows in one call; one launch up to 256 tokens): every output equals the
    oracle's."""
    spec = dict(NORMAL_EDGE.get(case) or ONE_TILE_EDGE[case])
    align = spec.pop("align", 1)
    say(f"[normal-edge, one call] {case}")
    idx, x, wts = _edge(**spec)
    E, R, K, H = spec["E"], spec["R"], spec["K"], spec["H"]
    (ntpr, _, ntpe, itr, _), recv_x, ridx, rw, nre, h = cgd.layout_and_normal_dispatch(
        dev_bf16(x), dev_i64(idx), dev_f32(wts), E, R, expert_alignment=align)
    torch.cuda.synchronize()
    ol = oracle.layout(idx, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])
    o = oracle.dispatch_normal(x, ol[2], E, K, ol[1], idx, wts, align=align, cap=h.recv_capacity, hidden=H)
    for got, key in ((h.rank_offset, "rank_offset"), (h.send_row, "send_row"), (h.recv_src_idx, "recv_src_idx"),
                     (ridx, "recv_topk_idx"), (nre, "num_recv_tokens_per_expert")):
        np.testing.assert_array_equal(got.cpu().numpy(), o[key], err_msg=key)
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), o["recv_topk_weights"].view(np.uint32))
    data = o["recv_src_idx"] >= 0
    np.testing.assert_array_equal(host_bits(recv_x)[data], o["recv_x"][data])


def test_normal_without_topk_and_counts():
    idx, x, wts = _edge(T=700, K=6, E=48, R=6, H=72, seed=3, p_neg=0.2)
    _normal_and_check(x, idx, wts, 48, 6, with_topk=False, with_counts=False)
    _normal_and_check(x, idx, wts, 48, 6, with_topk=True, with_counts=False)
    _normal_and_check(x, idx, wts, 48, 6, with_topk=False, with_counts=True, align=8)


def test_normal_flags_without_experts():
    """A caller's is_token_in_rank may flag a rank that holds none of the
    token's experts (at most num_topk flags per row): the row is still sent,
    with every recv_topk_idx slot -1."""
    T, K, E, R, H = 300, 3, 24, 6, 32
    idx, x, wts = _edge(T=T, K=K, E=E, R=R, H=H, seed=4, p_neg=0.3)
    rng = np.random.default_rng(4)
    itr_np = np.zeros((T, R), np.uint8)
    for t in range(T):
        itr_np[t, rng.permutation(R)[:rng.integers(0, K + 1)]] = 1
    itr = torch.from_numpy(itr_np.astype(bool)).to(DEV)
    ntpe = torch.from_numpy(np.bincount(idx[idx >= 0], minlength=E).astype(np.int32)).to(DEV)
    _normal_and_check(x, idx, wts, E, R, itr=itr, ntpe=ntpe)


def test_normal_extra_capacity_and_zero_tokens():
    idx, x, wts = _edge(T=200, K=4, E=32, R=4, H=40, seed=5)
    _normal_and_check(x, idx, wts, 32, 4, cap=oracle.normal_capacity(200, 4, 4) + 999)
    # no tokens
    e_idx = torch.empty((0, 4), dtype=torch.int64, device=DEV)
    _, _, ntpe, itr, _ = cgd.get_dispatch_layout(e_idx, 16, 4)
    recv_x, ridx, rw, nre, h = cgd.normal_dispatch(
        torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), itr, ntpe, e_idx,
        torch.empty((0, 4), dtype=torch.float32, device=DEV), num_experts=16, expert_alignment=4, recv_capacity=10)
    out, cw = cgd.normal_combine(recv_x, h, rw)
    torch.cuda.synchronize()
    assert h.rank_offset.cpu().tolist() == [0] * 5 and nre.cpu().tolist() == [0] * 16
    assert (h.recv_src_idx.cpu().numpy() == -1).all() and (ridx.cpu().numpy() == -1).all()
    assert (rw.cpu().numpy() == 0).all() and out.shape == (0, 64) and cw.shape == (0, 4)


def test_normal_plan_then_apply_equals_dispatch():
    w = synth.WORKLOADS["prefill"].replace(T=1500, H=1024)
    idx = synth.make_topk_idx(w.replace(name="prefill"), seed=9)[:w.T]
    wts = synth.make_weights(w.replace(name="prefill"), seed=9)[:w.T]
    x_np = synth.make_x(w, seed=9)
    _, ntpe, itr = _layout(idx, w.E, w.R)
    plan = cgd.normal_dispatch_plan(itr, ntpe, num_experts=w.E, expert_alignment=16)
    recv_x, ridx, rw, nre, h = cgd.normal_dispatch_apply(dev_bf16(x_np), plan, dev_i64(idx), dev_f32(wts))
    torch.cuda.synchronize()
    o = oracle.dispatch_normal(x_np, itr.cpu().numpy(), w.E, w.K, ntpe.cpu().numpy(), idx, wts, align=16)
    for got, key in ((h.rank_offset, "rank_offset"), (h.send_row, "send_row"), (h.recv_src_idx, "recv_src_idx"),
                     (ridx, "recv_topk_idx"), (rw, "recv_topk_weights"), (nre, "num_recv_tokens_per_expert")):
        np.testing.assert_array_equal(got.cpu().numpy(), o[key])
    data = o["recv_src_idx"] >= 0
    np.testing.assert_array_equal(host_bits(recv_x)[data], o["recv_x"][data])


def test_normal_cached_matches_fresh():
    w = synth.WORKLOADS["prefill"].replace(T=1000)
    inp = synth.make_inputs(w, seed=3)
    x_dev, recv_x, rw, h, o, itr = _normal_and_check(inp["x"], inp["topk_idx"], inp["topk_weights"], w.E, w.R)
    x2 = synth.make_x(w.replace(name="prefill-second-batch"), seed=3)
    recv2, _, _, _, h2 = cgd.normal_dispatch(dev_bf16(x2), handle=h)
    torch.cuda.synchronize()
    assert h2 is h
    o2 = oracle.dispatch_normal(x2, itr, w.E, w.K)
    data = o2["recv_src_idx"] >= 0
    np.testing.assert_array_equal(host_bits(recv2)[data], o2["recv_x"][data])


def test_normal_one_workspace_serves_many_sizes():
    for T in (1000, 3, 4096, 257, 1, 64, 65):
        idx, x, wts = _edge(T=T, K=8, E=256, R=8, H=64, seed=T)
        _normal_and_check(x, idx, wts, 256, 8)


def test_normal_determinism_20_repeats():
    w = synth.WORKLOADS["prefill"]
    inp = synth.make_inputs(w, seed=5)
    x, idx, wt = dev_bf16(inp["x"]), dev_i64(inp["topk_idx"]), dev_f32(inp["topk_weights"])
    ref = None
    for i in range(20):
        _, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx, w.E, w.R)
        recv_x, ridx, rw, nre, h = cgd.normal_dispatch(x, itr, ntpe, idx, wt, num_experts=w.E)
        out, cw = cgd.normal_combine(recv_x, h, rw)
        torch.cuda.synchronize()
        hh = hashlib.sha256()
        n = int(h.rank_offset[-1].item())  # rows past the data are unspecified
        for t in (h.rank_offset, h.send_row, h.recv_src_idx, ridx, rw, nre, recv_x[:n], out, cw):
            hh.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
        if ref is None:
            ref = hh.hexdigest()
        assert hh.hexdigest() == ref, f"repeat {i} differs"


@pytest.mark.parametrize("T,K,E,R,H,align,p_neg", [(4096, 8, 256, 8, 256, 1, 0.0), (128, 8, 256, 16, 1024, 1, 0.0),
                                                   (1025, 6, 96, 12, 136, 4, 0.3), (700, 16, 384, 384, 64, 1, 0.0),
                                                   (300, 4, 64, 1, 64, 8, 0.1), (1, 2, 8, 2, 8, 1, 0.0),
                                                   (0, 4, 16, 4, 64, 1, 0.0)])
def test_layout_and_normal_plan_in_one_launch(T, K, E, R, H, align, p_neg):
    """get_dispatch_layout + normal_dispatch_plan in one launch: layout
    outputs, rank offsets and aligned counts equal the oracle's, and the apply
    from that plan gives the oracle's rows, send_row and top-k metadata."""
    rng = np.random.default_rng(T + 7 * R)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64) if T else np.zeros((0, K), np.int64)
    idx[rng.random((T, K)) < p_neg] = -1
    x = synth.normal_bf16(synth.stream_key(T, 55, 1), T * H).reshape(T, H)
    wts = synth.softmax_weights(synth.stream_key(T, 55, 3), T, K)
    say(f"[normal] fused layout + plan: T={T} K={K} E={E} R={R} H={H} align={align}")
    idx_dev = dev_i64(idx)
    (ntpr, _, ntpe, itr, _), plan = cgd.layout_and_normal_dispatch_plan(idx_dev, E, R, expert_alignment=align)
    recv_x, ridx, rw, _, h = cgd.normal_dispatch_apply(dev_bf16(x), plan, idx_dev, dev_f32(wts))
    torch.cuda.synchronize()
    ol = oracle.layout(idx, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])
    o = oracle.dispatch_normal(x, ol[2], E, K, ol[1], idx, wts, align=align, cap=h.recv_capacity, hidden=H)
    np.testing.assert_array_equal(plan.rank_offset.cpu().numpy(), o["rank_offset"])
    np.testing.assert_array_equal(plan.num_recv_tokens_per_expert.cpu().numpy(), o["num_recv_tokens_per_expert"])
    np.testing.assert_array_equal(h.send_row.cpu().numpy(), o["send_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    np.testing.assert_array_equal(ridx.cpu().numpy(), o["recv_topk_idx"])
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), o["recv_topk_weights"].view(np.uint32))
    data = o["recv_src_idx"] >= 0
    np.testing.assert_array_equal(host_bits(recv_x)[data], o["recv_x"][data])


@pytest.mark.parametrize("T,K,E,R,H,align,p_neg,with_topk",
                         [(4096, 8, 256, 8, 7168, 1, 0.0, True), (128, 8, 256, 16, 1024, 1, 0.0, True),
                          (2049, 6, 96, 12, 136, 4, 0.2, True), (1500, 16, 512, 64, 256, 8, 0.0, True),
                          (700, 8, 64, 8, 64, 1, 0.0, False), (0, 4, 16, 4, 64, 2, 0.0, True),
                          (700, 9, 384, 384, 64, 1, 0.05, True),
                          # one tile: layout, plan and rows in one launch
                          (256, 8, 256, 8, 7168, 1, 0.0, True), (1, 8, 256, 16, 7168, 1, 0.0, True),
                          (200, 9, 384, 384, 64, 1, 0.05, True), (100, 6, 90, 6, 136, 4, 0.2, True),
                          (64, 16, 512, 64, 256, 8, 0.0, False), (65, 3, 48, 3, 8, 2, 0.3, True)])
def test_layout_and_normal_dispatch_in_one_call(T, K, E, R, H, align, p_neg, with_topk):
    """layout_and_normal_dispatch (the plan pulls x toward the caches, then the
    apply; a batch of one tile in one launch): layout outputs, plan, rows and
    per-row outputs equal the oracle's, and the handle serves the combine."""
    rng = np.random.default_rng(T + 11 * R)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64) if T else np.zeros((0, K), np.int64)
    idx[rng.random((T, K)) < p_neg] = -1
    x = synth.normal_bf16(synth.stream_key(T, 56, 1), T * H).reshape(T, H)
    wts = synth.softmax_weights(synth.stream_key(T, 56, 3), T, K)
    say(f"[normal] layout + dispatch in one call: T={T} K={K} E={E} R={R} H={H} align={align} topk={with_topk}")
    idx_dev = dev_i64(idx)
    (ntpr, _, ntpe, itr, _), recv_x, ridx, rw, nre, h = cgd.layout_and_normal_dispatch(
        dev_bf16(x), idx_dev, dev_f32(wts) if with_topk else None, E, R, expert_alignment=align)
    torch.cuda.synchronize()
    ol = oracle.layout(idx, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])
    o = oracle.dispatch_normal(x, ol[2], E, K, ol[1], idx, wts, align=align, cap=h.recv_capacity, hidden=H)
    np.testing.assert_array_equal(h.rank_offset.cpu().numpy(), o["rank_offset"])
    np.testing.assert_array_equal(nre.cpu().numpy(), o["num_recv_tokens_per_expert"])
    np.testing.assert_array_equal(h.send_row.cpu().numpy(), o["send_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    if with_topk:
        np.testing.assert_array_equal(ridx.cpu().numpy(), o["recv_topk_idx"])
        np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), o["recv_topk_weights"].view(np.uint32))
    else:
        assert ridx is None and rw is None
    data = o["recv_src_idx"] >= 0
    np.testing.assert_array_equal(host_bits(recv_x)[data], o["recv_x"][data])
    if T and with_topk:
        # the handle drives the combine: identity experts and no bias give
        # each token times its fan-out, as the two-call path's handle does
        out, cw = cgd.normal_combine(recv_x, h, rw)
        (_, _, _, _, _), plan = cgd.layout_and_normal_dispatch_plan(idx_dev, E, R, expert_alignment=align)
        rx2, _, rw2, _, h2 = cgd.normal_dispatch_apply(dev_bf16(x), plan, idx_dev, dev_f32(wts))
        out2, cw2 = cgd.normal_combine(rx2, h2, rw2)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
        assert torch.equal(cw.view(torch.int32), cw2.view(torch.int32))
