"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Layout, counts, offsets, dst_row, recv_src_idx and received rows must be
bit-exact; combine must be within 1e-2 relative (bf16 output, fp32
accumulation). Every input comes from the seeded generator; every expected
value from the oracle."""
import hashlib

import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import oracle
import synth
from gpu_util import (DEV, bf16_to_f64, check_combine, dev_bf16, dev_f32, dev_i64, host_bits, say,
                      term_magnitude)

pytestmark = pytest.mark.gpu

FULL_ORACLE_ROWS = 40_000_000  # recv_x elements up to which the oracle copies every row


def _run_layout(idx_np, E, R):
    ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(dev_i64(idx_np), E, R)
    torch.cuda.synchronize()
    return ntpr.cpu().numpy(), ntpe.cpu().numpy(), itr.cpu().numpy()


def _check_layout(idx_np, E, R):
    g = _run_layout(idx_np, E, R)
    o = oracle.layout(idx_np, E, R)
    np.testing.assert_array_equal(g[0], o[0])
    np.testing.assert_array_equal(g[1], o[1])
    np.testing.assert_array_equal(g[2], o[2])


def _check_rows_on_device(recv_x, x_dev, dst_np):
    """recv_x[dst[t,k]] == x[t] bit for bit for every selected slot (chunked)."""
    T, K = dst_np.shape
    sel_t, sel_k = np.nonzero(dst_np >= 0)
    rows = dst_np[sel_t, sel_k]
    step = 1 << 16
    for i in range(0, len(rows), step):
        r = torch.from_numpy(rows[i:i + step].astype(np.int64)).to(DEV)
        t = torch.from_numpy(sel_t[i:i + step].astype(np.int64)).to(DEV)
        a = recv_x.view(torch.int16).index_select(0, r)
        b = x_dev.view(torch.int16).index_select(0, t)
        assert torch.equal(a, b), f"row mismatch in slots {i}..{i + step}"


def _dispatch_and_check(w, idx_np, x_np, align=1, cap=None):
    x_dev = dev_bf16(x_np)
    idx_dev = dev_i64(idx_np)
    recv_x, _, h = cgd.dispatch(x_dev, idx_dev, w.E, w.R, expert_alignment=align, recv_capacity=cap)
    torch.cuda.synchronize()
    want_rows = x_np.size * w.K <= FULL_ORACLE_ROWS
    o = oracle.dispatch(x_np if want_rows else None, idx_np, w.E, w.R, align=align, cap=h.recv_capacity,
                        hidden=w.H, with_rows=want_rows)
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), o["expert_offset"])
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    if want_rows:
        g = host_bits(recv_x)
        data = o["recv_src_idx"] >= 0  # padding rows are unspecified
        np.testing.assert_array_equal(g[data], o["recv_x"][data])
    else:
        _check_rows_on_device(recv_x, x_dev, o["dst_row"])
    return x_dev, recv_x, h, o


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_parity(name):
    w = synth.WORKLOADS[name]
    say(f"[parity] {name}: T={w.T} H={w.H} K={w.K} E={w.E} R={w.R} routing={w.routing}")
    inp = synth.make_inputs(w, seed=0)
    _check_layout(inp["topk_idx"], w.E, w.R)
    say(f"[parity] {name}: layout ok")
    x_dev, recv_x, h, o = _dispatch_and_check(w, inp["topk_idx"], inp["x"])
    say(f"[parity] {name}: dispatch ok")

    # identity experts + softmax weights: combine(dispatch(x)) == x exactly
    wt_dev = dev_f32(inp["topk_weights"])
    back = cgd.combine(recv_x, h, wt_dev)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), x_dev.view(torch.int16))
    say(f"[parity] {name}: identity round trip ok")

    # independent expert outputs: the oracle on every token, in chunks of
    # tokens that keep the host arrays small at the largest sizes
    cap = h.recv_capacity
    y_np = synth.make_expert_out(w, cap, seed=0)
    out = cgd.combine(dev_bf16(y_np), h, wt_dev)
    torch.cuda.synchronize()
    got = host_bits(out)
    dst = o["dst_row"]
    chunk = max(1, 50_000_000 // (w.H * w.K))
    same = 0.0
    for t0 in range(0, w.T, chunk):
        tok = np.arange(t0, min(w.T, t0 + chunk))
        exp = oracle.combine(y_np, dst[tok], inp["topk_weights"][tok])
        same += len(tok) * check_combine(got[tok], exp, term_magnitude(y_np, dst[tok], inp["topk_weights"][tok]))
    frac = same / w.T
    say(f"[parity] {name}: combine ok on all {w.T} tokens, bit-identical fraction {frac:.6f}")
    assert frac > 0.99


@pytest.mark.parametrize("T", [1000, 2500])
def test_cached_dispatch_matches_fresh_dispatch(T):
    w = synth.WORKLOADS["prefill"].replace(T=T)
    inp = synth.make_inputs(w, seed=3)
    x_dev, recv_x, h, o = _dispatch_and_check(w, inp["topk_idx"], inp["x"])
    x2 = synth.make_x(w.replace(name="prefill-second-batch"), seed=3)
    recv2, _, h2 = cgd.dispatch(dev_bf16(x2), handle=h)
    torch.cuda.synchronize()
    assert h2 is h
    o2 = oracle.dispatch(x2, inp["topk_idx"], w.E, w.R)
    g = host_bits(recv2)
    data = o2["recv_src_idx"] >= 0
    np.testing.assert_array_equal(g[data], o2["recv_x"][data])


@pytest.mark.parametrize("T", [1500, 2100])
def test_plan_then_apply_equals_dispatch(T):
    w = synth.WORKLOADS["prefill"].replace(T=T, H=1024)
    inp = synth.make_inputs(w.replace(name="prefill"), seed=9)
    idx, x_np = inp["topk_idx"][:w.T], synth.make_x(w, seed=9)
    plan = cgd.dispatch_plan(dev_i64(idx), w.E, w.R, expert_alignment=4)
    recv_x, _, h = cgd.dispatch_apply(dev_bf16(x_np), plan)
    torch.cuda.synchronize()
    o = oracle.dispatch(x_np, idx, w.E, w.R, align=4)
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), o["expert_offset"])
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    data = o["recv_src_idx"] >= 0
    np.testing.assert_array_equal(host_bits(recv_x)[data], o["recv_x"][data])


@pytest.mark.parametrize("T,K,cap_extra", [(0, 4, 40), (1, 8, 0), (256, 8, 300), (200, 8, 40000), (257, 8, 0),
                                         (1500, 8, 0), (2100, 8, 5000), (1100, 16, 0), (8192, 4, 0),
                                         (8193, 2, 700)])
def test_plan_alone_writes_the_handle(T, K, cap_extra):
    """The plan needs only the routing and writes the whole handle: one
    launch for one tile, per-tile ranks then final rows for more (the apply
    afterwards is the broadcast kernel below 16384 slots or at top-k 16, the
    row copy above; one tile with many spare rows is planned by several
    blocks). Spare capacity must come back as -1 rows."""
    E, R, align = 64, 8, 4
    rng = np.random.default_rng(T + K)
    idx = np.array([rng.permutation(E)[:K] for _ in range(T)], dtype=np.int64).reshape(T, K)
    idx[rng.random((T, K)) < 0.05] = -1
    cap = cgd.dispatch_capacity(T, K, E, align) + cap_extra
    say(f"[plan alone] T={T} K={K} cap={cap}")
    plan = cgd.dispatch_plan(dev_i64(idx), E, R, expert_alignment=align, recv_capacity=cap)
    torch.cuda.synchronize()
    o = oracle.dispatch(None, idx, E, R, align=align, with_rows=False)
    h = plan.handle
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), o["expert_offset"])
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    src = h.recv_src_idx.cpu().numpy()
    n = len(o["recv_src_idx"])
    np.testing.assert_array_equal(src[:n], o["recv_src_idx"])
    assert (src[n:] == -1).all()
    if T:
        x = synth.make_x(synth.WORKLOADS["tiny"].replace(T=T, H=64), seed=T)
        recv_x, _, _ = cgd.dispatch_apply(dev_bf16(x), plan)
        torch.cuda.synchronize()
        data = np.nonzero(src >= 0)[0]
        np.testing.assert_array_equal(host_bits(recv_x)[data], x.view(np.uint16)[src[data]])


def _edge(T, K, E, R, H, align=1, p_neg=0.0, dup=False, seed=0, all_to=None, cap_extra=0):
    rng = np.random.default_rng(seed)
    if all_to is not None:
        idx = np.full((T, K), -1, np.int64)
        idx[:, 0] = all_to
    elif dup:
        idx = rng.integers(0, E, size=(T, K)).astype(np.int64)
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64) if T else \
            np.zeros((0, K), np.int64)
    if p_neg:
        idx[rng.random((T, K)) < p_neg] = -1
    w = synth.Workload("edge", T=T, H=H, K=K, E=E, R=R, align=align)
    x = synth.normal_bf16(synth.stream_key(seed, 99, 1), T * H).reshape(T, H)
    wts = synth.softmax_weights(synth.stream_key(seed, 99, 3), T, K)
    return w, idx, x, wts


EDGE_CASES = {
    "T=1": dict(T=1, K=8, E=256, R=8, H=7168),
    "ragged_T=300": dict(T=300, K=8, E=256, R=8, H=512),
    "ragged_T=1025_neg": dict(T=1025, K=6, E=96, R=12, H=136, p_neg=0.3),
    "all_minus_one_rows": dict(T=257, K=4, E=16, R=4, H=64, p_neg=0.9),
    "duplicates": dict(T=513, K=8, E=8, R=2, H=64, dup=True),
    "K=1": dict(T=777, K=1, E=32, R=4, H=8),
    "K=16_E=512_R=64": dict(T=700, K=16, E=512, R=64, H=256),
    "R=1": dict(T=300, K=4, E=64, R=1, H=64),
    "R=E=384": dict(T=600, K=9, E=384, R=384, H=64),
    "R=E=8": dict(T=90, K=3, E=8, R=8, H=64),
    "E=1": dict(T=100, K=1, E=1, R=1, H=32),
    "H=8": dict(T=513, K=2, E=4, R=2, H=8),
    "align16": dict(T=1000, K=8, E=256, R=8, H=64, align=16),
    "align32_neg": dict(T=333, K=4, E=64, R=16, H=24, align=32, p_neg=0.2),
    # one tile with 32256 alignment-padding rows: the plan spreads the -1 fill
    # over several blocks, each planning the tile
    "one_tile_align64": dict(T=100, K=4, E=512, R=8, H=16, align=64),
    "one_hot_expert": dict(T=2000, K=3, E=64, R=8, H=32, all_to=37),
    "extra_capacity": dict(T=200, K=4, E=32, R=4, H=40, cap_extra=1000),
    # batches of >= 16384 slots with top-k <= 8 get final rows from the plan
    # and take the row-copy apply; the others the single broadcast launch:
    # both sides of the switch
    "rowcopy_boundary_T=2048": dict(T=2048, K=8, E=32, R=4, H=64, cap_extra=5000),
    "bcast_boundary_T=2047": dict(T=2047, K=8, E=32, R=4, H=64),
    "rowcopy_ragged_H=1032_align4_neg": dict(T=2049, K=8, E=256, R=8, H=1032, align=4, p_neg=0.1),
    "rowcopy_K=5_duplicates": dict(T=4000, K=5, E=64, R=8, H=200, dup=True),
    "rowcopy_K=1_H=8": dict(T=16385, K=1, E=16, R=4, H=8),
    "rowcopy_one_hot_expert": dict(T=3000, K=6, E=64, R=8, H=72, all_to=5),
    # batches of at most 256 tokens plan and copy in one launch (every block
    # plans the whole batch)
    "fused_duplicates_T=200": dict(T=200, K=8, E=8, R=2, H=64, dup=True),
    "fused_align8_neg_T=250": dict(T=250, K=6, E=64, R=8, H=1032, align=8, p_neg=0.2),
    "fused_T=256_K=16_R=64": dict(T=256, K=16, E=512, R=64, H=520),
    "fused_extra_capacity_T=100": dict(T=100, K=4, E=32, R=4, H=40, cap_extra=300),
}


@pytest.mark.parametrize("case", list(EDGE_CASES))
def test_edge_case_parity(case):
    spec = dict(EDGE_CASES[case])
    cap_extra = spec.pop("cap_extra", 0)
    w, idx, x, wts = _edge(**spec)
    say(f"[edge] {case}")
    _check_layout(idx, w.E, w.R)
    cap = oracle.capacity(w.T, w.K, w.E, w.align) + cap_extra
    x_dev, recv_x, h, o = _dispatch_and_check(w, idx, x, align=w.align, cap=cap)
    y = synth.normal_bf16(synth.stream_key(7, 99, 5), cap * w.H).reshape(cap, w.H)
    out = cgd.combine(dev_bf16(y), h, dev_f32(wts))
    torch.cuda.synchronize()
    exp = oracle.combine(y, o["dst_row"], wts)
    frac = check_combine(host_bits(out), exp, term_magnitude(y, o["dst_row"], wts))
    assert frac > 0.99
    # tokens with no selected slot combine to +0
    empty = (idx < 0).all(axis=1)
    assert (host_bits(out)[empty] == 0).all()


def test_zero_tokens():
    w, idx, x, wts = _edge(T=0, K=4, E=16, R=4, H=64)
    ntpr, ntpe, itr = _run_layout(idx, w.E, w.R)
    assert ntpr.tolist() == [0] * 4 and ntpe.tolist() == [0] * 16 and itr.shape == (0, 4)
    recv_x, _, h = cgd.dispatch(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV),
                             torch.empty((0, 4), dtype=torch.int64, device=DEV), 16, 4, expert_alignment=4)
    out = cgd.combine(recv_x, h, torch.empty((0, 4), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert h.expert_offset.cpu().tolist() == [0] * 17
    assert (h.recv_src_idx.cpu().numpy() == -1).all() and h.recv_capacity == 16 * 3
    assert out.shape == (0, 64)


def test_one_workspace_serves_many_sizes():
    # the self-resetting workspace must be left zeroed by every call
    for T in (1000, 3, 4096, 257, 1):
        w, idx, x, wts = _edge(T=T, K=8, E=256, R=8, H=64, seed=T)
        _check_layout(idx, w.E, w.R)
        _dispatch_and_check(w, idx, x)


def _digest(*ts):
    h = hashlib.sha256()
    for t in ts:
        h.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def test_determinism_20_repeats():
    w = synth.WORKLOADS["prefill"]
    inp = synth.make_inputs(w, seed=5)
    x, idx, wt = dev_bf16(inp["x"]), dev_i64(inp["topk_idx"]), dev_f32(inp["topk_weights"])
    ref = None
    for i in range(20):
        ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx, w.E, w.R)
        recv_x, _, h = cgd.dispatch(x, idx, w.E, w.R)
        out = cgd.combine(recv_x, h, wt)
        torch.cuda.synchronize()
        d = _digest(ntpr, ntpe, itr, h.expert_offset, h.dst_row, h.recv_src_idx, recv_x, out)
        if ref is None:
            ref = d
        assert d == ref, f"repeat {i} differs"


def test_seeds_sweep_prefill_and_skewed():
    for name in ("prefill", "skewed"):
        w = synth.WORKLOADS[name]
        for seed in (1, 2, 3, 4):
            idx = synth.make_topk_idx(w, seed)
            _check_layout(idx, w.E, w.R)
            idx_dev = dev_i64(idx)
            x_small = torch.zeros((w.T, 8), dtype=torch.bfloat16, device=DEV)
            _, _, h = cgd.dispatch(x_small, idx_dev, w.E, w.R)
            torch.cuda.synchronize()
            o = oracle.dispatch(None, idx, w.E, w.R, with_rows=False)
            np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
            np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), o["expert_offset"])


@pytest.mark.parametrize("case", ["tiny", "prefill", "decode", "skewed", "stress", "R=E=384", "duplicates",
                                  "ragged_T=1025_neg", "R=1", "K=16_E=512_R=64", "one_tile_align64"])
def test_layout_and_plan_in_one_launch(case):
    """The fused launch gives the layout kernel's outputs and the plan that
    dispatch_apply completes into the same permutation, bit for bit."""
    if case in synth.WORKLOADS:
        w = synth.WORKLOADS[case]
        idx, x = synth.make_topk_idx(w, 0), None
        align = w.align
    else:
        spec = dict(EDGE_CASES[case])
        spec.pop("cap_extra", None)
        w, idx, x, _ = _edge(**spec)
        align = w.align
    say(f"[fused] {case}")
    (ntpr, _, ntpe, itr, _), plan = cgd.layout_and_dispatch_plan(dev_i64(idx), w.E, w.R, expert_alignment=align)
    xs = torch.zeros((w.T, 8), dtype=torch.bfloat16, device=DEV) if x is None else dev_bf16(x[:, :8].copy())
    _, _, h = cgd.dispatch_apply(xs, plan)
    torch.cuda.synchronize()
    o = oracle.layout(idx, w.E, w.R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), o[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), o[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), o[2])
    d = oracle.dispatch(None, idx, w.E, w.R, align=align, with_rows=False)
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), d["expert_offset"])
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), d["dst_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), d["recv_src_idx"])


@pytest.mark.parametrize("T,K,E,R,align,p_neg", [(1, 8, 256, 16, 1, 0.0), (128, 8, 256, 16, 1, 0.1),
                                                  (256, 4, 384, 384, 4, 0.2), (200, 16, 512, 64, 1, 0.0),
                                                  (100, 3, 8, 2, 16, 0.3), (257, 8, 64, 8, 1, 0.0),
                                                  (2100, 8, 256, 8, 1, 0.05)])
def test_layout_and_dispatch_in_one_call(T, K, E, R, align, p_neg):
    """get_dispatch_layout and dispatch in one call (one launch up to 256
    tokens, else the plan and the row copy): layout outputs, handle and rows
    equal the oracle's, bit for bit."""
    rng = np.random.default_rng(7 * T + K)
    idx = np.array([rng.permutation(E)[:K] for _ in range(T)], dtype=np.int64).reshape(T, K)
    idx[rng.random((T, K)) < p_neg] = -1
    x = synth.make_x(synth.WORKLOADS["tiny"].replace(T=T, H=72), seed=T)
    say(f"[layout and dispatch] T={T} K={K} E={E} R={R} align={align}")
    (ntpr, _, ntpe, itr, _), recv_x, _, h = cgd.layout_and_dispatch(dev_bf16(x), dev_i64(idx), E, R,
                                                                 expert_alignment=align)
    torch.cuda.synchronize()
    o = oracle.layout(idx, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), o[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), o[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), o[2])
    d = oracle.dispatch(x, idx, E, R, align=align)
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), d["expert_offset"])
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), d["dst_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), d["recv_src_idx"])
    data = d["recv_src_idx"] >= 0
    np.testing.assert_array_equal(host_bits(recv_x)[data], d["recv_x"][data])


def test_launches_split_over_token_ranges():
    """Batches larger than one grid (work-item ids are 32-bit: 2^25 waves per
    launch) are issued over token ranges. At hidden 8 and top-1 a token is
    one wave of the row copy, the combine, the rank-granular scatter and its
    combine, so 2^25 + 4099 tokens take two launches of each. Positions must
    match the oracle, every received row its token's row, and both combines
    of identity experts must return x."""
    T, K, E, R, H = (1 << 25) + 4099, 1, 16, 4, 8
    say(f"[parity] split launches: T={T} K={K} H={H}")
    idx = synth.topk_uniform(synth.stream_key(5, 123, 2), T, K, E)
    x = synth.normal_bf16(synth.stream_key(5, 123, 1), T * H).reshape(T, H)
    x_dev = dev_bf16(x)
    idx_dev = dev_i64(idx)
    recv_x, _, h = cgd.dispatch(x_dev, idx_dev, E, R)
    torch.cuda.synchronize()
    o = oracle.dispatch(None, idx, E, R, with_rows=False)
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), o["expert_offset"])
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    rows = torch.from_numpy(o["dst_row"].reshape(-1).astype(np.int64)).to(DEV)
    assert torch.equal(recv_x.view(torch.int64).view(-1, 2).index_select(0, rows), x_dev.view(torch.int64).view(T, 2))
    del rows
    ones = torch.ones((T, K), dtype=torch.float32, device=DEV)
    assert torch.equal(cgd.combine(recv_x, h, ones).view(torch.int16), x_dev.view(torch.int16))
    del recv_x, h
    say("[parity] split launches: expert path ok")
    ntpr, _, ntpe, itr, _ = cgd.get_dispatch_layout(idx_dev, E, R)
    nrecv, _, _, _, nh = cgd.normal_dispatch(x_dev, itr, ntpe, num_experts=E, num_topk=K)
    torch.cuda.synchronize()
    on = oracle.dispatch_normal(None, itr.cpu().numpy(), E, K)
    np.testing.assert_array_equal(nh.send_row.cpu().numpy(), on["send_row"])
    np.testing.assert_array_equal(nh.recv_src_idx.cpu().numpy(), on["recv_src_idx"])
    back, _ = cgd.normal_combine(nrecv, nh)
    torch.cuda.synchronize()
    assert torch.equal(back.view(torch.int16), x_dev.view(torch.int16))
    say("[parity] split launches: rank-granular path ok")


@pytest.mark.parametrize("nbytes", [16, 1 << 20 | 16, 64 << 20])
def test_copy_is_bitwise(nbytes):
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device=DEV)
    dst = torch.zeros_like(src)
    cgd.copy_(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
