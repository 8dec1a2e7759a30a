"""Parity of the FP8 payload HIP path with the CPU oracle.

The per-token cast (codes and scales, every scale format, row- and
column-major scales) and the cast back must be bit-exact: both sides decide
each code in fp32 with the same operations. FP8 dispatch (pre-cast tuple,
cast on the way, cached, rank-granular) must put exactly the oracle's codes
and scales in exactly the oracle's rows."""
import numpy as np
import pytest
import torch

import combine_get_dispatch_06_amd as cgd
import oracle
import synth
from gpu_util import DEV, bf16_to_f64, dev_bf16, dev_f32, dev_i64, host_bits, say

pytestmark = pytest.mark.gpu

FMTS = [cgd.SCALE_F32, cgd.SCALE_POW2, cgd.SCALE_UE8M0]


def _x(T, H, seed, spread=True):
    """N(0,1) bf16 rows, each 128-block scaled by 10^U(-3,3), with an all-zero
    block, a subnormal and a huge value planted."""
    w = synth.Workload("fp8", T=T, H=H, K=1, E=1, R=1)
    x = synth.make_x(w, seed=seed).astype(np.uint16)
    f = (x.astype(np.uint32) << 16).view(np.float32).reshape(T, H // 128, 128)
    if spread:
        rng = np.random.default_rng(seed)
        f = f * (10.0 ** rng.uniform(-3, 3, (T, H // 128, 1))).astype(np.float32)
    f = f.reshape(T, H).copy()
    if T > 2:
        f[0, :128] = 0.0
        f[1, 3] = 1e-40
        f[2, min(130, H - 1)] = -3e38
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _scales_np(sc: torch.Tensor) -> np.ndarray:
    return sc.cpu().contiguous().numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,H,colmajor", [(1, 128, False), (37, 256, True), (300, 7168, False),
                                          (128, 7168, True), (513, 4096, False)])
def test_cast_parity(fmt, T, H, colmajor):
    x = _x(T, H, seed=T + H)
    q, sc = cgd.per_token_cast_to_fp8(dev_bf16(x), fmt, column_major_scales=colmajor)
    torch.cuda.synchronize()
    if colmajor:
        assert sc.stride() == (1, T)
    oq, osc = oracle.cast_to_fp8(x, fmt)
    np.testing.assert_array_equal(q.view(torch.uint8).cpu().numpy(), oq)
    np.testing.assert_array_equal(_scales_np(sc).view(np.uint8), osc.view(np.uint8))
    back = cgd.per_token_cast_back((q, sc), fmt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(back), oracle.cast_back(oq, osc, fmt))


def test_cast_back_all_codes():
    """Every finite code in every position, with fp32 and UE8M0 scales."""
    T, H = 8, 1024
    rng = np.random.default_rng(0)
    codes = np.tile(np.arange(256, dtype=np.uint8), T * H // 256).reshape(T, H)
    codes[(codes & 0x7F) == 0x7F] = 0x12  # no NaN codes
    rng.shuffle(codes, axis=1)
    sf = (10.0 ** rng.uniform(-6, 6, (T, H // 128))).astype(np.float32)
    su = rng.integers(100, 150, (T, H // 128)).astype(np.uint8)
    q = torch.from_numpy(codes).to(DEV).view(torch.float8_e4m3fn)
    for fmt, s in ((cgd.SCALE_F32, sf), (cgd.SCALE_UE8M0, su)):
        back = cgd.per_token_cast_back((q, torch.from_numpy(s).to(DEV)), fmt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(back), oracle.cast_back(codes, s, fmt))


def _check_rows(recv, q_np, s_np, dst_np):
    """Received code rows and scale rows equal the source token's, for every
    destination row of dst_np ([T, K] or [T, R], -1 = none)."""
    rq, rs = recv
    sel_t, sel_k = np.nonzero(dst_np >= 0)
    rows = dst_np[sel_t, sel_k]
    got_q = rq.view(torch.uint8).cpu().numpy()[rows]
    np.testing.assert_array_equal(got_q, q_np[sel_t])
    np.testing.assert_array_equal(rs.cpu().numpy()[rows].view(np.uint8), s_np[sel_t].view(np.uint8))


@pytest.mark.parametrize("fmt,colmajor", [(cgd.SCALE_F32, False), (cgd.SCALE_F32, True), (cgd.SCALE_UE8M0, False),
                                          (cgd.SCALE_UE8M0, True)])
@pytest.mark.parametrize("T", [700, 2500])
def test_fp8_tuple_dispatch_and_cached(fmt, colmajor, T):
    w = synth.WORKLOADS["prefill"].replace(T=T, H=1024)
    idx = synth.make_topk_idx(w.replace(name="prefill"), seed=2)
    x = _x(w.T, w.H, seed=2)
    q, sc = cgd.per_token_cast_to_fp8(dev_bf16(x), fmt, column_major_scales=colmajor)
    recv, _, h = cgd.dispatch((q, sc), dev_i64(idx), w.E, w.R, expert_alignment=4)
    torch.cuda.synchronize()
    o = oracle.dispatch(None, idx, w.E, w.R, align=4, with_rows=False)
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), o["expert_offset"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    oq, osc = oracle.cast_to_fp8(x, fmt)
    _check_rows(recv, oq, osc, o["dst_row"])
    # cached: a second batch through the same handle
    x2 = _x(w.T, w.H, seed=3)
    q2, sc2 = cgd.per_token_cast_to_fp8(dev_bf16(x2), fmt, column_major_scales=colmajor)
    recv2, _, _ = cgd.dispatch((q2, sc2), handle=h)
    torch.cuda.synchronize()
    oq2, osc2 = oracle.cast_to_fp8(x2, fmt)
    _check_rows(recv2, oq2, osc2, o["dst_row"])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,K,E,R,H,p_neg", [(1, 8, 256, 8, 7168, 0.0), (700, 8, 256, 8, 1024, 0.0),
                                             (333, 4, 64, 16, 384, 0.2), (2000, 16, 512, 64, 256, 0.05),
                                             (64, 1, 8, 2, 128, 0.0), (2100, 8, 64, 8, 384, 0.1),
                                             (3000, 6, 96, 12, 1152, 0.0)])
def test_cast_on_dispatch_parity(fmt, T, K, E, R, H, p_neg):
    rng = np.random.default_rng(T + K)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx[rng.random((T, K)) < p_neg] = -1
    x = _x(T, H, seed=T)
    recv, _, h = cgd.dispatch(dev_bf16(x), dev_i64(idx), E, R, cast_fp8=fmt)
    torch.cuda.synchronize()
    o = oracle.dispatch(None, idx, E, R, with_rows=False)
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    oq, osc = oracle.cast_to_fp8(x, fmt)
    _check_rows(recv, oq, osc, o["dst_row"])


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,K", [(100, 8), (2100, 8), (1100, 16)])
def test_cached_cast_on_dispatch_equals_planned(fmt, T, K):
    """Cast on dispatch to the rows of an existing handle gives the same codes
    and scales as the cast on a fresh dispatch (same kernel, same rows)."""
    E, R, H = 64, 8, 512
    rng = np.random.default_rng(T)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    x = dev_bf16(_x(T, H, seed=T + 1))
    (q1, s1), _, h = cgd.dispatch(x, dev_i64(idx), E, R, cast_fp8=fmt)
    (q2, s2), _, h2 = cgd.dispatch(x, handle=h, cast_fp8=fmt)
    torch.cuda.synchronize()
    assert h2 is h
    data = h.recv_src_idx >= 0
    assert torch.equal(q1.view(torch.uint8)[data], q2.view(torch.uint8)[data])
    assert torch.equal(s1.view(torch.uint8)[data], s2.view(torch.uint8)[data])


def test_cast_on_dispatch_prefill_round_trip():
    """Prefill sizes, cast on dispatch; every received row checked against
    the oracle's codes and scales of its token (all tokens), and the combine
    of the cast-back rows (identity experts) within the FP8 error bound of x."""
    w = synth.WORKLOADS["prefill"]
    inp = synth.make_inputs(w, seed=0)
    x_dev = dev_bf16(inp["x"])
    recv, _, h = cgd.dispatch(x_dev, dev_i64(inp["topk_idx"]), w.E, w.R, cast_fp8=cgd.SCALE_F32)
    torch.cuda.synchronize()
    o = oracle.dispatch(None, inp["topk_idx"], w.E, w.R, with_rows=False)
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    tok = np.arange(w.T)
    oq, osc = oracle.cast_to_fp8(inp["x"], cgd.SCALE_F32)
    rows = o["dst_row"][tok]
    rq = recv[0].view(torch.uint8)
    for k in range(w.K):
        r = torch.from_numpy(rows[:, k].astype(np.int64)).to(DEV)
        np.testing.assert_array_equal(rq.index_select(0, r).cpu().numpy(), oq)
        np.testing.assert_array_equal(recv[1].index_select(0, r).cpu().numpy(), osc)
    back = cgd.per_token_cast_back(recv)
    out = cgd.combine(back, h, dev_f32(inp["topk_weights"]))
    torch.cuda.synchronize()
    xf = bf16_to_f64(inp["x"])
    err = np.abs(bf16_to_f64(host_bits(out)) - xf)
    s_all = osc  # every token's scales
    # half an e4m3 spacing (normal and subnormal range) plus two bf16 roundings
    bound = 2.0 ** -4 * np.abs(xf) * 1.01 + 2.0 ** -10 * np.repeat(s_all.astype(np.float64), 128, axis=1) \
        + 2.0 ** -6 * np.abs(xf) + 1e-30
    assert (err <= bound).all(), f"worst excess {np.max(err - bound)}"
    rel = np.sqrt((err ** 2).sum() / (xf ** 2).sum())
    say(f"[fp8] prefill cast-on-dispatch round trip relative L2 error {rel:.2e}")
    assert rel < 0.05


@pytest.mark.parametrize("fmt", [cgd.SCALE_F32, cgd.SCALE_UE8M0])
def test_fp8_normal_dispatch_and_cached(fmt):
    w = synth.WORKLOADS["prefill"].replace(T=900, H=512)
    idx = synth.make_topk_idx(w.replace(name="prefill"), seed=4)
    wts = synth.make_weights(w.replace(name="prefill"), seed=4)
    x = _x(w.T, w.H, seed=4)
    _, _, ntpe, itr, _ = cgd.get_dispatch_layout(dev_i64(idx), w.E, w.R)
    q, sc = cgd.per_token_cast_to_fp8(dev_bf16(x), fmt, column_major_scales=True)
    recv, ridx, rw, nre, h = cgd.normal_dispatch((q, sc), itr, ntpe, dev_i64(idx), dev_f32(wts), num_experts=w.E)
    torch.cuda.synchronize()
    o = oracle.dispatch_normal(None, itr.cpu().numpy(), w.E, w.K, ntpe.cpu().numpy(), idx, wts)
    np.testing.assert_array_equal(h.send_row.cpu().numpy(), o["send_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    np.testing.assert_array_equal(ridx.cpu().numpy(), o["recv_topk_idx"])
    oq, osc = oracle.cast_to_fp8(x, fmt)
    _check_rows(recv, oq, osc, o["send_row"])
    x2 = _x(w.T, w.H, seed=5)
    q2, sc2 = cgd.per_token_cast_to_fp8(dev_bf16(x2), fmt)
    recv2, _, _, _, _ = cgd.normal_dispatch((q2, sc2), handle=h)
    torch.cuda.synchronize()
    oq2, osc2 = oracle.cast_to_fp8(x2, fmt)
    _check_rows(recv2, oq2, osc2, o["send_row"])


def test_fp8_zero_tokens():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    q, sc = cgd.per_token_cast_to_fp8(x)
    idx = torch.empty((0, 4), dtype=torch.int64, device=DEV)
    recv, _, h = cgd.dispatch(x, idx, 16, 4, expert_alignment=2, cast_fp8=cgd.SCALE_F32)
    recv2, _, _ = cgd.dispatch((q, sc), idx, 16, 4, expert_alignment=2)
    torch.cuda.synchronize()
    assert q.shape == (0, 256) and sc.shape == (0, 2)
    assert recv[0].shape == (16, 256) and recv[1].shape == (16, 2)
    assert (h.recv_src_idx.cpu().numpy() == -1).all()
    assert recv2[0].shape == (16, 256)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T,K,E,R,H,A,extra,p_neg", [(100, 8, 256, 8, 1024, 1, 0, 0.0), (2049, 8, 256, 8, 384, 4, 37, 0.1),
                                                     (1100, 16, 512, 64, 256, 16, 0, 0.0),
                                                     (4096, 8, 256, 8, 7168, 1, 0, 0.0),
                                                     # one tile: plan, cast and rows in one launch
                                                     (200, 9, 384, 384, 128, 1, 5000, 0.05),
                                                     (1, 8, 256, 8, 7168, 1, 0, 0.0)])
def test_layout_and_dispatch_cast_parity(fmt, T, K, E, R, H, A, extra, p_neg):
    """layout_and_dispatch with the cast on the way (one call: the plan pulls x
    into the caches, the cast reads it there; a batch of one tile casts in the
    plan's own launch): layout outputs, handle, aligned
    counts and every received row's codes and scales as the oracle's; rows
    without data keep their sentinel bytes."""
    rng = np.random.default_rng(T + K + A)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    idx[rng.random((T, K)) < p_neg] = -1
    x = _x(T, H, seed=T + A)
    cap = cgd.dispatch_capacity(T, K, E, A) + extra
    rq = torch.full((cap, H), 0xA5, dtype=torch.uint8, device=DEV)
    rs = torch.full((cap, H // 128), 0x5A, dtype=torch.uint8, device=DEV)
    if fmt != cgd.SCALE_UE8M0:
        rs = torch.full((cap, H // 128), -7.0, dtype=torch.float32, device=DEV)
    say(f"[fp8] layout_and_dispatch cast fmt={fmt} T={T} K={K} E={E} R={R} H={H} A={A}")
    lay, recv, nre, h = cgd.layout_and_dispatch(dev_bf16(x), dev_i64(idx), E, R, expert_alignment=A,
                                                recv_capacity=cap, recv_x=(rq, rs), cast_fp8=fmt)
    torch.cuda.synchronize()
    ntpr, _, ntpe, itr, _ = lay
    o_ntpr, o_ntpe, o_itr = oracle.layout(idx, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), o_ntpr)
    np.testing.assert_array_equal(ntpe.cpu().numpy(), o_ntpe)
    np.testing.assert_array_equal(itr.cpu().numpy(), o_itr)
    o = oracle.dispatch(None, idx, E, R, align=A, with_rows=False)
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), o["expert_offset"])
    src = h.recv_src_idx.cpu().numpy()
    np.testing.assert_array_equal(src[:len(o["recv_src_idx"])], o["recv_src_idx"])
    assert (src[len(o["recv_src_idx"]):] == -1).all()
    np.testing.assert_array_equal(nre.cpu().numpy(), np.diff(o["expert_offset"]))
    assert recv[0] is rq and recv[1] is rs
    oq, osc = oracle.cast_to_fp8(x, fmt)
    _check_rows(recv, oq, osc, o["dst_row"])
    empty = torch.from_numpy(np.flatnonzero(src < 0)).to(DEV)
    if empty.numel():
        assert (rq.index_select(0, empty) == 0xA5).all()
        sv = rs.index_select(0, empty)
        assert ((sv == 0x5A) if fmt == cgd.SCALE_UE8M0 else (sv == -7.0)).all()


@pytest.mark.parametrize("fmt,T,K,E,R,H,A,p_neg", [(cgd.SCALE_F32, 4096, 8, 256, 8, 7168, 1, 0.0),
                                                   (cgd.SCALE_UE8M0, 2049, 6, 96, 12, 384, 4, 0.2),
                                                   (cgd.SCALE_POW2, 1500, 16, 512, 64, 256, 8, 0.0),
                                                   (cgd.SCALE_F32, 128, 8, 256, 16, 1024, 1, 0.0),
                                                   (cgd.SCALE_UE8M0, 300, 4, 64, 8, 128, 1, 0.1),
                                                   (cgd.SCALE_F32, 0, 4, 16, 4, 256, 2, 0.0),
                                                   (cgd.SCALE_POW2, 700, 9, 384, 384, 128, 1, 0.05),
                                                   # one tile: layout, plan, cast and rows in one launch
                                                   (cgd.SCALE_UE8M0, 200, 9, 384, 384, 128, 1, 0.05),
                                                   (cgd.SCALE_POW2, 1, 8, 256, 16, 7168, 1, 0.0),
                                                   (cgd.SCALE_F32, 256, 8, 256, 8, 7168, 1, 0.0),
                                                   (cgd.SCALE_F32, 100, 6, 90, 6, 384, 4, 0.2)])
def test_layout_and_normal_dispatch_cast_parity(fmt, T, K, E, R, H, A, p_neg):
    """Rank-granular layout + dispatch with the cast done by the plan's idle
    blocks (in the one launch of a one-tile batch): the cast tuple equals the
    oracle's per-token cast, the layout and handle the oracle's, and every
    received row holds its token's codes and scales."""
    rng = np.random.default_rng(T + 3 * K)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64) if T else np.zeros((0, K), np.int64)
    idx[rng.random((T, K)) < p_neg] = -1
    x = _x(T, H, seed=T + 9) if T else np.zeros((0, H), np.uint16)
    wts = synth.softmax_weights(synth.stream_key(T, 57, 3), T, K)
    say(f"[fp8] layout_and_normal_dispatch cast fmt={fmt} T={T} K={K} E={E} R={R} H={H} A={A}")
    lay, recv, ridx, rw, nre, h = cgd.layout_and_normal_dispatch(dev_bf16(x), dev_i64(idx), dev_f32(wts), E, R,
                                                                 expert_alignment=A, cast_fp8=fmt)
    torch.cuda.synchronize()
    ntpr, _, ntpe, itr, _ = lay
    ol = oracle.layout(idx, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])
    o = oracle.dispatch_normal(None, ol[2], E, K, ol[1], idx, wts, align=A, cap=h.recv_capacity)
    np.testing.assert_array_equal(h.rank_offset.cpu().numpy(), o["rank_offset"])
    np.testing.assert_array_equal(nre.cpu().numpy(), o["num_recv_tokens_per_expert"])
    np.testing.assert_array_equal(h.send_row.cpu().numpy(), o["send_row"])
    np.testing.assert_array_equal(h.recv_src_idx.cpu().numpy(), o["recv_src_idx"])
    np.testing.assert_array_equal(ridx.cpu().numpy(), o["recv_topk_idx"])
    np.testing.assert_array_equal(rw.cpu().numpy().view(np.uint32), o["recv_topk_weights"].view(np.uint32))
    if T:
        oq, osc = oracle.cast_to_fp8(x, fmt)
        _check_rows(recv, oq, osc, o["send_row"])
        # the library's standalone cast gives the same tuple the plan's blocks wrote
        q2, s2 = cgd.per_token_cast_to_fp8(dev_bf16(x), fmt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(q2.view(torch.uint8).cpu().numpy(), oq)
        np.testing.assert_array_equal(_scales_np(s2).view(np.uint8), osc.view(np.uint8))


@pytest.mark.parametrize("T,fmt", [(1000, cgd.SCALE_F32), (200, cgd.SCALE_F32), (200, cgd.SCALE_UE8M0)])
def test_layout_and_normal_dispatch_cast_writes_the_callers_tuple(T, fmt):
    """x_fp8 given: the plan's blocks (for one tile, the one launch's moving
    waves) cast into the caller's (codes, scales)."""
    K, E, R, H = 8, 64, 8, 512
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    x = _x(T, H, seed=5)
    q = torch.full((T, H), 0x7E, dtype=torch.uint8, device=DEV)
    sc = (torch.zeros((T, H // 128), dtype=torch.uint8, device=DEV) if fmt == cgd.SCALE_UE8M0 else
          torch.zeros((T, H // 128), dtype=torch.float32, device=DEV))
    say(f"[fp8] layout_and_normal_dispatch cast into the caller's tuple T={T} fmt={fmt}")
    cgd.layout_and_normal_dispatch(dev_bf16(x), dev_i64(idx), None, E, R, cast_fp8=fmt, x_fp8=(q, sc))
    torch.cuda.synchronize()
    oq, osc = oracle.cast_to_fp8(x, fmt)
    np.testing.assert_array_equal(q.cpu().numpy(), oq)
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint8), osc.view(np.uint8))


# Routing edge cases for the cast on dispatch (hidden 128 or 256); up to 256
# tokens the plan, the cast and the rows take one launch.
CAST_EDGE = {
    "T=1": dict(T=1, K=8, E=256, R=8),
    "one_tile_duplicates": dict(T=200, K=8, E=8, R=2, dup=True),
    "duplicates_T=513": dict(T=513, K=8, E=8, R=2, dup=True),
    "one_tile_all_minus_one": dict(T=100, K=4, E=16, R=4, p_neg=0.9),
    "one_tile_R=E=384_K=9": dict(T=200, K=9, E=384, R=384),
    "one_tile_align64_spare_rows": dict(T=100, K=4, E=512, R=8, align=64),
    "one_tile_extra_capacity": dict(T=100, K=4, E=32, R=4, extra=300),
    "one_tile_E=1": dict(T=100, K=1, E=1, R=1),
    "align32_neg_T=333": dict(T=333, K=4, E=64, R=16, align=32, p_neg=0.2),
}


@pytest.mark.parametrize("fmt", [cgd.SCALE_F32, cgd.SCALE_UE8M0])
@pytest.mark.parametrize("case", list(CAST_EDGE))
def test_cast_on_dispatch_edge_cases(case, fmt):
    """layout_and_dispatch with the cast over routing edge cases (repeated
    experts, empty routings, R > 64, alignment padding, spare rows): layout,
    handle and received codes and scales as the oracle's; rows without data
    keep their sentinel bytes."""
    spec = dict(CAST_EDGE[case])
    T, K, E, R = spec["T"], spec["K"], spec["E"], spec["R"]
    A, extra = spec.get("align", 1), spec.get("extra", 0)
    H = 256 if T <= 256 else 128
    rng = np.random.default_rng(T + 13 * K)
    if spec.get("dup"):
        idx = rng.integers(0, E, size=(T, K)).astype(np.int64)
    else:
        idx = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    if spec.get("p_neg"):
        idx[rng.random((T, K)) < spec["p_neg"]] = -1
    x = _x(T, H, seed=T + 17)
    cap = cgd.dispatch_capacity(T, K, E, A) + extra
    rq = torch.full((cap, H), 0xA5, dtype=torch.uint8, device=DEV)
    rs = (torch.full((cap, H // 128), 0x5A, dtype=torch.uint8, device=DEV) if fmt == cgd.SCALE_UE8M0 else
          torch.full((cap, H // 128), -7.0, dtype=torch.float32, device=DEV))
    say(f"[fp8] cast on dispatch edge case {case} fmt={fmt}")
    (ntpr, _, ntpe, itr, _), recv, nre, h = cgd.layout_and_dispatch(dev_bf16(x), dev_i64(idx), E, R,
                                                                    expert_alignment=A, recv_capacity=cap,
                                                                    recv_x=(rq, rs), cast_fp8=fmt)
    torch.cuda.synchronize()
    ol = oracle.layout(idx, E, R)
    np.testing.assert_array_equal(ntpr.cpu().numpy(), ol[0])
    np.testing.assert_array_equal(ntpe.cpu().numpy(), ol[1])
    np.testing.assert_array_equal(itr.cpu().numpy(), ol[2])
    o = oracle.dispatch(None, idx, E, R, align=A, with_rows=False)
    np.testing.assert_array_equal(h.dst_row.cpu().numpy(), o["dst_row"])
    np.testing.assert_array_equal(h.expert_offset.cpu().numpy(), o["expert_offset"])
    src = h.recv_src_idx.cpu().numpy()
    np.testing.assert_array_equal(src[:len(o["recv_src_idx"])], o["recv_src_idx"])
    assert (src[len(o["recv_src_idx"]):] == -1).all()
    np.testing.assert_array_equal(nre.cpu().numpy(), np.diff(o["expert_offset"]))
    oq, osc = oracle.cast_to_fp8(x, fmt)
    _check_rows(recv, oq, osc, o["dst_row"])
    empty = torch.from_numpy(np.flatnonzero(src < 0)).to(DEV)
    if empty.numel():
        assert (rq.index_select(0, empty) == 0xA5).all()
        sv = rs.index_select(0, empty)
        assert ((sv == 0x5A) if fmt == cgd.SCALE_UE8M0 else (sv == -7.0)).all()
