#!/usr/bin/env python3
"""Benchmark of the MoE layout / dispatch / combine hot path on one MI355X.

One step = get_dispatch_layout -> dispatch -> combine over one batch of the
workload (default: prefill, 4096 tokens, hidden 7168, top-8 of 256 experts,
8 logical ranks), with identity experts (combine reads the dispatched rows)
and softmax routing weights. Inputs come from the seeded generator and are
resident in HBM before timing starts.

Inputs rotate: --sets distinct seeded (x, topk_idx, topk_weights) sets
(seeds seed..seed+sets-1; 295 MB at prefill, more than the 256 MB Infinity
Cache), step k running set k mod sets, so each step's x was last touched
several steps earlier and is read from HBM. The headline is the wall time of
--steps such steps replayed from HIP graphs, each graph holding whole
rotations of the sets and at least 10 consecutive steps (the serving
setting, where one captured model step holds every layer's calls; --timing
eager times Python launches instead). The same figures with one x reused
every step (which stays in the Infinity Cache) are reported as warm_x, and
with the caches swept by a read-only pass before every step as cold_cache.

Per-call durations (kernel_us, and the whole dispatch / combine / apply
figures derived from them) are device times: 20 back-to-back calls of one
kind captured in a HIP graph (sets rotating), 20 replays each between two HIP
events recorded on the stream the kernels run on, i.e. 400 launches per
figure; every time, GB/s and fraction of peak is a median over the replays.
dispatch_* time the whole dispatch of the step, plan and rows (the expert and
rank-granular paths fuse the layout into the plan, so it is counted there
too); dispatch_apply_* time the row movement alone, i.e. the cached dispatch
that reuses a handle. The same split from HIP events around each call of
--kernel-samples eager steps is kept under "eager" (it carries each event's
own few µs and, for small batches, the host's launch cost); the cold_cache
leg is timed that way, since its sweep runs between steps. layout_us
(get_dispatch_layout alone) and launch_floor_us (libcgd's empty kernel) are
per-call device times as above.

Prints one JSON line with the whole-step token throughput, those figures, the
roofline entry of the dominant data kernel and the CPU oracle's throughput on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD public specification
METRIC = "dispatch+combine HBM GB/s & tokens/s; layout µs at 4096 tok, top-8/256 exp"
FLUSH_BYTES = 512 << 20  # read-only sweep that evicts the 256 MB Infinity Cache
FP8_FORMATS = {"f32": 0, "pow2": 1, "ue8m0": 2}


# ---------------------------------------------------------------------------
# Algorithmic bytes: each tensor counted once (x read once).
# ---------------------------------------------------------------------------

def algorithmic_bytes(w, N: int) -> dict:
    """dispatch: x read, rows written, dst_row and recv_src_idx written; its
    apply (the row copy after the plan) reads x and dst_row and writes the
    rows; combine reads the rows, dst_row and weights and writes the output."""
    T, H, K, E, R = w.T, w.H, w.K, w.E, w.R
    return {
        "layout": T * K * 8 + T * R + (E + R) * 4,
        "dispatch": T * H * 2 + N * H * 2 + T * K * 4 + N * 4,
        "apply": T * H * 2 + N * H * 2 + T * K * 4,
        "combine": N * H * 2 + 2 * T * K * 4 + T * H * 2,
    }


def fp8_row_bytes(w, fmt: int) -> int:
    """Bytes of one FP8 row: H codes plus H/128 scales (4 bytes, 1 for UE8M0)."""
    return w.H + (w.H // 128) * (1 if fmt == 2 else 4)


def algorithmic_bytes_fp8(w, N: int, fmt: int) -> dict:
    """Expert path with the cast on dispatch: bf16 x read once, FP8 rows written."""
    T, H, K = w.T, w.H, w.K
    b = algorithmic_bytes(w, N)
    b["dispatch"] = T * H * 2 + N * fp8_row_bytes(w, fmt) + T * K * 4 + N * 4
    b["apply"] = T * H * 2 + N * fp8_row_bytes(w, fmt) + T * K * 4
    return b


def algorithmic_bytes_normal(w, N: int, fmt: int | None = None) -> dict:
    """Rank-granular calls (N = rows sent), each tensor once."""
    T, H, K, E, R = w.T, w.H, w.K, w.E, w.R
    b = {
        "layout": T * K * 8 + T * R + (E + R) * 4,
        # x, is_token_in_rank, topk_idx/weights in; rows, send_row, recv_src_idx,
        # recv_topk_idx/weights out
        "dispatch": T * H * 2 + T * R + T * K * 12 + N * H * 2 + T * R * 4 + N * (4 + K * 12),
        # rows, send_row, recv_topk_weights in; combined_x, combined_topk_weights out
        "combine": N * H * 2 + T * R * 4 + N * K * 4 + T * H * 2 + T * K * 4,
    }
    if fmt is not None:
        # codes + scales instead of bf16 rows; the cast reads x and writes the tuple
        rb = fp8_row_bytes(w, fmt)
        b["cast"] = T * H * 2 + T * rb
        b["dispatch"] += T * (rb - 2 * H) + N * (rb - 2 * H)
    b["apply"] = b["dispatch"]
    return b


# ---------------------------------------------------------------------------
# The three paths. Each holds --sets input sets on the device and shared
# outputs; step(i, ev) runs one step on set i, recording ev[j] before call j
# and ev[-1] after the last call.
# ---------------------------------------------------------------------------

class _Path:
    labels: tuple = ()           # one per call of a step
    dispatch_labels: tuple = ()  # the calls that make up the whole dispatch
    split_labels: tuple = ()     # calls of split_step, the same work as separate calls (if any)
    apply_label: str | None = None  # the row movement alone, a label of the split (or plain) step
    data_kernels: tuple = ()     # (label, bytes key, traffic kernels) of the data-moving calls

    def __init__(self, w, sets, dev, fmt):
        import numpy as np
        import torch
        self.w, self.dev, self.fmt = w, dev, fmt
        self.inp = sets
        self.idx = [torch.from_numpy(s["topk_idx"]).to(dev) for s in sets]
        self.x = [torch.from_numpy(s["x"].view(np.int16)).view(torch.bfloat16).to(dev) for s in sets]
        self.wt = [torch.from_numpy(s["topk_weights"]).to(dev) for s in sets]
        self.out = torch.empty((w.T, w.H), dtype=torch.bfloat16, device=dev)
        self.rows = [0] * len(sets)

    @staticmethod
    def _rec(ev, j):
        if ev and ev[j] is not None:
            ev[j].record()

    @property
    def dispatch_span(self) -> tuple:
        """Event indices around the whole dispatch (its calls are consecutive)."""
        a = self.labels.index(self.dispatch_labels[0])
        return a, a + len(self.dispatch_labels)

    def nbytes(self, i: int) -> dict:
        raise NotImplementedError

    def graph_calls(self) -> dict:
        """label -> fn(i), one call each (on set i) for graph_call_us: the
        whole dispatch ("dispatch"), the combine ("combine") and the calls of
        the split step. Runs after check(), whose handles they reuse."""
        raise NotImplementedError


class ExpertPath(_Path):
    """bf16: layout and dispatch in one call (layout_and_dispatch: the layout,
    the plan and the rows; one launch for a batch of at most one 256-token
    tile, such as decode), then combine. The split step makes the same calls
    separately: layout + plan (layout_and_dispatch_plan), the row movement
    alone (dispatch_apply, i.e. the cached dispatch), combine. FP8: the same
    with the cast on dispatch (layout_and_dispatch with cast_fp8)."""

    def __init__(self, w, sets, dev, fmt):
        import torch
        import combine_get_dispatch_06_amd as cgd
        super().__init__(w, sets, dev, fmt)
        self.cgd = cgd
        cap = cgd.dispatch_capacity(w.T, w.K, w.E, w.align)
        self.recv_x = torch.empty((cap, w.H), dtype=torch.bfloat16, device=dev)
        if fmt is not None:
            # FP8 rows land in recv_q; the identity expert's bf16 output (the
            # cast-back rows, made outside the timed steps) is recv_x
            self.recv_q = (torch.empty((cap, w.H), dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn),
                           torch.empty((cap, w.H // 128), dtype=torch.uint8 if fmt == 2 else torch.float32,
                                       device=dev))
        self.one_launch = w.T <= 256  # plan (cast) and rows in one launch
        self.split_labels = ("layout_and_plan", "dispatch_apply", "combine")
        self.labels = ("dispatch", "combine")
        self.dispatch_labels = ("dispatch",)
        self.apply_label = "dispatch_apply"
        # roofline candidates: the longest single kernel (the one-launch
        # dispatch of a decode batch, else the row movement alone) or combine
        self.data_kernels = ((("dispatch", "dispatch", ("rank_kernel",)) if self.one_launch else
                              ("dispatch_apply", "apply", APPLY_KERNELS)),
                             ("combine", "combine", ("combine_kernel",)))
        self.handles = [None] * len(sets)

    def step(self, i, ev=None):
        cgd, w = self.cgd, self.w
        self._rec(ev, 0)
        _, _, _, h = self._dispatch(i)
        self._rec(ev, 1)
        cgd.combine(self.recv_x, h, self.wt[i], out=self.out)
        self._rec(ev, 2)
        self.handles[i] = h

    def split_step(self, i, ev=None):
        cgd, w = self.cgd, self.w
        self._rec(ev, 0)
        _, plan = cgd.layout_and_dispatch_plan(self.idx[i], w.E, w.R, expert_alignment=w.align)
        self._rec(ev, 1)
        if self.fmt is None:
            _, _, h = cgd.dispatch_apply(self.x[i], plan, recv_x=self.recv_x)
        else:
            _, _, h = cgd.dispatch_apply(self.x[i], plan, recv_x=self.recv_q, cast_fp8=self.fmt)
        self._rec(ev, 2)
        cgd.combine(self.recv_x, h, self.wt[i], out=self.out)
        self._rec(ev, 3)
        self.handles[i] = h

    def _dispatch(self, i):
        cgd, w = self.cgd, self.w
        if self.fmt is None:
            return cgd.layout_and_dispatch(self.x[i], self.idx[i], w.E, w.R, expert_alignment=w.align,
                                           recv_x=self.recv_x)
        return cgd.layout_and_dispatch(self.x[i], self.idx[i], w.E, w.R, expert_alignment=w.align,
                                       recv_x=self.recv_q, cast_fp8=self.fmt)

    def _apply(self, i):
        # the cached dispatch: the handle's rows alone (dispatch_apply's kernels)
        if self.fmt is None:
            return self.cgd.dispatch(self.x[i], handle=self.handles[i], recv_x=self.recv_x)
        return self.cgd.dispatch(self.x[i], handle=self.handles[i], recv_x=self.recv_q, cast_fp8=self.fmt)

    def graph_calls(self):
        cgd, w = self.cgd, self.w
        return {"dispatch": self._dispatch,
                "layout_and_plan": lambda i: cgd.layout_and_dispatch_plan(self.idx[i], w.E, w.R,
                                                                          expert_alignment=w.align),
                "dispatch_apply": self._apply,
                "combine": lambda i: cgd.combine(self.recv_x, self.handles[i], self.wt[i], out=self.out)}

    def check(self, i):
        """combine(dispatch(x)) returns x: exactly for bf16, within the FP8
        rounding for FP8 payloads (the cast-back rows of this set's dispatch)."""
        import torch
        self.step(i)
        if self.fmt is not None:
            self.cgd.per_token_cast_back(self.recv_q, self.fmt, out=self.recv_x)
            self.step(i)
        torch.cuda.synchronize()
        x = self.x[i]
        if self.fmt is None:
            assert torch.equal(self.out.view(torch.int16), x.view(torch.int16)), f"round trip failed (set {i})"
        else:
            rel = ((self.out.float() - x.float()).norm() / x.float().norm()).item()
            assert rel < 0.05, f"FP8 round trip error {rel} (set {i})"
        self.rows[i] = int(self.handles[i].expert_offset[-1].item())

    def nbytes(self, i):
        n = self.rows[i]
        return algorithmic_bytes(self.w, n) if self.fmt is None else algorithmic_bytes_fp8(self.w, n, self.fmt)

    def describe(self):
        return {"dispatch": (("layout_and_dispatch (one launch: layout + plan + rows)" if self.fmt is None else
                              "layout_and_dispatch with the cast (one launch: layout + plan + cast rows)")
                             if self.one_launch else
                             "layout_and_dispatch (layout + plan with x pulled toward the caches, then the rows)"
                             if self.fmt is None else
                             "layout_and_dispatch with the cast (layout + plan with x pulled toward the caches, "
                             "then the cast on dispatch)"),
                "split": "layout_and_dispatch_plan, then dispatch_apply (the cached dispatch: rows alone)",
                "experts": "identity (combine reads dispatched rows)" if self.fmt is None else
                "identity (combine reads the cast-back FP8 rows, made before timing)"}


class NormalPath(_Path):
    """layout, rank-granular plan and apply in one call
    (layout_and_normal_dispatch: the plan pulls x toward the caches for the
    apply, or with the FP8 payload casts x in its idle blocks), combine
    (identity experts, no bias); the split step makes the same calls
    separately (layout + plan in one launch, [the per-token cast,] the
    apply)."""
    labels = ("dispatch", "combine")
    dispatch_labels = ("dispatch",)
    apply_label = "dispatch_apply"
    data_kernels = (("dispatch_apply", "apply", ("normal_scatter_kernel",)),
                    ("combine", "combine", ("normal_combine_kernel",)))

    def __init__(self, w, sets, dev, fmt):
        import torch
        import combine_get_dispatch_06_amd as cgd
        super().__init__(w, sets, dev, fmt)
        self.cgd = cgd
        cap = cgd.normal_capacity(w.T, w.K, w.R)
        self.recv_x = torch.empty((cap, w.H), dtype=torch.bfloat16, device=dev)
        if fmt is not None:
            self.recv_q = (torch.empty((cap, w.H), dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn),
                           torch.empty((cap, w.H // 128), dtype=torch.uint8 if fmt == 2 else torch.float32,
                                       device=dev))
        self.last = [None] * len(sets)
        self.split_labels = (("layout_and_plan", "dispatch_apply", "combine") if fmt is None else
                             ("layout_and_plan", "cast", "dispatch_apply", "combine"))

    def step(self, i, ev=None):
        cgd = self.cgd
        self._rec(ev, 0)
        (_, _, _, itr, _), _, _, rw, _, h = self._dispatch(i)
        self._rec(ev, 1)
        cgd.normal_combine(self.recv_x, h, rw, out=self.out)
        self._rec(ev, 2)
        self.last[i] = (h, itr, rw)

    def split_step(self, i, ev=None):
        """The step's work as separate calls (layout + plan, [cast,] apply, combine)."""
        cgd, w = self.cgd, self.w
        self._rec(ev, 0)
        (_, _, _, itr, _), plan = cgd.layout_and_normal_dispatch_plan(self.idx[i], w.E, w.R,
                                                                      expert_alignment=w.align)
        self._rec(ev, 1)
        n = 2
        if self.fmt is None:
            x, recv = self.x[i], self.recv_x
        else:
            x, recv = cgd.per_token_cast_to_fp8(self.x[i], self.fmt), self.recv_q
            self._rec(ev, n)
            n += 1
        _, _, rw, _, h = cgd.normal_dispatch_apply(x, plan, self.idx[i], self.wt[i], recv_x=recv)
        self._rec(ev, n)
        cgd.normal_combine(self.recv_x, h, rw, out=self.out)
        self._rec(ev, n + 1)
        self.last[i] = (h, itr, rw)

    def _dispatch(self, i):
        cgd, w = self.cgd, self.w
        if self.fmt is None:
            return cgd.layout_and_normal_dispatch(self.x[i], self.idx[i], self.wt[i], w.E, w.R,
                                                  expert_alignment=w.align, recv_x=self.recv_x)
        return cgd.layout_and_normal_dispatch(self.x[i], self.idx[i], self.wt[i], w.E, w.R,
                                              expert_alignment=w.align, recv_x=self.recv_q, cast_fp8=self.fmt)

    def graph_calls(self):
        import torch
        cgd, w = self.cgd, self.w
        # the apply alone needs a plan per set that no later plan overwrites:
        # each set's plan gets a workspace of its own (made once, here)
        nws = cgd.layout_and_normal_workspace_bytes(w.T, w.K, w.E, w.R)
        plans, xs = {}, {}
        for i in range(len(self.x)):
            ws = torch.zeros(nws, dtype=torch.uint8, device=self.dev)
            plans[i] = cgd.layout_and_normal_dispatch_plan(self.idx[i], w.E, w.R, expert_alignment=w.align,
                                                           workspace=ws)[1]
            xs[i] = self.x[i] if self.fmt is None else cgd.per_token_cast_to_fp8(self.x[i], self.fmt)
        recv = self.recv_x if self.fmt is None else self.recv_q
        calls = {"dispatch": self._dispatch,
                 "layout_and_plan": lambda i: cgd.layout_and_normal_dispatch_plan(self.idx[i], w.E, w.R,
                                                                                  expert_alignment=w.align),
                 "dispatch_apply": lambda i: cgd.normal_dispatch_apply(xs[i], plans[i], self.idx[i], self.wt[i],
                                                                       recv_x=recv),
                 "combine": lambda i: cgd.normal_combine(self.recv_x, self.last[i][0], self.last[i][2],
                                                         out=self.out)}
        if self.fmt is not None:
            calls["cast"] = lambda i: cgd.per_token_cast_to_fp8(self.x[i], self.fmt)
        return calls

    def check(self, i):
        """each token comes back as bf16(x * ranks it was sent to): exactly for
        bf16, within the FP8 rounding for FP8 payloads."""
        import torch
        self.step(i)
        if self.fmt is not None:
            self.cgd.per_token_cast_back(self.recv_q, self.fmt, out=self.recv_x)
            self.step(i)
        torch.cuda.synchronize()
        h, itr, _ = self.last[i]
        n = itr.sum(dim=1, dtype=torch.float32).unsqueeze(1)
        want = (self.x[i].float() * n).to(torch.bfloat16)
        if self.fmt is None:
            assert torch.equal(self.out.view(torch.int16), want.view(torch.int16)), f"round trip failed (set {i})"
        else:
            rel = ((self.out.float() - want.float()).norm() / want.float().norm()).item()
            assert rel < 0.05, f"FP8 round trip error {rel} (set {i})"
        self.rows[i] = int(h.rank_offset[-1].item())

    def nbytes(self, i):
        return algorithmic_bytes_normal(self.w, self.rows[i], self.fmt)

    def describe(self):
        return {"path": "normal (one row per flagged rank)",
                "dispatch": (("layout_and_normal_dispatch (layout, rank-granular plan and rows in one launch)"
                              if self.w.T <= 256 else
                              "layout_and_normal_dispatch (layout + rank-granular plan with x pulled toward the "
                              "caches, then the apply)") if self.fmt is None else
                             ("layout_and_normal_dispatch with the cast (layout, rank-granular plan, cast and rows "
                              "in one launch)" if self.w.T <= 256 else
                              "layout_and_normal_dispatch with the cast (layout + rank-granular plan whose idle "
                              "blocks cast x, then the apply of the FP8 tuple)")),
                "experts": "identity (combine reads dispatched rows), no bias" if self.fmt is None else
                "identity (combine reads the cast-back FP8 rows, made before timing), no bias"}


class PackedPath(_Path):
    """layout and packed (fixed-capacity) dispatch in one call
    (layout_and_low_latency_dispatch; one launch up to 256 tokens), combine
    over the packed rows."""
    labels = ("dispatch", "combine")
    dispatch_labels = ("dispatch",)
    # the packed dispatch is the plan and the apply: its traffic is their sum
    data_kernels = (("dispatch", "dispatch", ("rank_kernel", "finalize_kernel", "scatter_kernel",
                                              "scatter_bcast_kernel", "scatter_cast_kernel")),
                    ("combine", "combine", ("combine_kernel",)))

    def __init__(self, w, sets, dev, fmt):
        import numpy as np
        import torch
        import combine_get_dispatch_06_amd as cgd
        super().__init__(w, sets, dev, fmt)
        self.cgd = cgd
        # capacity: the largest per-expert count of any set rounded up to 64
        # (no slot dropped), fixed before timing like any low-latency buffer
        most = max(int(np.bincount(s["topk_idx"][s["topk_idx"] >= 0], minlength=w.E).max()) for s in sets)
        self.cap = -(-most // 64) * 64
        self.recv = torch.empty((w.E, self.cap, w.H), dtype=torch.bfloat16, device=dev)
        if fmt is not None:
            self.recv_q = (torch.empty((w.E * self.cap, w.H), dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn),
                           torch.empty((w.E * self.cap, w.H // 128), dtype=torch.uint8 if fmt == 2 else torch.float32,
                                       device=dev))
        self.count = [None] * len(sets)
        self.handles = [None] * len(sets)

    def _dispatch(self, i):
        cgd, w = self.cgd, self.w
        if self.fmt is None:
            return cgd.layout_and_low_latency_dispatch(self.x[i], self.idx[i], w.E, w.R, expert_capacity=self.cap,
                                                       out=self.recv)
        return cgd.layout_and_low_latency_dispatch(self.x[i], self.idx[i], w.E, w.R, expert_capacity=self.cap,
                                                   use_fp8=True, scale_format=self.fmt, out=self.recv_q)

    def step(self, i, ev=None):
        cgd, w = self.cgd, self.w
        self._rec(ev, 0)
        _, _, count, h = self._dispatch(i)
        self._rec(ev, 1)
        cgd.low_latency_combine(self.recv, self.wt[i], h, out=self.out)
        self._rec(ev, 2)
        self.count[i] = count
        self.handles[i] = h

    def graph_calls(self):
        cgd, w = self.cgd, self.w
        return {"layout": lambda i: cgd.get_dispatch_layout(self.idx[i], w.E, w.R), "dispatch": self._dispatch,
                "combine": lambda i: cgd.low_latency_combine(self.recv, self.wt[i], self.handles[i], out=self.out)}

    def check(self, i):
        import torch
        self.step(i)
        if self.fmt is not None:
            self.cgd.per_token_cast_back(self.recv_q, self.fmt, out=self.recv.view(-1, self.w.H))
            self.step(i)
        torch.cuda.synchronize()
        x = self.x[i]
        if self.fmt is None:
            assert torch.equal(self.out.view(torch.int16), x.view(torch.int16)), f"round trip failed (set {i})"
        else:
            rel = ((self.out.float() - x.float()).norm() / x.float().norm()).item()
            assert rel < 0.05, f"FP8 round trip error {rel} (set {i})"
        self.rows[i] = int(self.count[i].sum().item())

    def nbytes(self, i):
        n = self.rows[i]
        return algorithmic_bytes(self.w, n) if self.fmt is None else algorithmic_bytes_fp8(self.w, n, self.fmt)

    def describe(self):
        return {"path": f"packed (fixed capacity {self.cap} rows per expert)",
                "dispatch": "layout_and_low_latency_dispatch (layout, plan and rows; one launch up to 256 tokens)",
                "experts": "identity (combine reads the packed rows)"}


# ---------------------------------------------------------------------------
# Timing
# ---------------------------------------------------------------------------

def stats(a) -> dict:
    import numpy as np
    a = np.asarray(a, dtype=np.float64)
    return {"median": float(np.median(a)), "min": float(np.min(a)), "max": float(np.max(a))}


def kernel_samples(path, order, flush=None):
    """Two eager loops of one step per entry of `order` (set indices),
    optionally after a cache sweep outside the events. The first records
    events around every call (the per-call split); the second only around the
    whole dispatch and the combine, since each recorded event adds a few µs
    of its own to the interval it closes.
    -> {label: per-sample µs, "dispatch", "combine", "step"}, set index per sample."""
    import numpy as np
    import torch
    split = getattr(path, "split_step", None) if path.split_labels else None
    labels = path.split_labels if split else path.labels
    ns = len(labels) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(ns)] for _ in order]
    for ev, i in zip(evs, order):
        if flush is not None:
            flush()
        (split or path.step)(i, ev)
    n = len(path.labels) + 1
    a, b = path.dispatch_span
    keep = {a, b, n - 2, n - 1}
    whole = [[torch.cuda.Event(enable_timing=True) if j in keep else None for j in range(n)] for _ in order]
    for ev, i in zip(whole, order):
        if flush is not None:
            flush()
        path.step(i, ev)
    torch.cuda.synchronize()
    us = {lab: np.array([e[j].elapsed_time(e[j + 1]) * 1e3 for e in evs]) for j, lab in enumerate(labels)}
    us["step"] = np.array([e[0].elapsed_time(e[-1]) * 1e3 for e in evs])
    us["dispatch"] = np.array([e[a].elapsed_time(e[b]) * 1e3 for e in whole])
    us["combine"] = np.array([e[n - 2].elapsed_time(e[n - 1]) * 1e3 for e in whole])
    return us, np.asarray(order)


def summarize(path, us, sets_of_sample) -> dict:
    """Medians over samples: per-call µs, whole-dispatch µs, GB/s and
    fractions of the HBM peak (bytes of each sample's own input set)."""
    import numpy as np
    nb = [path.nbytes(int(i)) for i in sets_of_sample]
    disp = us["dispatch"]  # events only around the whole dispatch
    comb = us["combine"]

    def rate(key, t):
        return np.array([b[key] for b in nb]) / (t * 1e-6) / 1e9

    out = {"kernel_us": {lab: stats(us[lab]) for lab in (path.split_labels or path.labels)},
           "step_us": stats(us["step"]),
           "dispatch_us": float(np.median(disp)), "combine_us": float(np.median(comb))}
    out["kernel_us"]["combine"] = stats(comb)  # the whole-dispatch loop's figure (one event fewer)
    d, c = rate("dispatch", disp), rate("combine", comb)
    out.update(dispatch_GBps=float(np.median(d)), dispatch_frac_of_peak=float(np.median(d)) / HBM_PEAK_GBPS,
               combine_GBps=float(np.median(c)), combine_frac_of_peak=float(np.median(c)) / HBM_PEAK_GBPS,
               dispatch_tokens_per_s=float(np.median(path.w.T / (disp * 1e-6))),
               combine_tokens_per_s=float(np.median(path.w.T / (comb * 1e-6))))
    if path.apply_label:
        a = rate("apply", us[path.apply_label])
        out.update(dispatch_apply_us=float(np.median(us[path.apply_label])), dispatch_apply_GBps=float(np.median(a)),
                   dispatch_apply_frac_of_peak=float(np.median(a)) / HBM_PEAK_GBPS)
    if "layout_and_plan" in us:
        out["layout_and_plan_us"] = float(np.median(us["layout_and_plan"]))
    if "dispatch" in out["kernel_us"]:
        out["kernel_us"]["dispatch"] = stats(disp)
    return out


STEPS_PER_GRAPH = 10  # at least this many consecutive steps per captured graph


def _capture(fn, seq, s):
    """fn(i) for each i of seq, captured in one HIP graph on stream s."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in seq:
            fn(i)
    return g


def graph_wall(path, order, steps: int, warmup: int) -> float:
    """Wall seconds of `steps` steps, step k on set order[k mod len(order)],
    replayed from HIP graphs that each hold a whole number of rotations of
    `order` and at least STEPS_PER_GRAPH steps (a captured model step holds
    every layer's calls likewise, so one replay's launch cost is shared by
    many calls), plus one graph for the remainder. Captured on a side stream
    after untimed steps on it, so every workspace exists before capture."""
    import torch
    L = len(order)
    per = L * -(-STEPS_PER_GRAPH // L)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            for i in sorted(set(order)):
                path.step(i)
    s.synchronize()
    full = _capture(path.step, [order[k % L] for k in range(per)], s)
    rem = steps % per
    tail = _capture(path.step, [order[k % L] for k in range(rem)], s) if rem else None
    for _ in range(-(-warmup // per)):
        full.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps // per):
        full.replay()
    if tail is not None:
        tail.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def eager_wall(path, order, steps: int) -> float:
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        path.step(order[k % len(order)])
    torch.cuda.synchronize()
    return time.perf_counter() - t0


def timed_wall(args, path, order):
    """Wall seconds of args.steps steps and how they were launched."""
    if args.timing == "graph":
        try:
            return graph_wall(path, order, args.steps, args.warmup), \
                f"HIP graph replays, >= {STEPS_PER_GRAPH} steps per graph"
        except Exception as exc:  # capture unsupported here: time eager launches
            print(f"graph capture failed ({exc}); timing eager launches", file=sys.stderr)
    return eager_wall(path, order, args.steps), "eager launches"


GRAPH_CALLS = 20    # back-to-back calls per captured graph
GRAPH_REPLAYS = 20  # timed replays: GRAPH_CALLS * GRAPH_REPLAYS launches per figure


def graph_call_us(fn, order=(0,), calls: int = GRAPH_CALLS, replays: int = GRAPH_REPLAYS) -> dict:
    """Device time per call of fn(i), i cycling through `order`: `calls`
    back-to-back calls captured in one HIP graph on a side stream (after
    untimed calls there, so every workspace exists before capture), replayed
    `replays` times, each replay between two HIP events recorded on that
    stream; a replay's interval / calls is one sample. Eager event pairs
    around a small call time the host's Python launch cost instead (the GPU
    finishes such a call before the next is submitted), and each recorded
    event adds a few µs of its own."""
    import numpy as np
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    seq = [order[k % len(order)] for k in range(calls)]
    with torch.cuda.stream(s):
        for _ in range(2):
            for i in sorted(set(seq)):
                fn(i)
    s.synchronize()
    g = _capture(fn, seq, s)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    with torch.cuda.stream(s):
        g.replay()
        for e0, e1 in ev:
            e0.record(s)
            g.replay()
            e1.record(s)
    torch.cuda.synchronize()
    per = np.array([e0.elapsed_time(e1) * 1e3 / calls for e0, e1 in ev])
    return {**stats(per), "launches": calls * replays}


def graph_summary(path, order, calls: int = GRAPH_CALLS, replays: int = GRAPH_REPLAYS) -> dict:
    """Per-call device times of the path's calls (graph_call_us, sets cycling
    through `order`), the whole dispatch and the combine with their GB/s and
    fractions of the HBM peak (bytes averaged over the sets of `order`)."""
    import numpy as np
    per = {lab: graph_call_us(fn, order, calls, replays) for lab, fn in path.graph_calls().items()}
    nb = [path.nbytes(int(i)) for i in order]

    def rate(key, t):
        return float(np.mean([b[key] for b in nb])) / (t * 1e-6) / 1e9

    disp, comb = per["dispatch"]["median"], per["combine"]["median"]
    out = {"kernel_us": per, "dispatch_us": disp, "combine_us": comb,
           "dispatch_GBps": rate("dispatch", disp), "combine_GBps": rate("combine", comb),
           "dispatch_tokens_per_s": path.w.T / (disp * 1e-6), "combine_tokens_per_s": path.w.T / (comb * 1e-6)}
    out["dispatch_frac_of_peak"] = out["dispatch_GBps"] / HBM_PEAK_GBPS
    out["combine_frac_of_peak"] = out["combine_GBps"] / HBM_PEAK_GBPS
    if path.apply_label:
        a = per[path.apply_label]["median"]
        out.update(dispatch_apply_us=a, dispatch_apply_GBps=rate("apply", a),
                   dispatch_apply_frac_of_peak=rate("apply", a) / HBM_PEAK_GBPS)
    if "layout_and_plan" in per:
        out["layout_and_plan_us"] = per["layout_and_plan"]["median"]
    return out


def copy_ceilings(dev) -> dict:
    """Device-to-device copy rate of 1 GiB (read + write bytes per second), by
    torch and by libcgd's own 16-byte copy (cgd_copy), event-timed medians."""
    import numpy as np
    import torch
    import combine_get_dispatch_06_amd as cgd
    a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)

    def timed(fn, n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for _ in range(3):
            fn()
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return np.array([e0.elapsed_time(e1) for e0, e1 in ev]) * 1e3

    copy = timed(lambda: b.copy_(a), 5)
    own = timed(lambda: cgd.copy_(b, a), 5)
    del a, b
    return {"copy_1GiB_GBps": float(2 * (1 << 30) / (np.median(copy) * 1e-6) / 1e9),
            "cgd_copy_1GiB_GBps": float(2 * (1 << 30) / (np.median(own) * 1e-6) / 1e9)}


def input_digests(inp: dict) -> dict:
    import hashlib
    return {k: hashlib.sha256(v.tobytes()).hexdigest()[:16] for k, v in inp.items()}


def cpu_baseline(w, inp, budget_s: float) -> dict:
    """The CPU oracle, as it is, on whole steps of the same workload until the
    time budget is used (at least one step)."""
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.layout(inp["topk_idx"], w.E, w.R)
        d = oracle.dispatch(inp["x"], inp["topk_idx"], w.E, w.R)
        oracle.combine(d["recv_x"], d["dst_row"], inp["topk_weights"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": w.T * reps / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} whole steps (layout+dispatch+combine) of the {w.name} workload (seed 0), "
                      f"single-threaded C oracle, {el:.1f} s on {cpu_model()} ({os.cpu_count()} cpus visible)"}


def _oracle_slice_worker(args) -> tuple:
    """One process of the parallel CPU baseline: whole oracle steps over its
    token slice until the budget is used -> (tokens processed, seconds)."""
    name, seed, lo, hi, budget_s = args
    import oracle
    import synth
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w, seed=seed)
    idx, x, wt = inp["topk_idx"][lo:hi], inp["x"][lo:hi], inp["topk_weights"][lo:hi]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.layout(idx, w.E, w.R)
        d = oracle.dispatch(x, idx, w.E, w.R)
        oracle.combine(d["recv_x"], d["dst_row"], wt)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return reps * (hi - lo), el


def cpu_baseline_parallel(w, seed: int, cores: int, budget_s: float) -> dict:
    """The same oracle steps with the batch's tokens split into `cores`
    contiguous slices, one process each (the per-core token split of the
    layout operator's multi-core strategy): the sum of the slices' token
    rates. Each slice is planned on its own (its own segment offsets), so
    this is a throughput figure of the same work, not one dispatch."""
    import multiprocessing as mp
    bounds = [(w.T * i // cores, w.T * (i + 1) // cores) for i in range(cores)]
    with mp.get_context("spawn").Pool(cores) as pool:
        res = pool.map(_oracle_slice_worker, [(w.name, seed, lo, hi, budget_s) for lo, hi in bounds])
    sizes = sorted({hi - lo for lo, hi in bounds})
    return {"value": sum(tok / el for tok, el in res), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{cores} processes, each whole oracle steps (layout+dispatch+combine) over a contiguous "
                      f"slice of {'-'.join(map(str, sizes))} tokens of the {w.name} workload (seed {seed}) "
                      f"for {budget_s:.0f} s, on {cpu_model()}"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def roofline(path, summary, traffic_json, tkey) -> dict:
    """The dominant data kernel (longest median) with its achieved GB/s
    (median over samples of algorithmic bytes / duration) against the peak."""
    cands = {lab: (summary["dispatch_us"] if lab == "dispatch" else summary["kernel_us"][lab]["median"])
             for lab, _, _ in path.data_kernels}
    dom = max(cands, key=cands.get)
    lab, key, kernels = next(d for d in path.data_kernels if d[0] == dom)
    if dom == path.apply_label:
        achieved = summary["dispatch_apply_GBps"]
    elif dom == "combine":
        achieved = summary["combine_GBps"]
    else:
        achieved = summary["dispatch_GBps"]
    traffic = lookup_traffic_sum(traffic_json, tkey, kernels)
    return {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic, "duration_us": cands[dom]}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sets", type=int, default=5,
                    help="distinct seeded input sets rotated every step (seeds seed..seed+sets-1)")
    ap.add_argument("--kernel-samples", type=int, default=200,
                    help="eager steps whose calls are event-timed for the per-kernel medians (>= 200)")
    ap.add_argument("--path", choices=("expert", "normal", "packed"), default="expert",
                    help="expert: one received row per selected expert (default); normal: one per flagged rank; "
                         "packed: fixed-capacity per-expert buffers (the low-latency layout)")
    ap.add_argument("--timing", choices=("graph", "eager"), default="graph",
                    help="graph (default): time replays of steps captured once per input set in HIP graphs; "
                         "eager: time the Python launches")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="extra event-timed steps, each after a read-only sweep of 512 MiB (evicts the 256 MB "
                         "Infinity Cache without leaving dirty lines); 0 skips them")
    ap.add_argument("--graph-calls", type=int, default=GRAPH_CALLS,
                    help="back-to-back calls per captured graph for the per-call device times")
    ap.add_argument("--graph-replays", type=int, default=GRAPH_REPLAYS,
                    help="timed replays of each per-call graph (calls x replays launches per figure)")
    ap.add_argument("--skip-warm", action="store_true",
                    help="skip the warm_x leg (one x every step), e.g. so that a profiler's per-kernel averages "
                         "cover the rotated-input launches alone")
    ap.add_argument("--fp8", choices=tuple(FP8_FORMATS), default=None,
                    help="FP8 (e4m3fn) dispatch payload with this scale format: the expert path casts on "
                         "dispatch, the normal path casts first and dispatches the (codes, scales) tuple")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=10.0, help="0 skips the CPU baseline")
    ap.add_argument("--cpu-baseline-cores", type=int, default=0,
                    help="also time the oracle over this many token slices in parallel processes "
                         "(cpu_baseline_parallel); 0 skips it")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM traffic per launch (from rocprofv3 counters), if present")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write --traffic-json from rocprofv3 --pmc counter_collection.csv files and exit")
    args = ap.parse_args()

    if args.traffic_from:
        return write_traffic(args)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(this path has no inter-GPU transport)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import combine_get_dispatch_06_amd as cgd
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.ones(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 5}), flush=True)
        return 0

    w = synth.WORKLOADS[args.workload]
    fmt = FP8_FORMATS[args.fp8] if args.fp8 else None
    nsets = max(1, args.sets)
    sets = [synth.make_inputs(w, seed=args.seed + i) for i in range(nsets)]
    path = {"expert": ExpertPath, "normal": NormalPath, "packed": PackedPath}[args.path](w, sets, dev, fmt)
    rotation = list(range(nsets))
    set_bytes = sum(v.nbytes for s in sets for v in s.values())

    # first call timed on its own (cf. the first-call latency discussed on the
    # pages), after cgd.init has loaded libcgd's GPU code (timed too)
    torch.cuda.synchronize()
    t = time.perf_counter()
    cgd.init(dev)
    init_ms = (time.perf_counter() - t) * 1e3
    t = time.perf_counter()
    path.step(0)
    torch.cuda.synchronize()
    first_ms = (time.perf_counter() - t) * 1e3
    for i in rotation:  # every set must round-trip (identity experts)
        path.check(i)
    for k in range(args.warmup):
        path.step(rotation[k % nsets])
    torch.cuda.synchronize()

    samples = max(args.kernel_samples, 1)
    us, which = kernel_samples(path, [rotation[k % nsets] for k in range(samples)])
    eager = summarize(path, us, which)
    gc, gr = max(1, args.graph_calls), max(1, args.graph_replays)
    rotated = graph_summary(path, rotation, gc, gr)
    wall, timing = timed_wall(args, path, rotation)

    warm = None
    if not args.skip_warm:
        us0, which0 = kernel_samples(path, [0] * samples)
        warm = graph_summary(path, [0], gc, gr)
        warm["eager"] = summarize(path, us0, which0)
        wall0, _ = timed_wall(args, path, [0])
        warm.update(ms_per_step=wall0 / args.steps * 1e3, tokens_per_s=w.T * args.steps / wall0)
        warm["how"] = "one input set (seed %d) every step: x stays in the Infinity Cache" % args.seed

    cold = None
    if args.cold_steps > 0:
        sweep = torch.empty(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)
        sink = torch.empty((), dtype=torch.int64, device=dev)

        def flush():
            torch.sum(sweep, dim=0, dtype=torch.int64, out=sink)  # reads 512 MiB, writes 8 bytes

        usc, whichc = kernel_samples(path, [rotation[k % nsets] for k in range(args.cold_steps)], flush=flush)
        cold = summarize(path, usc, whichc)
        cold["flush"] = "read-only sweep of 512 MiB (a reduction) before every step, outside the events"
        del sweep

    layout_alone = graph_call_us(lambda i: cgd.get_dispatch_layout(path.idx[i], w.E, w.R), rotation, gc, gr)
    floor = graph_call_us(lambda i: cgd.empty_(dev), (0,), gc, gr)
    ctx = copy_ceilings(dev)
    tkey = w.name + ("" if args.path == "expert" else ":" + args.path) + (f":fp8-{args.fp8}" if fmt is not None else "")
    roof = roofline(path, rotated, args.traffic_json, tkey)
    roof.update(copy_ceiling=ctx["cgd_copy_1GiB_GBps"], frac_of_copy_ceiling=roof["achieved"] / ctx["cgd_copy_1GiB_GBps"])

    dtype = "bf16" if fmt is None else "fp8_e4m3 dispatch / bf16 combine"
    res = {
        "metric": METRIC,
        "value": w.T * args.steps / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded generator: uniform distinct top-k or Zipf(1.2), N(0,1) bf16 x, softmax weights)",
        "config": {"workload": w.name, "num_tokens": w.T, "hidden": w.H, "num_topk": w.K, "num_experts": w.E,
                   "num_ranks": w.R, "expert_alignment": w.align, "routing": w.routing,
                   "inputs": f"{nsets} seeded sets (seeds {args.seed}..{args.seed + nsets - 1}, "
                             f"{set_bytes / 1e6:.0f} MB) rotated every step",
                   **path.describe(), **({} if fmt is None else {"fp8_scales": args.fp8}),
                   "rows_sent": path.rows, "timing": timing},
        "layout_us": layout_alone,
        "launch_floor_us": floor,
        **{k: v for k, v in rotated.items() if k != "kernel_us"},
        "kernel_us": rotated["kernel_us"],
        "kernel_us_how": f"device time per call: {gc} back-to-back calls per HIP graph, "
                         f"{gr} replays between HIP events on the launch stream, sets rotating",
        "eager": {**eager, "how": f"HIP events around each call of {samples} eager steps, sets rotating "
                                  "(host-bound for small batches)"},
        "kernel_samples": samples,
        "init_ms": init_ms,
        "first_step_ms": first_ms,
        "warm_x": warm,
        "cold_cache": cold,
        **ctx,
        "inputs_sha256": input_digests(sets[0]),
        "bytes_per_call": path.nbytes(0),
        "roofline": roof,
    }
    if args.cpu_baseline_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(w, sets[0], args.cpu_baseline_seconds)
        if args.cpu_baseline_cores > 1:
            res["cpu_baseline_parallel"] = cpu_baseline_parallel(w, args.seed, args.cpu_baseline_cores,
                                                                 args.cpu_baseline_seconds)
    print(json.dumps(res), flush=True)
    return 0


# ---------------------------------------------------------------------------
# Measured traffic (rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
# ---------------------------------------------------------------------------

APPLY_KERNELS = ("scatter_kernel", "scatter_bcast_kernel", "scatter_cast_kernel")
PLAN_KERNELS = ("rank_kernel", "finalize_kernel")


def lookup_traffic(path: str, key: str, kernel: str):
    """Measured HBM bytes per launch of `kernel` for workload `key`, if the
    table was taken from the current kernel sources."""
    if not os.path.exists(path):
        return None
    try:
        entry = json.load(open(path)).get(key, {}).get(kernel)
        if entry and entry.get("source_hash") == kernel_source_hash():
            return entry["bytes_per_launch"]
    except Exception:
        return None
    return None


def lookup_traffic_sum(path: str, key: str, kernels) -> float | None:
    """Measured bytes of a unit of several launches: the sum over the listed
    kernels present in the table for `key` (the ones that ran when the
    counters were taken); None unless all of them are current."""
    if not os.path.exists(path):
        return None
    try:
        entries = json.load(open(path)).get(key, {})
    except Exception:
        return None
    present = [k for k in kernels if k in entries]
    vals = [lookup_traffic(path, key, k) for k in present]
    if not present or None in vals:
        return None
    return float(sum(vals))


def _counter_per_kernel(path: str, counter: str) -> dict:
    """Average per-dispatch value of `counter` for each kernel name in a
    rocprofv3 counter_collection.csv (values summed over a dispatch's rows)."""
    import csv
    per = {}
    for r in csv.DictReader(open(path)):
        if r.get("Counter_Name") != counter:
            continue
        key = (r["Kernel_Name"], r["Dispatch_Id"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return {name: sum(v) / len(v) for name, v in out.items()}


def write_traffic(args) -> int:
    """HBM bytes per launch of the dominant kernels from FETCH_SIZE/WRITE_SIZE
    (KiB per dispatch), each scaled by bytes / counter of a plain copy."""
    fetch = _counter_per_kernel(args.traffic_from[0], "FETCH_SIZE")
    write = _counter_per_kernel(args.traffic_from[1], "WRITE_SIZE")
    cfetch = _counter_per_kernel(args.traffic_from[2], "FETCH_SIZE")
    cwrite = _counter_per_kernel(args.traffic_from[3], "WRITE_SIZE")
    copy_bytes = args.copy_calibration << 20 if args.copy_calibration else 512 << 20
    copy_f = max(cfetch.values())
    copy_w = max(cwrite.values())
    f_scale = copy_bytes / copy_f
    w_scale = copy_bytes / copy_w
    entry = {}
    if args.path == "normal":
        shorts = ("normal_scatter_kernel", "normal_combine_kernel", "normal_plan_kernel", "layout_kernel",
                  "cast_to_fp8_kernel")
    else:
        shorts = APPLY_KERNELS + PLAN_KERNELS + ("combine_kernel", "layout_acc_kernel")
    for short in shorts:
        fk = [k for k in fetch if "cgd::" + short in k]
        wk = [k for k in write if "cgd::" + short in k]
        if fk and wk:
            fb, wb = fetch[fk[0]] * f_scale, write[wk[0]] * w_scale
            entry[short] = {"bytes_per_launch": fb + wb, "fetch_bytes": fb, "write_bytes": wb,
                            "fetch_kib_raw": fetch[fk[0]], "write_kib_raw": write[wk[0]],
                            "source_hash": kernel_source_hash()}
    data = {}
    if os.path.exists(args.traffic_json):
        data = json.load(open(args.traffic_json))
    data[args.workload + ("" if args.path == "expert" else ":" + args.path)
         + (f":fp8-{args.fp8}" if args.fp8 else "")] = entry
    data["calibration"] = {"copy_bytes": copy_bytes, "copy_fetch_kib": copy_f, "copy_write_kib": copy_w,
                           "fetch_bytes_per_unit": f_scale, "write_bytes_per_unit": w_scale}
    json.dump(data, open(args.traffic_json, "w"), indent=1)
    print(json.dumps(data), flush=True)
    return 0


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and layout whitespace
    removed: measured traffic stays attached to the code it was taken on
    (any change to the code, not to its comments, invalidates it)."""
    import hashlib
    import re
    hsh = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_get_dispatch_06_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, f), encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)  # block comments
        text = re.sub(r"//[^\n]*", " ", text)               # line comments (no "//" inside strings here)
        hsh.update(f.encode() + b"\0" + " ".join(text.split()).encode())
    return hsh.hexdigest()[:16]


if __name__ == "__main__":
    sys.exit(main())
