"""Benchmark of the expert-parallel dispatch/combine core on one MI355X.

One step = the whole path on one batch: ep_layout_notify (the layout and notify
stages in one launch), ep_dispatch, ep_combine (identity experts: combine reads
dispatch's receive rows), all on torch's current stream, inputs already resident
in HBM.  The two-launch form of the first stages (ep_get_layout, then ep_notify)
is timed beside it.  The default workload
is the prefill one: 4096 tokens, hidden 7168 bf16, top-8 of 256 experts over 64
emulated ranks (8 nodes x 8), 24 channels, seed 0.

The metric is dispatch+combine HBM throughput: the bytes the method must move
(x read once per token, each receive row written once and read back once,
metadata) over the dispatch+combine time of the timed steps (one HIP event
pair per step around the two calls, averaged).  Each kernel's own average
launch duration -- the roofline figure -- is taken from back-to-back launches
between one event pair, which is what a kernel trace reports for it.
``ms_per_step`` is the wall time of a whole step including layout and notify.
Beside the metric: the cached-mode and fp8-row dispatch forms, the E4M3
quantiser, the quantising dispatch and its cached mode, the dequantiser, the
grouping by expert and the dispatch straight into the grouped layout, a
cold-cache cross-check and the oracle's throughput on the host.  Prints one
JSON line.

    python bench.py [--steps K] [--warmup W] [--workload prefill] [--no-cpu-baseline] [--no-variants]
                    [--no-other-workloads] [--cold-steps N]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E


def dispatch_bytes(T, H, K, R, N) -> int:
    """x read once per token, topk ids (i64) and weights (f32) read, every
    receive row written with its weights (f32), local ids (i64) and src_info
    (2 x i32), and the [t][R] send_slot map written."""
    return T * 2 * H + T * K * 12 + N * (2 * H + 4 * K + 8 * K + 8) + 4 * T * R


def combine_bytes(T, H, K, R, N) -> int:
    """every receive row and its weights read once, the send_slot map read,
    the combined rows (bf16) and weights (f32) written."""
    return N * 2 * H + N * 4 * K + 4 * T * R + T * 2 * H + T * 4 * K


def dispatch_fp8_bytes(T, H, K, R, N, S) -> int:
    """as dispatch_bytes with 1-byte rows and S fp32 scales per row moved beside them."""
    return T * (H + 4 * S) + T * K * 12 + N * (H + 4 * S + 4 * K + 8 * K + 8) + 4 * T * R


def dispatch_to_fp8_bytes(T, H, K, R, N, S) -> int:
    """the quantising dispatch: bf16 x read once per token, ids and weights read, every receive row written
    as E4M3 codes with its S fp32 scales and its metadata, and the [t][R] send_slot map written."""
    return T * 2 * H + T * K * 12 + N * (H + 4 * S + 4 * K + 8 * K + 8) + 4 * T * R


def dispatch_cached_to_fp8_bytes(T, H, R, N, S) -> int:
    """the cached quantising dispatch: bf16 x and the [t][R] send_slot map read once, every receive row
    written as E4M3 codes with its S fp32 scales."""
    return T * 2 * H + 4 * T * R + N * (H + 4 * S)


def dequantize_bytes(N, H, S) -> int:
    """E4M3 rows and their S fp32 scales read once, bf16 rows written."""
    return N * (H + 4 * S) + N * 2 * H


def quantize_bytes(T, H, S) -> int:
    """bf16 rows read once, E4M3 rows (1 byte an element) and S fp32 scales per row written."""
    return T * 2 * H + T * (H + 4 * S)


def dispatch_cached_bytes(T, R, N, row_bytes, S) -> int:
    """rows (and their scales) read once per token, the [t][R] send_slot map
    read, every receive row (and its scales) written."""
    return T * (row_bytes + 4 * S) + 4 * T * R + N * (row_bytes + 4 * S)


def group_bytes(H, K, N, M) -> int:
    """every receive row read once and every grouped row (M = sum of the
    aligned per-expert sizes) written, the receive ids (i64) and weights read,
    the slot->position map, grouped row indices and weights written."""
    return N * 2 * H + M * 2 * H + N * K * (8 + 4 + 4) + M * (4 + 4)


def dispatch_grouped_bytes(T, H, K, R, N, M) -> int:
    """dispatch straight into the grouped layout: x, ids and weights read once,
    the receive metadata and send_slot written, the slot->position map, and
    every grouped row with its index and weight written (no receive rows)."""
    return T * 2 * H + 12 * T * K + 4 * T * R + N * (12 * K + 8) + 4 * N * K + M * (2 * H + 8)


def layout_notify_bytes(T, K, R, E, C) -> int:
    nodes = max(1, R // 8)
    return T * K * 8 + T * R + 4 * (R + nodes + E) + T * R + 4 * (R + nodes + E) + 4 * (R + nodes) * (C + 1) + 4 * E


PROFILE = os.path.join(ROOT, "profiles", "ep_kernels_prefill_hbm_bytes.txt")
KERNEL_SOURCES = {"dispatch_pull_kernel": ["ep_dispatch.hip", "ep_internal.h"],
                  "dispatch_pull_kernel_fp8": ["ep_dispatch.hip", "ep_internal.h"],
                  "dispatch_kernel_cached_bf16": ["ep_dispatch.hip", "ep_internal.h"],
                  "dispatch_kernel_cached_fp8": ["ep_dispatch.hip", "ep_internal.h"],
                  "group_kernels": ["ep_group.hip", "ep_internal.h"],
                  "dispatch_grouped_pull_kernel": ["ep_dispatch.hip", "ep_internal.h"],
                  "quantize_e4m3_kernel": ["ep_quant.hip", "ep_internal.h"],
                  "dispatch_kernel_to_fp8": ["ep_dispatch.hip", "ep_internal.h"],
                  "dequantize_e4m3_kernel": ["ep_quant.hip", "ep_internal.h"],
                  "dispatch_kernel_cached_to_fp8": ["ep_dispatch.hip", "ep_internal.h"],
                  "combine_kernel": ["ep_combine.hip", "ep_internal.h"],
                  "combine_staged_kernel": ["ep_combine.hip", "ep_internal.h"]}


def combine_kernel_name(T, H) -> str:
    """The combine kernel the library launches for these rows: bf16 rows of 14 KiB
    and more from 4096 tokens are written in bursts from LDS."""
    return "combine_staged_kernel" if 2 * H >= 14 * 1024 and T >= 4096 else "combine_kernel"


def source_code_only(text: bytes) -> bytes:
    """A HIP source without its comments and with runs of white space made one
    space: what the counters' validity depends on (a comment edit leaves it)."""
    import re

    s = text.decode()
    s = re.sub(r"/\*.*?\*/", " ", s, flags=re.S)
    s = re.sub(r"//[^\n]*", " ", s)
    return re.sub(r"\s+", " ", s).strip().encode()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by a plain copy of known
    size), or None when that summary does not cover this workload or the
    kernel's sources (comments aside) changed since the counters were taken."""
    import hashlib

    if workload != "prefill" or not os.path.exists(PROFILE):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "combine_ep_get_02_amd", "csrc", f), "rb") as fh:
            h.update(source_code_only(fh.read()))
    fields = {}
    with open(PROFILE) as fh:
        for line in fh:
            parts = line.split()
            if len(parts) == 3 and parts[0] in ("traffic_bytes", "source_sha256"):
                fields[(parts[0], parts[1])] = parts[2]
    if fields.get(("source_sha256", kernel)) != h.hexdigest()[:16]:
        return None
    v = fields.get(("traffic_bytes", kernel))
    return int(v) if v is not None else None


def cpu_baseline(d, wl, n_recv, budget_s: float = 12.0) -> dict:
    """The oracle (single-threaded C) on the same workload, full steps repeated
    until about budget_s of CPU time has passed."""
    import oracle

    o = oracle.Oracle()
    x, idx, w = d["x"], d["topk_idx"], d["topk_weights"]
    reps, t0 = 0, time.perf_counter()
    t_lay = t_note = t_disp = t_comb = 0.0
    while True:
        z = time.perf_counter()
        lay = o.layout(idx, wl.experts, wl.ranks)
        y = time.perf_counter()
        note = o.notify(lay["is_token_in_rank"], lay["num_tokens_per_rank"], lay["num_tokens_per_rdma_rank"],
                        lay["num_tokens_per_expert"], wl.channels, wl.expert_alignment)
        a = time.perf_counter()
        t_lay += y - z
        t_note += a - y
        dis = o.dispatch(x, idx, w, lay["is_token_in_rank"], note["gbl_channel_prefix_matrix"],
                         note["recv_gbl_rank_prefix_sum"], wl.experts)
        b = time.perf_counter()
        o.combine(dis["recv_x"], dis["recv_topk_weights"], dis["send_slot"], note["num_recv_tokens"])
        c = time.perf_counter()
        t_disp += b - a
        t_comb += c - b
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= 20:
            break
    T, H, K, R = wl.tokens, wl.hidden, wl.topk, wl.ranks
    alg = dispatch_bytes(T, H, K, R, n_recv) + combine_bytes(T, H, K, R, n_recv)
    dc = (t_disp + t_comb) / reps
    return {"value": round(alg / dc / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full {wl.name} steps (layout+notify+dispatch+combine, t={T}, h={H}, k={K}, "
                      f"R={R}); value = dispatch+combine algorithmic bytes / oracle dispatch+combine time",
            "us_dispatch_plus_combine": round(dc * 1e6, 1),
            "us_per_stage": {"layout": round(t_lay / reps * 1e6, 1), "notify": round(t_note / reps * 1e6, 1),
                             "dispatch": round(t_disp / reps * 1e6, 1), "combine": round(t_comb / reps * 1e6, 1)},
            "host_cores": os.cpu_count(), "host_cpu": host_cpu_model()}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class HipEvents:
    """HIP events on torch's current stream, created with
    hipEventDisableSystemFence: recording one then skips the system-scope
    cache write-back that a default event performs, which otherwise adds a few
    microseconds to every bracketed launch.  Uses the HIP runtime the process
    has already loaded (torch's), so the events and torch's streams belong to
    the same runtime."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes

        import torch

        torch.zeros(1, device="cuda")  # runtime loaded and device initialised
        paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln})
        # the events must come from the runtime that owns torch's streams
        torch_dir = os.path.dirname(torch.__file__)
        own = [q for q in paths if q.startswith(torch_dir)] or paths
        if len(own) != 1:
            raise RuntimeError(f"cannot tell which HIP runtime owns torch's streams: {paths}")
        self._ct = ctypes
        self._hip = ctypes.CDLL(own[0])
        self._torch = torch
        self._live = []

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def event(self):
        e = self._ct.c_void_p()
        self._check(self._hip.hipEventCreateWithFlags(self._ct.byref(e), self._ct.c_uint(self.DISABLE_SYSTEM_FENCE)),
                    "hipEventCreateWithFlags")
        self._live.append(e)
        return e

    def pair(self):
        return self.event(), self.event()

    def record(self, e):
        stream = self._ct.c_void_p(self._torch.cuda.current_stream().cuda_stream)
        self._check(self._hip.hipEventRecord(e, stream), "hipEventRecord")

    def elapsed_us(self, a, c) -> float:
        ms = self._ct.c_float()
        self._check(self._hip.hipEventSynchronize(c), "hipEventSynchronize")
        self._check(self._hip.hipEventElapsedTime(self._ct.byref(ms), a, c), "hipEventElapsedTime")
        return ms.value * 1e3

    def mean_us(self, fn, n: int) -> float:
        """mean duration of n back-to-back calls of fn between one event pair"""
        a, c = self.pair()
        self.record(a)
        for _ in range(n):
            fn()
        self.record(c)
        return self.elapsed_us(a, c) / n

    def brackets_us(self, fn, brackets: int, per: int) -> list[float]:
        """per-launch means of `brackets` groups of `per` back-to-back calls"""
        return [self.mean_us(fn, per) for _ in range(brackets)]

    def close(self):
        self._torch.cuda.synchronize()
        for e in self._live:
            self._hip.hipEventDestroy(e)
        self._live = []


def time_workloads(ep, inputs, names, timer, brackets: int = 5, per: int = 4) -> dict:
    """dispatch and combine on other workloads (identity experts, inputs in
    HBM): each kernel's per-launch time as the median and minimum over
    `brackets` groups of `per` back-to-back launches, GB/s from the median."""
    import torch

    out = {}
    for name in names:
        d = inputs.generate(name)
        wl = d["workload"]
        T, H, K, E, R, C = wl.tokens, wl.hidden, wl.topk, wl.experts, wl.ranks, wl.channels
        shape = ep.make_shape(T, H, K, E, R, C, 0, wl.expert_alignment)
        x = torch.from_numpy(d["x"].view(np.int16)).cuda().view(torch.bfloat16)
        idx = torch.from_numpy(d["topk_idx"]).cuda()
        w = torch.from_numpy(d["topk_weights"]).cuda()
        probe = ep.allocate(shape, 0)
        ep.run_layout(probe, idx)
        n = ep.run_notify(probe, read_back=True)
        del probe
        b = ep.allocate(shape, n)
        calls = {"layout": lambda: ep.run_layout(b, idx), "notify": lambda: ep.run_notify(b),
                 "layout_notify": lambda: ep.run_layout_notify(b, idx),
                 "dispatch": lambda: ep.run_dispatch(b, x, idx, w), "combine": lambda: ep.run_combine(b)}
        for f in calls.values():
            f()
        t = {k: sorted(timer.brackets_us(f, brackets, per)) for k, f in calls.items()}
        med = {k: float(np.median(v)) for k, v in t.items()}
        # the whole step from a HIP graph: no host launch cost between the kernels
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in ("layout_notify", "dispatch", "combine"):
                calls[k]()
        graph_us = timer.mean_us(graph.replay, brackets * per)
        db, cb = dispatch_bytes(T, H, K, R, n), combine_bytes(T, H, K, R, n)
        live = b.in_rank.bool().any(1)
        # identity experts return x (compared as values: the accumulator starts at +0, so -0 returns as +0)
        ok = bool(torch.equal(b.combined_x[live].float(), x[live].float())) and int(b.dev_status.item()) == 0
        out[name] = {
            "config": f"t={T}, h={H}, topk={K}, experts={E}, ranks={R}, channels={C}", "num_recv_tokens": n,
            "us_dispatch_median": round(med["dispatch"], 2), "us_dispatch_min": round(t["dispatch"][0], 2),
            "us_combine_median": round(med["combine"], 2), "us_combine_min": round(t["combine"][0], 2),
            "us_layout_median": round(med["layout"], 2), "us_notify_median": round(med["notify"], 2),
            "us_layout_notify_median": round(med["layout_notify"], 2),
            "us_step_graph": round(graph_us, 2),
            "GB/s_dispatch_plus_combine": round((db + cb) / (med["dispatch"] + med["combine"]) / 1e3, 2),
            "pct_peak": round(100 * (db + cb) / (med["dispatch"] + med["combine"]) / 1e3 / HBM_PEAK_GBPS, 2),
            "identity_check": ok}
        del b, x, idx, w
        torch.cuda.empty_cache()
    return out


def time_variants(ep, inputs, d, shape, b, x, idx, w, n_recv, steps: int, timer) -> dict:
    """Cached-mode and fp8-row dispatch on the same workload, reported beside
    the metric (which stays the bf16 path).  Each call's duration is the mean
    of `steps` back-to-back launches after one warm-up; each result is checked
    against the bf16 dispatch just measured (cached rows equal, fp8 rows and
    scales found at the same send_slot rows)."""
    import torch

    wl = d["workload"]
    T, H, K, R = wl.tokens, wl.hidden, wl.topk, wl.ranks

    def mean_us(fn):
        fn()
        return timer.mean_us(fn, steps)

    def rate(nbytes, us):
        return {"us": round(us, 2), "bytes": nbytes, "GB/s": round(nbytes / us / 1e3, 2),
                "pct_peak": round(100 * nbytes / us / 1e3 / HBM_PEAK_GBPS, 2)}

    out = {}
    live = b.send_slot >= 0
    rows = b.send_slot[live].long()
    tok = torch.arange(T, device=x.device).unsqueeze(1).expand(T, R)[live]

    # dispatch without a workspace: the routing worked out from is_token_in_rank and the
    # prefix sums inside the call (same metadata outputs, so b's buffers are reused)
    rx2, ss2 = torch.empty_like(b.recv_x), torch.empty_like(b.send_slot)
    out["dispatch_no_workspace"] = rate(dispatch_bytes(T, H, K, R, n_recv), mean_us(
        lambda: ep.ep_dispatch(shape, x, idx, w, b.in_rank, b.gbl, b.recv_gbl, None, n_recv, rx2, b.recv_w,
                               b.recv_idx, b.src_info, ss2, b.dev_status)))
    out["dispatch_no_workspace"]["check"] = bool(torch.equal(ss2, b.send_slot) and
                                                 torch.equal(rx2.view(torch.int16), b.recv_x.view(torch.int16)))
    del rx2, ss2

    cx = torch.empty_like(b.recv_x)
    out["dispatch_cached_bf16"] = rate(dispatch_cached_bytes(T, R, n_recv, 2 * H, 0), mean_us(
        lambda: ep.ep_dispatch_cached(shape, x, 2, None, 0, b.send_slot, n_recv, cx, None, b.dev_status)))
    out["dispatch_cached_bf16"]["check"] = bool(torch.equal(cx.view(torch.int16), b.recv_x.view(torch.int16)))
    del cx

    # fp8 rows: e4m3 with one fp32 scale per 128-element block, as a caller would quantise them
    x8n, scn = inputs.fp8_rows(d["x"])
    x8, sc = torch.from_numpy(x8n).cuda(), torch.from_numpy(scn).cuda()
    S = sc.shape[1]
    rx = torch.empty((n_recv, H), dtype=torch.uint8, device=x.device)
    rs = torch.empty((n_recv, S), dtype=torch.float32, device=x.device)
    slot8 = torch.empty_like(b.send_slot)
    out["dispatch_fp8"] = rate(dispatch_fp8_bytes(T, H, K, R, n_recv, S), mean_us(
        lambda: ep.ep_dispatch_fp8(shape, x8, sc, S, idx, w, b.in_rank, b.gbl, b.recv_gbl, b.workspace, n_recv, rx,
                                   rs, b.recv_w, b.recv_idx, b.src_info, slot8, b.dev_status)))
    out["dispatch_fp8"]["check"] = bool(torch.equal(slot8, b.send_slot) and torch.equal(rx[rows], x8[tok])
                                        and torch.equal(rs[rows], sc[tok]))
    out["dispatch_fp8"]["num_scales"] = S
    out["dispatch_fp8_push"] = rate(dispatch_fp8_bytes(T, H, K, R, n_recv, S), mean_us(
        lambda: ep.ep_dispatch_fp8(shape, x8, sc, S, idx, w, b.in_rank, b.gbl, b.recv_gbl, b.workspace, n_recv, rx,
                                   rs, b.recv_w, b.recv_idx, b.src_info, slot8, b.dev_status, form=ep.EP_FORM_PUSH)))
    out["dispatch_fp8_push"]["check"] = bool(torch.equal(slot8, b.send_slot) and torch.equal(rx[rows], x8[tok])
                                             and torch.equal(rs[rows], sc[tok]))
    cx8, cs8 = torch.empty_like(rx), torch.empty_like(rs)
    out["dispatch_cached_fp8"] = rate(dispatch_cached_bytes(T, R, n_recv, H, S), mean_us(
        lambda: ep.ep_dispatch_cached(shape, x8, 1, sc, S, b.send_slot, n_recv, cx8, cs8, b.dev_status)))
    out["dispatch_cached_fp8"]["check"] = bool(torch.equal(cx8, rx) and torch.equal(cs8, rs))
    del cx8, cs8

    # the library's E4M3 quantiser on the same bf16 rows (groups of 128 channels), alone and
    # followed by the fp8 dispatch of what it wrote: a caller's whole fp8 path from bf16 rows.
    # Checked by what the quantiser fixes: every group's largest magnitude is coded +-448, and the
    # scales are amax / 448 as the caller-side recipe above makes them.
    q8 = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    qs = torch.empty((T, S), dtype=torch.float32, device=x.device)
    out["quantize_fp8"] = rate(quantize_bytes(T, H, S), mean_us(lambda: ep.ep_quantize_fp8(x, T, H, S, q8, qs)))
    qv = q8.cpu().view(torch.float8_e4m3fn).float().view(T, S, H // S)
    out["quantize_fp8"]["check"] = bool(torch.all(qv.abs().amax(dim=2) == 448.0) and torch.equal(qs, sc))
    out["quantize_fp8"]["num_scales"] = S
    out["quantize_fp8"]["traffic"] = measured_traffic("quantize_e4m3_kernel", wl.name)
    del qv

    def quant_then_dispatch():
        ep.ep_quantize_fp8(x, T, H, S, q8, qs)
        ep.ep_dispatch_fp8(shape, q8, qs, S, idx, w, b.in_rank, b.gbl, b.recv_gbl, b.workspace, n_recv, rx, rs,
                           b.recv_w, b.recv_idx, b.src_info, slot8, b.dev_status)

    out["quantize_then_dispatch_fp8"] = rate(quantize_bytes(T, H, S) + dispatch_fp8_bytes(T, H, K, R, n_recv, S),
                                             mean_us(quant_then_dispatch))
    out["quantize_then_dispatch_fp8"]["check"] = bool(torch.equal(slot8, b.send_slot) and
                                                      torch.equal(rx[rows], q8[tok]) and torch.equal(rs[rows], qs[tok]))
    # the same path in one launch: each token's bf16 row read once and quantised once (push form);
    # checked against the two calls just made
    rx2, rs2, slot2 = torch.empty_like(rx), torch.empty_like(rs), torch.empty_like(slot8)
    out["dispatch_to_fp8"] = rate(dispatch_to_fp8_bytes(T, H, K, R, n_recv, S), mean_us(
        lambda: ep.ep_dispatch_to_fp8(shape, x, S, idx, w, b.in_rank, b.gbl, b.recv_gbl, b.workspace, n_recv, rx2, rs2,
                                      b.recv_w, b.recv_idx, b.src_info, slot2, b.dev_status)))
    out["dispatch_to_fp8"]["check"] = bool(torch.equal(slot2, slot8) and torch.equal(rx2, rx) and torch.equal(rs2, rs))
    out["dispatch_to_fp8"]["traffic"] = measured_traffic("dispatch_kernel_to_fp8", wl.name)
    # the same in cached mode, from the send_slot just written: the same codes and scales
    cq, cqs = torch.empty_like(rx2), torch.empty_like(rs2)
    out["dispatch_cached_to_fp8"] = rate(dispatch_cached_to_fp8_bytes(T, H, R, n_recv, S), mean_us(
        lambda: ep.ep_dispatch_cached_to_fp8(shape, x, S, slot2, n_recv, cq, cqs, b.dev_status)))
    out["dispatch_cached_to_fp8"]["check"] = bool(torch.equal(cq, rx2) and torch.equal(cqs, rs2))
    out["dispatch_cached_to_fp8"]["traffic"] = measured_traffic("dispatch_kernel_cached_to_fp8", wl.name)
    del cq, cqs
    # the receive side's dequantiser on those rows (E4M3 codes and scales -> bf16); checked on the host on
    # a sample of rows: torch's float8 decoding times the scale in fp32, rounded to bf16 by torch
    back = torch.empty((n_recv, H), dtype=torch.bfloat16, device=x.device)
    out["dequantize_fp8"] = rate(dequantize_bytes(n_recv, H, S),
                                 mean_us(lambda: ep.ep_dequantize_fp8(rx2, rs2, n_recv, H, S, back)))
    hs = min(n_recv, 512)
    want = (rx2[:hs].cpu().view(torch.float8_e4m3fn).float() *
            rs2[:hs].cpu().repeat_interleave(H // S, dim=1)).to(torch.bfloat16)
    out["dequantize_fp8"]["check"] = bool(torch.equal(back[:hs].cpu().view(torch.int16), want.view(torch.int16)))
    out["dequantize_fp8"]["traffic"] = measured_traffic("dequantize_e4m3_kernel", wl.name)
    del rx2, rs2, slot2, back
    del rx, rs, x8, sc, q8, qs

    # grouping of the receive rows by local expert (bf16 rows of the dispatch just measured)
    M = int(b.recv_per_expert.sum().item())
    g = ep.allocate_group(b, M)
    out["group_by_expert"] = rate(group_bytes(H, K, n_recv, M), mean_us(lambda: ep.run_group(b, g, n_recv)))
    entries = g.grouped_row >= 0
    gr = g.grouped_row[entries].long()
    out["group_by_expert"]["check"] = bool(
        int(g.num_grouped.item()) == M and int(entries.sum().item()) == int((idx >= 0).sum().item())
        and torch.equal(g.grouped_x[entries].view(torch.int16), b.recv_x[gr].view(torch.int16))
        and not bool(g.grouped_x[~entries].view(torch.int16).any().item()))
    out["group_by_expert"]["grouped_rows"] = M
    del g
    for key, kernel in (("dispatch_cached_bf16", "dispatch_kernel_cached_bf16"), ("dispatch_fp8", "dispatch_pull_kernel_fp8"),
                        ("dispatch_cached_fp8", "dispatch_kernel_cached_fp8")):
        out[key]["traffic"] = measured_traffic(kernel, wl.name)
    out["group_by_expert"]["traffic"] = measured_traffic("group_kernels", wl.name)
    # dispatch straight into the grouped layout: same grouped rows, no receive rows
    # (the two-call result it is checked against is made first)
    g = ep.allocate_group(b, M)
    ep.run_group(b, g, n_recv)
    g2 = ep.allocate_group(b, M)
    out["dispatch_grouped"] = rate(dispatch_grouped_bytes(T, H, K, R, n_recv, M),
                                   mean_us(lambda: ep.run_dispatch_grouped(b, g2, x, idx, w)))
    torch.cuda.synchronize()
    out["dispatch_grouped"]["check"] = bool(
        int(g2.num_grouped.item()) == M and torch.equal(g2.grouped_row, g.grouped_row)
        and torch.equal(g2.grouped_x.view(torch.int16), g.grouped_x.view(torch.int16)))
    out["dispatch_grouped"]["grouped_rows"] = M
    out["dispatch_grouped"]["traffic"] = measured_traffic("dispatch_grouped_pull_kernel", wl.name)
    del g, g2
    out["dev_status"] = int(b.dev_status.item())
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the timings reported beside the metric: dispatch without a workspace, cached mode, "
                         "fp8 rows, the E4M3 quantiser and dequantiser, the quantising dispatches, the grouping "
                         "and the dispatch straight into the grouped layout")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing of the step")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the dispatch/combine timings of the other four workloads reported beside the metric")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="extra steps with a 1 GiB scratch write before each, untimed, to evict the caches")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times) and exit; used to "
                         "scale the HBM byte counters of a profiler against a copy of known size")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch

        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n}))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the path; --gpus {args.gpus} is not supported "
              f"(the library has no multi-GPU path)", file=sys.stderr)
        return 2

    import torch

    from combine_ep_get_02_amd import ep, inputs

    if not os.path.exists(ep.LIBRARY):
        import __graft_entry__

        __graft_entry__.build()

    torch.cuda.set_device(0)
    d = inputs.generate(args.workload)
    wl = d["workload"]
    T, H, K, E, R, C = wl.tokens, wl.hidden, wl.topk, wl.experts, wl.ranks, wl.channels
    shape = ep.make_shape(T, H, K, E, R, C, 0, wl.expert_alignment)
    x = torch.from_numpy(d["x"].view(np.int16)).cuda().view(torch.bfloat16)
    idx = torch.from_numpy(d["topk_idx"]).cuda()
    w = torch.from_numpy(d["topk_weights"]).cuda()

    probe = ep.allocate(shape, 0)
    ep.run_layout(probe, idx)
    n_recv = ep.run_notify(probe, read_back=True)
    del probe
    b = ep.allocate(shape, n_recv)

    timer = HipEvents()
    calls = {"layout": lambda: ep.run_layout(b, idx), "notify": lambda: ep.run_notify(b),
             "layout_notify": lambda: ep.run_layout_notify(b, idx),
             "dispatch": lambda: ep.run_dispatch(b, x, idx, w), "combine": lambda: ep.run_combine(b)}

    def step(ev=None):
        calls["layout_notify"]()
        if ev is not None:
            timer.record(ev[0])
        calls["dispatch"]()
        calls["combine"]()
        if ev is not None:
            timer.record(ev[1])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole steps; one event pair per step around dispatch+combine
    events = [timer.pair() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dc_steps = [timer.elapsed_us(a, c) for a, c in events]
    us_dc = float(np.mean(dc_steps))

    # each kernel's average launch duration: K back-to-back launches between one event pair
    us = {k: timer.mean_us(f, args.steps) for k, f in calls.items()}

    # the same step captured once in a HIP graph and replayed K times
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        ga, gc = timer.pair()
        w0 = time.perf_counter()
        timer.record(ga)
        for _ in range(args.steps):
            g.replay()
        timer.record(gc)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - w0) / args.steps
        graph = {"us_per_step_gpu": round(timer.elapsed_us(ga, gc) / args.steps, 2),
                 "ms_per_step_wall": round(wall * 1e3, 4),
                 "note": "layout_notify+dispatch+combine captured with torch.cuda.graph, K replays back to back"}

    # correctness guard on the measured buffers: identity experts return x
    live = b.in_rank.bool().any(1)
    ok = bool(torch.equal(b.combined_x[live], x[live])) and int(b.dev_status.item()) == 0

    # cold-cache cross-check: evict with a 1 GiB write before each (untimed) dispatch+combine
    cold = None
    if args.cold_steps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cev = [(timer.pair(), timer.pair()) for _ in range(args.cold_steps)]
        for (d0, d1), (c0, c1) in cev:
            calls["layout_notify"]()
            scratch.fill_(7)
            timer.record(d0)
            calls["dispatch"]()
            timer.record(d1)
            scratch.fill_(9)
            timer.record(c0)
            calls["combine"]()
            timer.record(c1)
        torch.cuda.synchronize()
        # the push form, which a caller takes when x is only in HBM
        pev = [timer.pair() for _ in range(args.cold_steps)]
        for p0, p1 in pev:
            calls["layout_notify"]()
            scratch.fill_(7)
            timer.record(p0)
            ep.run_dispatch(b, x, idx, w, form=ep.EP_FORM_PUSH)
            timer.record(p1)
        torch.cuda.synchronize()
        # the same, with x written again after the scratch write, as the layer before
        # dispatch writes it: x is then in the caches a freshly written tensor is in
        xs = x.clone()
        fev = [timer.pair() for _ in range(args.cold_steps)]
        for f0, f1 in fev:
            calls["layout_notify"]()
            scratch.fill_(7)
            x.copy_(xs)
            timer.record(f0)
            calls["dispatch"]()
            timer.record(f1)
        torch.cuda.synchronize()
        us_cd = float(np.mean([timer.elapsed_us(*dp) for dp, _ in cev]))
        us_cp = float(np.mean([timer.elapsed_us(*pp) for pp in pev]))
        us_cc = float(np.mean([timer.elapsed_us(*cp) for _, cp in cev]))
        cold_bytes = dispatch_bytes(T, H, K, R, n_recv) + combine_bytes(T, H, K, R, n_recv)
        cold = {"us_dispatch": round(us_cd, 2), "us_dispatch_push": round(us_cp, 2), "us_combine": round(us_cc, 2),
                "us_dispatch_fresh_x": round(float(np.mean([timer.elapsed_us(*fp) for fp in fev])), 2),
                "pct_peak_dispatch_plus_combine": round(100 * cold_bytes / (us_cd + us_cc) / 1e3 / HBM_PEAK_GBPS, 2),
                "pct_peak_dispatch_push_plus_combine":
                    round(100 * cold_bytes / (us_cp + us_cc) / 1e3 / HBM_PEAK_GBPS, 2),
                "note": "one launch each after a 1 GiB scratch write, single-call events; us_dispatch: the default "
                        "(pull) form, us_dispatch_push: EP_FORM_PUSH, the form for x only in HBM; fresh_x: x "
                        "copied in again after the scratch write, before dispatch"}
        del scratch, xs

    variants = None if args.no_variants else time_variants(ep, inputs, d, shape, b, x, idx, w, n_recv, args.steps,
                                                             timer)
    if variants is not None:
        ok = ok and variants["dev_status"] == 0 and all(v["check"] for k, v in variants.items() if k != "dev_status")

    # median and minimum at this workload, over brackets of back-to-back launches
    spread = {k: sorted(timer.brackets_us(calls[k], 5, max(1, args.steps // 5))) for k in calls}
    others = None
    if not args.no_other_workloads:
        others = time_workloads(ep, inputs, [n for n in inputs.WORKLOADS if n != wl.name], timer)
        ok = ok and all(v["identity_check"] for v in others.values())

    db, cb = dispatch_bytes(T, H, K, R, n_recv), combine_bytes(T, H, K, R, n_recv)
    gbps = (db + cb) / us_dc / 1e3
    if us["dispatch"] >= us["combine"]:
        dom, dom_bytes, dom_us = "dispatch_pull_kernel", db, us["dispatch"]
    else:
        dom, dom_bytes, dom_us = combine_kernel_name(T, H), cb, us["combine"]
    achieved = dom_bytes / dom_us / 1e3
    out = {
        "metric": "dispatch+combine µs/iter and HBM GB/s (% peak) at t=4096,h=7168,topk=8",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: t={T}, h={H}, topk={K}, experts={E}, emulated ranks={R} "
                               f"({max(1, R // 8)} nodes x 8), channels={C}, uniform routing, seed {wl.seed}",
                   "global_batch": T, "seq_len": 1, "parallelism": "single GPU share (one source rank)"},
        "us_per_iter_dispatch_plus_combine": round(us_dc, 2),
        "us_dispatch_plus_combine_median_min": [round(float(np.median(dc_steps)), 2), round(float(min(dc_steps)), 2)],
        "pct_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "us_layout": round(us["layout"], 2),
        "us_notify": round(us["notify"], 2),
        "us_layout_notify": round(us["layout_notify"], 2),
        "us_dispatch": round(us["dispatch"], 2),
        "us_combine": round(us["combine"], 2),
        "timing": "value: dispatch+combine bytes / mean time between one event pair per timed step around "
                  "dispatch+combine; us_<kernel>: mean of back-to-back launches between one event pair; "
                  "events created with hipEventDisableSystemFence",
        "num_recv_tokens": n_recv,
        "bytes_dispatch": db,
        "bytes_combine": cb,
        "bytes_layout_notify": layout_notify_bytes(T, K, R, E, C),
        "identity_check": ok,
        "us_median_min": {k: [round(float(np.median(v)), 2), round(v[0], 2)] for k, v in spread.items()},
        "cold": cold,
        "graph": graph,
        "variants": variants,
        "other_workloads": others,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom, wl.name), "algorithmic_bytes": dom_bytes,
                     "us_per_launch": round(dom_us, 2)},
    }
    timer.close()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(d, wl, n_recv)
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
