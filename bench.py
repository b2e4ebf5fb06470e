#!/usr/bin/env python3
"""Throughput of the MTP draft / verify LM-head path on one MI355X.

One step is one MTP round of the workload: its draft calls (GEMV + argmax over
the packed candidate table) followed by one verify call (GEMM + per-row argmax
+ greedy acceptance over the full head). Default workload: MTP3 single stream,
H=2048, 248,320-row head, 65,536-row candidate table, 3 draft calls (M=1) and
one verify call (M=4).

    python bench.py [--steps K] [--warmup W] [--workload NAME]

Inputs are seeded synthetic data (N(0,0.02) bf16 head, N(0,1) bf16 hidden
states, seeded sorted candidate subset), resident in HBM before timing. The
draft calls of one step read three different copies of the candidate table, so
no call is served from the 256 MB Infinity Cache by its predecessor; the
verify head (>= 1 GB) cannot stay cached between steps. Per-call durations
come from one HIP event per call of every timed step, stamped by the library
with the end of the call's last kernel on the launch stream
(mtp_time_next_call): a call's time is the span from the previous call's end to
its own end. A warm-up of at least --warmup-seconds precedes the timed steps.
Prints one JSON line.

--workload draft_ablation adds context.draft_tables: the M = 1 draft timed over
the full head, the 65,536-row and the nested 32,768-row tables (and the pages'
per-rank shard shape, 32,768 x 2,560), with us per call, GB/s and the fraction
of peak and of the streaming-read ceiling for each.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("draft/verify calls/s and achieved HBM GB/s (% peak) at 248,320-vocab, 64K draft")
HBM_PEAK_GBPS = 8000.0
# sources that define each path's kernels and their launch configuration
# Device code of each path (launch.hpp holds host-side launch structs only).
KERNEL_SOURCES = {
    "valu": ("common.hpp", "gemv_valu.hip"),
    "mfma": ("common.hpp", "gemm_mfma.hip"),
    "dma": ("common.hpp", "gemm_dma.hip"),
    "fp8": ("common.hpp", "fp8.hip"),
    "fp4": ("common.hpp", "fp4.hip"),
    "pack": ("pack.hip",),
    "probe": ("probe.hip",),
}


def rows_path(M: int, H: int) -> str:
    """Kernel family a row-major bf16 call of M hidden rows at width H runs on
    (the selection rule of the C ABI): the vector-ALU kernel while one pass
    keeps every hidden row's slice in registers (16-byte chunks per lane
    rounded up to an instantiated count, at most 32 chunk slices), the LDS-DMA
    matrix-core kernel for H % 64 == 0, else the register-staged one."""
    need = -(-(H // 8) // 64)
    ncl = next((n for n in (1, 2, 3, 4, 5, 6, 8, 10, 12, 16, 20, 24, 32) if n >= need), 0)
    mr = 1
    while ncl and mr < 8 and mr < M and 2 * mr * ncl <= 32:
        mr *= 2
    if ncl and mr >= M:
        return "valu"
    return "dma" if H % 64 == 0 else "mfma"


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mtp3_single")
    ap.add_argument("--table-copies", type=int, default=3)
    ap.add_argument("--layout", choices=("auto", "rows", "tiled"), default="auto",
                    help="table layout: row-major, or the 64-row tiled layout of include/mtp.h "
                         "(auto: rows when every call has at most 8 hidden rows)")
    ap.add_argument("--table", choices=("bf16", "fp8", "mxfp4"), default="bf16",
                    help="precision of the draft's candidate table: bf16 rows, E4M3 rows "
                         "with power-of-two row scales (mtp_pack_candidates_fp8, or "
                         "mtp_pack_tiled_fp8 with --layout tiled), or MXFP4 rows (E2M1 codes, "
                         "one E8M0 scale per 32 elements; mtp_pack_candidates_mxfp4, or "
                         "mtp_pack_tiled_mxfp4 with --layout tiled); the verify always reads "
                         "the bf16 head")
    ap.add_argument("--mx-scale", choices=("ocp", "fit"), default="ocp",
                    help="block scale rule of the MXFP4 packs: the OCP MX rule "
                         "floor(log2 max|w|) - 2 (default), or the smallest e with "
                         "max|w| <= 6 * 2^e (no element saturates)")
    ap.add_argument("--agree-rows", type=int, default=512,
                    help="hidden rows of the untimed check of how often a quantised draft "
                         "picks the bf16 draft's token")
    ap.add_argument("--draft-source", choices=("table", "gather"), default="table",
                    help="draft calls read a packed candidate table (default), or head rows "
                         "through a per-call id list (mtp_draft_argmax_gather; with --table "
                         "fp8 or mxfp4, the gathered draft over a head quantised once; "
                         "row-major only)")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of a captured HIP graph (mtp_graph_*); "
                         "per-call durations still come from event-bracketed eager launches")
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="after the --warmup steps, keep running untimed steps until the warm-up "
                         "has lasted this long, so that the timed steps start with the GPU's "
                         "clocks and queues already in their steady state")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the CPU oracle sample")
    return ap.parse_args()


def code_text(src: str) -> str:
    """C/C++/HIP source without its comments and with runs of blank space
    collapsed, so that an edit of comments or layout leaves the hash alone.
    String and character literals are kept whole (a "//" inside one is not a
    comment)."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(path: str) -> str:
    """Hash of a kernel family's sources (code only: see code_text). A profile
    summary carries it, and the bench uses a summary's counters only when
    its hash equals that of the sources as they are now."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_argmax_amd", "csrc")
    for name in KERNEL_SOURCES[path]:
        p = os.path.join(csrc, name)
        if os.path.exists(p):
            h.update(name.encode())
            h.update(code_text(open(p, encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, profile: str, path: str):
    """HBM bytes per launch of the verify or draft call, from the committed
    rocprofv3 counter summary of the workload (profiles/verify_<profile>_pmc.txt),
    if it was taken from the current sources."""
    p = os.path.join(ROOT, "profiles", f"verify_{profile}_pmc.txt")
    if not os.path.exists(p):
        return None
    text = open(p).read()
    key = "hbm_bytes_per_launch" if kernel == "verify" else f"{kernel}_hbm_bytes_per_launch"
    m_hash = re.search(r"^kernel_source_hash:\s*(\S+)", text, re.M)
    m_bytes = re.search(rf"^{key}:\s*([0-9.eE+]+)", text, re.M)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(path):
        return None
    return float(m_bytes.group(1))


def main() -> int:
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this path has no "
              "multi-GPU mode.", file=sys.stderr)
        return 2
    import torch

    from speculative_decoding_argmax_amd import mtp
    from speculative_decoding_argmax_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 2
    wk = wl.workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.graph:
        # graph capture needs a created stream (the null stream cannot be
        # captured); everything below runs on it
        torch.cuda.set_stream(torch.cuda.Stream(dev))
    stream = torch.cuda.current_stream()

    t0 = time.time()
    head = wl.head_weights(wk.V, wk.H, wk.seed)
    ids = wl.candidate_ids(wk.V, wk.C, wk.seed)
    hiddens = [wl.hidden_states(wk.Md, wk.H, wk.seed, block=c) for c in range(wk.draft_calls)]
    hv = wl.hidden_states(wk.Mv, wk.H, wk.seed, block=100)

    def up(a, dt=np.int16):
        return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(dev)

    layout = args.layout
    fp4 = args.table == "mxfp4"
    mx_rule = mtp.MX_SCALE_RULES[args.mx_scale]
    if layout == "auto":
        layout = "rows" if max(wk.Md, wk.Mv) <= 8 else "tiled"
    gather = args.draft_source == "gather"
    fp8 = args.table == "fp8"
    if gather and layout != "rows":
        print("--draft-source gather runs on the row-major head (use --layout rows)",
              file=sys.stderr)
        return 2
    head_d = up(head)
    ids_d = up(ids, np.int32)
    tables = []
    for _ in range(1 if gather else max(1, args.table_copies)):
        if fp8 and gather:
            # every head row quantised once; each call gathers its own rows
            tq = torch.empty((wk.V, wk.H), dtype=torch.uint8, device=dev)
            ts = torch.empty(wk.V, dtype=torch.float32, device=dev)
            mtp.mtp_pack_candidates_fp8(head_d, None, tq, ts, C=wk.V)
            tables.append((tq, ts))
            continue
        if fp4 and gather:
            # every head row quantised once; each call gathers its own rows
            tq = torch.empty((wk.V, wk.H // 2), dtype=torch.uint8, device=dev)
            ts = torch.empty((wk.V, wk.H // 32), dtype=torch.uint8, device=dev)
            mtp.mtp_pack_candidates_mxfp4(head_d, None, tq, ts, C=wk.V, rule=mx_rule)
            tables.append((tq, ts))
            continue
        if fp4 and layout == "tiled":
            tq, ts = mtp.alloc_tiled_mxfp4(wk.C, wk.H, dev)
            mtp.mtp_pack_tiled_mxfp4(head_d, ids_d, tq, ts, rule=mx_rule)
            tables.append((tq, ts))
            continue
        if fp4:
            tq = torch.empty((wk.C, wk.H // 2), dtype=torch.uint8, device=dev)
            ts = torch.empty((wk.C, wk.H // 32), dtype=torch.uint8, device=dev)
            mtp.mtp_pack_candidates_mxfp4(head_d, ids_d, tq, ts, rule=mx_rule)
            tables.append((tq, ts))
            continue
        if fp8 and layout == "rows":
            tq = torch.empty((wk.C, wk.H), dtype=torch.uint8, device=dev)
            ts = torch.empty(wk.C, dtype=torch.float32, device=dev)
            mtp.mtp_pack_candidates_fp8(head_d, ids_d, tq, ts)
            tables.append((tq, ts))
            continue
        if fp8:
            tq, ts = mtp.alloc_tiled_fp8(wk.C, wk.H, dev)
            mtp.mtp_pack_tiled_fp8(head_d, ids_d, tq, ts)
            tables.append((tq, ts))
            continue
        if layout == "rows":
            t = torch.empty((wk.C, wk.H), dtype=torch.int16, device=dev)
            mtp.mtp_pack_candidates(head_d, ids_d, t)
        else:
            t = mtp.alloc_tiled(wk.C, wk.H, dev)
            mtp.mtp_pack_tiled(head_d, ids_d, t)
        tables.append(t)
    if layout == "tiled" or fp8 or fp4:
        # counter calibration for rocprofv3 runs (untimed): one plain
        # gather-copy of known size, the row-major candidate pack, which
        # these layouts do not otherwise run
        calib = torch.empty((wk.C, wk.H), dtype=torch.int16, device=dev)
        mtp.mtp_pack_candidates(head_d, ids_d, calib)
        torch.cuda.synchronize()
        del calib
    if layout == "tiled":
        head_v = mtp.alloc_tiled(wk.V, wk.H, dev)
        mtp.mtp_pack_tiled(head_d, None, head_v, C=wk.V)
    else:
        head_v = head_d
    h_d = [up(h) for h in hiddens]
    hv_d = up(hv)
    out_ids = [torch.empty(wk.Md, dtype=torch.int32, device=dev) for _ in range(wk.draft_calls)]
    out_logit = [torch.empty(wk.Md, dtype=torch.float32, device=dev)
                 for _ in range(wk.draft_calls)]
    ws_d = mtp.alloc_workspace(mtp.mtp_draft_workspace_bytes(wk.Md, wk.C, wk.H), dev)
    ws_v = mtp.alloc_workspace(mtp.mtp_verify_workspace_bytes(wk.B, wk.k, wk.V, wk.H), dev)
    v_arg = torch.empty((wk.B, wk.k + 1), dtype=torch.int32, device=dev)
    v_logit = torch.empty((wk.B, wk.k + 1), dtype=torch.float32, device=dev)
    v_acc = torch.empty(wk.B, dtype=torch.int32, device=dev)
    v_tok = torch.empty((wk.B, wk.k + 1), dtype=torch.int32, device=dev)
    # drafts with the workload's agreement rate against the target's argmax
    # (taken from one untimed verify call; the timed calls only read them)
    # gathered drafts: one sorted id list of C candidates per draft call, each
    # from its own seed, so no call re-reads rows the previous one cached
    gather_ids = [up(wl.candidate_ids(wk.V, wk.C, wk.seed + 1000 * (c + 1)), np.int32)
                  for c in range(wk.draft_calls)] if gather else None

    def draft_call(c, table):
        if fp8 and gather:
            mtp.mtp_draft_argmax_fp8_gather(h_d[c], table[0], table[1], gather_ids[c],
                                            out_ids[c], out_logit[c], ws=ws_d)
        elif fp4 and gather:
            mtp.mtp_draft_argmax_mxfp4_gather(h_d[c], table[0], table[1], gather_ids[c],
                                              out_ids[c], out_logit[c], ws=ws_d)
        elif fp4 and layout == "tiled":
            mtp.mtp_draft_argmax_tiled_mxfp4(h_d[c], table[0], table[1], wk.C, ids_d, out_ids[c],
                                             out_logit[c], ws=ws_d)
        elif fp4:
            mtp.mtp_draft_argmax_mxfp4(h_d[c], table[0], table[1], ids_d, out_ids[c],
                                       out_logit[c], ws=ws_d)
        elif fp8 and layout == "rows":
            mtp.mtp_draft_argmax_fp8(h_d[c], table[0], table[1], ids_d, out_ids[c], out_logit[c],
                                     ws=ws_d)
        elif fp8:
            mtp.mtp_draft_argmax_tiled_fp8(h_d[c], table[0], table[1], wk.C, ids_d, out_ids[c],
                                           out_logit[c], ws=ws_d)
        elif gather:
            mtp.mtp_draft_argmax_gather(h_d[c], head_d, gather_ids[c], out_ids[c], out_logit[c],
                                        ws=ws_d)
        elif layout == "rows":
            mtp.mtp_draft_argmax(h_d[c], table, ids_d, out_ids[c], out_logit[c], ws=ws_d)
        else:
            mtp.mtp_draft_argmax_tiled(h_d[c], table, wk.C, ids_d, out_ids[c], out_logit[c],
                                       ws=ws_d)

    def verify_call(drafts_dev):
        if layout == "rows":
            mtp.mtp_verify_accept(hv_d, head_v, drafts_dev, wk.B, wk.k, v_arg, v_acc, v_tok,
                                  v_logit, ws=ws_v)
        else:
            mtp.mtp_verify_accept_tiled(hv_d, head_v, wk.V, drafts_dev, wk.B, wk.k, v_arg, v_acc,
                                        v_tok, v_logit, ws=ws_v)

    zero_d = torch.zeros((wk.B, wk.k), dtype=torch.int32, device=dev)
    verify_call(zero_d)
    torch.cuda.synchronize()
    t_now = v_arg.cpu().numpy()
    if wk.p is None:
        drafts = wl.uniform_drafts(wk.B, wk.k, ids, wk.seed)
    else:
        drafts = wl.select_drafts(t_now, wl.agreement_draws(wk.B, wk.k, wk.p, wk.C, wk.seed), ids)
    drafts_d = up(drafts, np.int32)
    setup_s = time.time() - t0

    n_tab = len(tables)

    def step(i: int, ev=None):
        # ev: one event per call, the draft calls' then the verify's, which the
        # library stamps with the end of the call's last kernel
        # (mtp_time_next_call with a stop event only)
        for c in range(wk.draft_calls):
            if ev is not None:
                mtp.mtp_time_next_call(None, ev[c])
            draft_call(c, tables[(i * wk.draft_calls + c) % n_tab])
        if ev is not None:
            mtp.mtp_time_next_call(None, ev[-1])
        verify_call(drafts_d)

    # Warm-up: the --warmup steps, then more untimed steps until the warm-up
    # has lasted --warmup-seconds. A short timed region started right after
    # set-up (host uploads, packing, one synchronising verify call) otherwise
    # runs while the GPU is still raising its clocks.
    t_w = time.perf_counter()
    n_warm = 0
    for i in range(args.warmup):
        step(i)
        n_warm += 1
    torch.cuda.synchronize()
    while time.perf_counter() - t_w < args.warmup_seconds:
        for _ in range(20):
            step(n_warm)
            n_warm += 1
        torch.cuda.synchronize()
    warmup_s = time.perf_counter() - t_w

    K = args.steps
    graphs = []
    if args.graph:
        # step i reads table copies (i * draft_calls + c) % n_tab: one graph
        # per phase i % n_tab
        for ph in range(n_tab):
            g = mtp.Graph()
            g.begin()
            step(ph)
            g.end()
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % n_tab].launch()
        torch.cuda.synchronize()

    # Per-call timing: the library launches each call's last kernel with a stop
    # event (hipExtLaunchKernel), which takes that dispatch's own end time; a
    # call's time is the span from the previous call's end to its own end (its
    # kernels plus the bubble before them). Stop stamps cost the stream about
    # 0.6 us per call, against about 5 us for a start stamp or 7 us for a
    # marker event, so every timed step carries them.
    every = 1

    def timed_steps(with_events: bool, use_graph: bool):
        E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
        if use_graph:
            # graph replays: one event pair around each replay
            evs = {i: (E(), E()) for i in range(0, K, every)} if with_events else {}
        else:
            steps_ev = list(range(K)) if with_events else []
            pool = iter(mtp.timing_events((wk.draft_calls + 1) * len(steps_ev), stream))
            evs = {i: [next(pool) for _ in range(wk.draft_calls + 1)] for i in steps_ev}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            ev = evs.get(i)
            if use_graph:
                if ev:
                    ev[0].record(stream)
                graphs[i % n_tab].launch()
                if ev:
                    ev[1].record(stream)
            else:
                step(i, ev)
        torch.cuda.synchronize()
        return time.perf_counter() - t0, list(evs.values())

    t_total, evs = timed_steps(True, bool(graphs))
    graph_step_ms = None
    if graphs:
        graph_step_ms = [e[0].elapsed_time(e[1]) for e in evs]
        # per-call durations: the same calls launched eagerly, each timed by
        # its own event pair
        _, evs = timed_steps(True, False)

    # per-call durations: from the previous call's end to the call's end (the
    # very first call of the timed steps has no previous stamp); the draft
    # figure of a step is the mean of its draft calls
    stops = [ev for e in evs for ev in e]
    span = [None] + [mtp.elapsed_ms(stops[j - 1], stops[j]) for j in range(1, len(stops))]
    n_call = wk.draft_calls + 1
    draft_ms, verify_ms = [], []
    for i in range(len(evs)):
        d = [span[i * n_call + c] for c in range(wk.draft_calls) if span[i * n_call + c] is not None]
        if d:
            draft_ms.append(statistics.mean(d))
        verify_ms.append(span[i * n_call + wk.draft_calls])

    # Untimed context: the same steps without per-launch events, and the
    # draft call re-reading one table (Infinity Cache may serve part of it).
    t_noev, _ = timed_steps(False, bool(graphs))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        draft_call(0, tables[0])
    e1.record(stream)
    torch.cuda.synchronize()
    warm_draft_us = e0.elapsed_time(e1) * 1000.0 / K

    # Untimed context: isolated single calls (the device idle before each),
    # and the read rate a plain streaming read reaches over buffers of each
    # call's weight size (the practical ceiling of these HBM-bound calls).
    def one_call_us(fn, reps=15):
        out = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1000.0)
        return round(statistics.median(out), 2)

    single_draft_us = one_call_us(lambda: draft_call(0, tables[0]))
    single_verify_us = one_call_us(lambda: verify_call(drafts_d))
    sink = torch.empty(mtp.MTP_STREAM_SINK_WORDS, dtype=torch.int32, device=dev)

    def stream_gbps(bufs, nbytes, reps):
        # untimed reads first: the single calls above left the device idle
        for i in range(reps):
            mtp.mtp_stream_read(bufs[i % len(bufs)], sink, nbytes)
        e0.record(stream)
        for i in range(reps):
            mtp.mtp_stream_read(bufs[i % len(bufs)], sink, nbytes)
        e1.record(stream)
        torch.cuda.synchronize()
        return round(nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)

    tab_bufs = [t[0] if isinstance(t, tuple) else t for t in tables]
    tab_bytes = min(b.numel() * b.element_size() for b in tab_bufs)
    head_bytes = head_v.numel() * head_v.element_size()
    stream_read = {"draft_table_bytes": int(tab_bytes),
                   "draft_table_GBps": stream_gbps(tab_bufs, tab_bytes, 60),
                   "head_bytes": int(head_bytes),
                   "head_GBps": stream_gbps([head_v], head_bytes, 20)}

    # Atomic round trip (the unit the cross-workgroup finish repeats three or
    # four times at the end of every call): chains of dependent agent-scope
    # fetch-and-adds, one lane per workgroup, alone, in one workgroup per CU
    # on their own lines, and in one workgroup per CU on one line.
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    words = torch.zeros(64 * cus, dtype=torch.int32, device=dev)
    ticks = torch.zeros(cus, dtype=torch.int64, device=dev)

    def round_trip_us(wgs, same, iters=64, reps=5):
        per = []
        for _ in range(reps):
            mtp.mtp_probe_atomic(words, ticks, wgs, iters, same)
            torch.cuda.synchronize()
            t = (ticks[:wgs].cpu() & ((1 << 63) - 1)).tolist()
            per.append(statistics.median(t) / iters / 100.0)
        return round(statistics.median(per), 3)

    atomic_round_trip = {"alone_us": round_trip_us(1, False),
                         "one_wg_per_cu_own_lines_us": round_trip_us(cus, False),
                         "one_wg_per_cu_one_line_us": round_trip_us(cus, True, iters=16),
                         "method": "median over workgroups of one lane's chain of dependent "
                                   "agent-scope fetch-and-adds (mtp_probe_atomic), in 100 MHz "
                                   "real-time counter ticks, median of 5 launches"}

    # Draft-head ablation (workloads that list table sizes): the same M = 1
    # draft over each table, plus the pages' per-rank shard shape as context.
    draft_tables = None
    if wk.tables:
        draft_tables = draft_table_ablation(wk, mtp, wl, head_d, dev, up, sink, stream,
                                            fmt=args.table, mx_rule=mx_rule)

    # Acceptance of the last timed verify call (the GPU's own outputs): the
    # share of drafts accepted, and tokens emitted per verify (accepted drafts
    # plus the bonus token).
    torch.cuda.synchronize()
    g_verify = {"argmax": v_arg.cpu().numpy(), "logit": v_logit.cpu().numpy(),
                "accept": v_acc.cpu().numpy(), "tokens": v_tok.cpu().numpy()}
    g_drafts = [(out_ids[c].cpu().numpy(), out_logit[c].cpu().numpy())
                for c in range(wk.draft_calls)]
    acceptance = {
        "rate": round(float(g_verify["accept"].sum()) / (wk.B * wk.k), 4) if wk.k else None,
        "mean_emitted_per_verify": round(float((g_verify["accept"] + 1).sum()) / wk.B, 4),
        "drafts_per_sequence": wk.k,
    }

    agreement = None
    if fp8 or fp4:
        # how often the quantised draft picks the bf16 draft's token (512
        # hidden rows of the workload's distribution; untimed)
        n_rows = max(1, min(args.agree_rows, 4096))
        hx = up(wl.hidden_states(n_rows, wk.H, wk.seed, block=900))
        t16 = torch.empty((wk.C, wk.H), dtype=torch.int16, device=dev)
        mtp.mtp_pack_candidates(head_d, ids_d, t16)
        a8 = torch.empty(n_rows, dtype=torch.int32, device=dev)
        a16 = torch.empty(n_rows, dtype=torch.int32, device=dev)
        ws_x = mtp.alloc_workspace(mtp.mtp_draft_workspace_bytes(n_rows, wk.C, wk.H), dev)
        if fp8 and gather:
            mtp.mtp_draft_argmax_fp8_gather(hx, tables[0][0], tables[0][1], gather_ids[0], a8,
                                            ws=ws_x)
        elif fp4 and gather:
            mtp.mtp_draft_argmax_mxfp4_gather(hx, tables[0][0], tables[0][1], gather_ids[0], a8,
                                              ws=ws_x)
        elif fp4 and layout == "tiled":
            mtp.mtp_draft_argmax_tiled_mxfp4(hx, tables[0][0], tables[0][1], wk.C, ids_d, a8,
                                             ws=ws_x)
        elif fp4:
            mtp.mtp_draft_argmax_mxfp4(hx, tables[0][0], tables[0][1], ids_d, a8, ws=ws_x)
        elif layout == "rows":
            mtp.mtp_draft_argmax_fp8(hx, tables[0][0], tables[0][1], ids_d, a8, ws=ws_x)
        else:
            mtp.mtp_draft_argmax_tiled_fp8(hx, tables[0][0], tables[0][1], wk.C, ids_d, a8,
                                           ws=ws_x)
        if gather:
            mtp.mtp_draft_argmax_gather(hx, head_d, gather_ids[0], a16)
        else:
            mtp.mtp_draft_argmax(hx, t16, ids_d, a16)
        agreement = round(float((a8 == a16).float().mean().item()), 4)
        del t16

    H, C, V, Md, Mv = wk.H, wk.C, wk.V, wk.Md, wk.Mv
    # algorithmic bytes: weight rows + hidden rows + small outputs (winner ids,
    # logits; verify also reads drafts and writes acceptance)
    if fp4:
        # codes (half a byte per element) + one scale byte per 32 elements
        # (+ the id list when gathered)
        draft_bytes = C * H // 2 + C * H // 32 + Md * H * 2 + Md * (4 + 4 + 4) + \
            (C * 4 if gather else 0)
    elif fp8:
        # codes + one scale per row (+ the id list when gathered)
        draft_bytes = C * H + C * 4 + Md * H * 2 + Md * (4 + 4 + 4) + (C * 4 if gather else 0)
    else:
        draft_bytes = C * H * 2 + Md * H * 2 + Md * (4 + 4 + 4) + (C * 4 if gather else 0)
    verify_bytes = V * H * 2 + Mv * H * 2 + wk.B * wk.k * 4 + Mv * (4 + 4 + 4) + wk.B * 4
    d_us = statistics.mean(draft_ms) * 1000.0
    v_us = statistics.mean(verify_ms) * 1000.0
    calls_per_step = wk.draft_calls + 1
    value = calls_per_step * K / t_total

    def stats(ms, nbytes):
        us = [m * 1000.0 for m in ms]
        mean = statistics.mean(us)
        q = np.percentile(us, [10, 50, 90])
        return {"us_mean": round(mean, 2), "us_p10": round(float(q[0]), 2),
                "us_p50": round(float(q[1]), 2), "us_p90": round(float(q[2]), 2),
                "calls_per_s": round(1e6 / mean, 1), "bytes": int(nbytes),
                "GBps": round(nbytes / mean / 1e3, 1),
                "frac_peak": round(nbytes / mean / 1e3 / HBM_PEAK_GBPS, 4)}

    draft_stats = stats(draft_ms, draft_bytes)
    verify_stats = stats(verify_ms, verify_bytes)
    # dominant kernel of the step: the one with more time per step
    if v_us >= d_us * wk.draft_calls:
        dom_name, dom_bytes, dom_us = "verify", verify_bytes, v_us
    else:
        dom_name, dom_bytes, dom_us = "draft", draft_bytes, d_us
    # row-major calls with few rows run on the vector-ALU kernel; tiled ones
    # on the DMA-fed matrix-core kernel
    dom_rows = wk.Mv if dom_name == "verify" else wk.Md
    path = "dma" if layout == "tiled" else rows_path(dom_rows, wk.H)
    # counter summaries: one per workload in its default layout, plus the
    # row-major runs of the batched workloads
    default_layout = "rows" if max(wk.Md, wk.Mv) <= 8 else "tiled"
    profile = wk.name if layout == default_layout else f"{wk.name}_{layout}"
    traffic = measured_traffic(dom_name, profile, path) if args.table == "bf16" and \
        args.draft_source == "table" else None
    achieved = dom_bytes / dom_us / 1e3
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": traffic, "kernel": dom_name, "kernel_family": path,
                "kernel_source_hash": kernel_source_hash(path),
                "algorithmic_bytes_per_launch": int(dom_bytes)}

    dom_stream = stream_read["head_GBps"] if dom_name == "verify" else \
        stream_read["draft_table_GBps"]
    stream_read["dominant_kernel_frac_of_stream_read"] = round(achieved / dom_stream, 4)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(t_total * 1000.0 / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8-e4m3 draft rows, bf16 hidden and head" if fp8 else
                  "mxfp4 draft rows (e2m1, e8m0 block scales), bf16 hidden and head" if fp4
                  else "bf16"),
        "data": "synthetic",
        "config": {
            "workload": f"{wk.name}: {wk.draft_calls} draft calls (M={Md}, {C}-row table) + 1 "
                        f"verify call (M={Mv}, {V}-row head), H={H}",
            "H": H, "V": V, "C": C, "B": wk.B, "k": wk.k, "draft_calls": wk.draft_calls,
            "accumulate": "f32", "table_copies": n_tab, "seed": wk.seed, "layout": layout,
            "step": "hip_graph" if graphs else "eager",
            "draft_source": args.draft_source,
            "draft_table": args.table,
            "mx_scale": args.mx_scale if fp4 else None,
        },
        "calls": {"draft": draft_stats, "verify": verify_stats},
        "context": {
            "ms_per_step_without_kernel_events": round(t_noev * 1000.0 / K, 4),
            "kernel_event_steps": f"every timed step ({len(evs)} of {K}); one stop event per "
                                  "call, stamped with the end of the call's last kernel; a call's "
                                  "time runs from the previous call's end to its own",
            "warmup_steps_run": n_warm,
            "warmup_s": round(warmup_s, 3),
            "step_mode": "hip_graph" if graphs else "eager",
            "graph_step_us_mean": round(statistics.mean(graph_step_ms) * 1000.0, 2)
            if graph_step_ms else None,
            "draft_same_table_us": round(warm_draft_us, 2),
            "single_call_us": {"draft": single_draft_us, "verify": single_verify_us},
            "stream_read": stream_read,
            "atomic_round_trip": atomic_round_trip,
            "acceptance": acceptance,
            "quantised_draft_agrees_with_bf16": agreement,
            "agreement_rows": (max(1, min(args.agree_rows, 4096)) if (fp8 or fp4) else None),
            "draft_tables": draft_tables,
            "setup_s": round(setup_s, 1),
        },
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"], orc = cpu_baseline(wk, head, ids, hiddens, hv, drafts,
                                                   args.cpu_seconds)
        # the oracle's outputs for the same inputs, against the GPU's outputs
        # of the last timed step
        lists = [wl.candidate_ids(wk.V, wk.C, wk.seed + 1000 * (c + 1))
                 for c in range(wk.draft_calls)] if gather else None
        result["parity"] = oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g_drafts,
                                         g_verify, args.table, lists, args.mx_scale)
    print(json.dumps(result), flush=True)
    return 0


def draft_table_ablation(wk, mtp, wl, head_d, dev, up, sink, stream, reps=200, copies=3,
                         fmt="bf16", mx_rule=0):
    """M = 1 draft calls over each table size of the ablation: the full head
    (identity ids), the 65,536-row subset and the nested 32,768-row subset,
    all at the workload's width, plus 32,768 rows x 2,560 (the pages' per-rank
    draft shard, drawn as its own rows: no head of that width exists here).

    Each size is packed ``copies`` times and the calls rotate over the copies,
    so no call is served from the Infinity Cache its predecessor filled. One
    event pair brackets ``reps`` back-to-back calls, so the time per call
    includes the gaps between launches. The streaming-read probe over the same
    bytes gives the practical read ceiling for each size. fmt "fp8" / "mxfp4":
    the same tables quantised by the library's pack, drafted by the fp8 /
    MXFP4 kernel.
    """
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    shapes = [(n, wk.H) for n in wk.tables] + [(32_768, 2_560)]
    out = []
    for n, H in shapes:
        if H == wk.H:
            ids = (np.arange(wk.V, dtype=np.int32) if n == wk.V
                   else wl.candidate_ids(wk.V, n, wk.seed))
            ids_d = up(ids, np.int32)
            src, src_ids = head_d, ids_d
        else:
            ids_d = up(wl.candidate_ids(wk.V, n, wk.seed), np.int32)
            src, src_ids = up(wl.head_weights(n, H, wk.seed + 1)), None
        tabs = []
        for _ in range(copies):
            if fmt == "fp8":
                t = (torch.empty((n, H), dtype=torch.uint8, device=dev),
                     torch.empty(n, dtype=torch.float32, device=dev))
                mtp.mtp_pack_candidates_fp8(src, src_ids, t[0], t[1], C=n)
            elif fmt == "mxfp4":
                t = (torch.empty((n, H // 2), dtype=torch.uint8, device=dev),
                     torch.empty((n, H // 32), dtype=torch.uint8, device=dev))
                mtp.mtp_pack_candidates_mxfp4(src, src_ids, t[0], t[1], C=n, rule=mx_rule)
            elif src_ids is None:
                t = src.clone()
            else:
                t = torch.empty((n, H), dtype=torch.int16, device=dev)
                mtp.mtp_pack_candidates(src, src_ids, t)
            tabs.append(t)
        h = up(wl.hidden_states(1, H, wk.seed, block=0))
        oid = torch.empty(1, dtype=torch.int32, device=dev)
        olog = torch.empty(1, dtype=torch.float32, device=dev)
        ws = mtp.alloc_workspace(mtp.mtp_draft_workspace_bytes(1, n, H), dev)
        def call(i):
            t = tabs[i % copies]
            if fmt == "fp8":
                mtp.mtp_draft_argmax_fp8(h, t[0], t[1], ids_d, oid, olog, ws=ws)
            elif fmt == "mxfp4":
                mtp.mtp_draft_argmax_mxfp4(h, t[0], t[1], ids_d, oid, olog, ws=ws)
            else:
                mtp.mtp_draft_argmax(h, t, ids_d, oid, olog, ws=ws)

        for i in range(20):
            call(i)
        e0.record(stream)
        for i in range(reps):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / reps
        if fmt == "fp8":
            tab_bytes = n * H + n * 4
        elif fmt == "mxfp4":
            tab_bytes = n * H // 2 + n * H // 32
        else:
            tab_bytes = n * H * 2
        nbytes = tab_bytes + H * 2 + 12
        # the streaming-read probe over the codes (the larger buffer)
        rbufs = [t[0] if isinstance(t, tuple) else t for t in tabs]
        rbytes = rbufs[0].numel() * rbufs[0].element_size()
        for i in range(reps):
            mtp.mtp_stream_read(rbufs[i % copies], sink, rbytes)
        e0.record(stream)
        for i in range(reps):
            mtp.mtp_stream_read(rbufs[i % copies], sink, rbytes)
        e1.record(stream)
        torch.cuda.synchronize()
        sr_gbps = rbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        gbps = nbytes / us / 1e3
        out.append({"rows": n, "H": H, "table": fmt, "bytes": int(nbytes),
                    "us_per_call": round(us, 2),
                    "calls_per_s": round(1e6 / us, 1), "GBps": round(gbps, 1),
                    "frac_peak": round(gbps / HBM_PEAK_GBPS, 4),
                    "stream_read_GBps": round(sr_gbps, 1),
                    "frac_of_stream_read": round(gbps / sr_gbps, 4),
                    "note": "pages' per-rank shard shape (context)" if H != wk.H else
                            ("full head, identity ids" if n == wk.V else "candidate subset")})
        del tabs
    return out


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wk, head, ids, hiddens, hv, drafts, budget_s):
    """The CPU oracle on the same step: its draft calls and verify call,
    repeated until the time budget is spent (at least once)."""
    import oracle
    table = oracle.pack(head, ids)
    times, draft_s, verify_s = [], [], []
    first = None
    t_begin = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        outs = []
        for h in hiddens:
            t1 = time.perf_counter()
            outs.append(oracle.draft(h, table, ids))
            draft_s.append(time.perf_counter() - t1)
        t1 = time.perf_counter()
        v = oracle.verify(hv, head, wk.B, wk.k, drafts)
        verify_s.append(time.perf_counter() - t1)
        if first is None:
            first = {"drafts": outs, "verify": v, "table": table}
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_begin >= budget_s:
            break
    step_s = statistics.median(times)
    return {"value": round((wk.draft_calls + 1) / step_s, 3), "unit": "calls/s",
            "cores": oracle.threads(), "cpu_model": cpu_model(), "kind": "oracle",
            "draft_ms_median": round(statistics.median(draft_s) * 1e3, 3),
            "verify_ms_median": round(statistics.median(verify_s) * 1e3, 3),
            "sample": f"{len(times)} full {wk.name} step(s) ({wk.draft_calls} draft + 1 verify "
                      f"call), median {step_s:.3f} s per step"}, first


def oracle_parity(wk, head, ids, hiddens, hv, drafts, orc, g_drafts, g_verify, table="bf16",
                  gather_lists=None, mx_scale="ocp"):
    """The GPU outputs of the last timed step against the oracle's outputs for
    the same inputs. A pick passes if it equals the oracle's, or if the row is a
    near tie (oracle runner-up within 1e-3 x |max| of the max) and the pick
    scores at least max - 1e-3 x |max| under the oracle; its logit must be
    within 2e-3 x |oracle logit of the pick|. Acceptance must equal the
    oracle's acceptance of the GPU's verify argmax. Draft logits are the
    table's own: bf16, or the oracle's fp8 / MXFP4 quantisation of the same
    rows; gathered drafts (gather_lists: each call's id list) take the
    candidate set of their list."""
    import oracle

    def rows(gpu_ids, gpu_logit, ref, pick_logit):
        rep = {"rows": int(len(gpu_ids)), "exact": 0, "near_tie_rows": 0, "near_tie_diff": 0,
               "violations": 0, "max_logit_rel": 0.0}
        for m in range(len(gpu_ids)):
            g = int(gpu_ids[m])
            top, runner = float(ref["exact"][m]), float(ref["runner_exact"][m])
            tol = 1e-3 * abs(top)
            near = runner >= top - tol
            rep["near_tie_rows"] += int(near)
            if g == int(ref["id"][m]):
                rep["exact"] += 1
                zg = top
            else:
                zg = pick_logit(m, g)
                if zg is None or not (near and zg >= top - tol):
                    rep["violations"] += 1
                    continue
                rep["near_tie_diff"] += 1
            rel = abs(float(gpu_logit[m]) - zg) / max(abs(zg), 1e-30)
            rep["max_logit_rel"] = max(rep["max_logit_rel"], rel)
            if rel > 2e-3:
                rep["violations"] += 1
        rep["max_logit_rel"] = float(f"{rep['max_logit_rel']:.3g}")
        return rep

    def position(row_ids, g):
        """Index of id g in the sorted id list row_ids (None: not there)."""
        k = int(np.searchsorted(row_ids, g))
        return k if k < len(row_ids) and int(row_ids[k]) == g else None

    def draft_check(c, h):
        """Oracle result and pick-logit function of draft call c."""
        if gather_lists is not None:
            lst = np.asarray(gather_lists[c])
            rows_ = np.unique(lst[(lst >= 0) & (lst < wk.V)]).astype(np.int32)
        else:
            rows_ = np.asarray(ids, np.int32)
        if table == "bf16":
            w = orc["table"] if gather_lists is None else oracle.pack(head, rows_)
            ref = oracle.draft(h, w, rows_)

            def pick(m, g):
                k = position(rows_, g)
                return None if k is None else \
                    float(oracle.pair_logits(h, w, np.array([m]), np.array([k]))[0])
        elif table == "fp8":
            q, e = quant["fp8"]
            q, e = (q, e) if gather_lists is None else (q[rows_], e[rows_])
            ref = oracle.draft_fp8(h, q, e, rows_)

            def pick(m, g):
                k = position(rows_, g)
                return None if k is None else \
                    float(oracle.draft_fp8(h[m:m + 1], q[k:k + 1], e[k:k + 1])["exact"][0])
        else:
            q, sc = quant["mxfp4"]
            q, sc = (q, sc) if gather_lists is None else (q[rows_], sc[rows_])
            ref = oracle.draft_mxfp4(h, q, sc, rows_)

            def pick(m, g):
                k = position(rows_, g)
                return None if k is None else \
                    float(oracle.draft_mxfp4(h[m:m + 1], q[k:k + 1], sc[k:k + 1])["exact"][0])
        return ref, pick

    # the oracle's quantisation of the drafted rows (the whole head when gathered)
    quant = {}
    if table == "fp8":
        quant["fp8"] = oracle.quantize_fp8(head, None if gather_lists is not None else ids)
    elif table == "mxfp4":
        quant["mxfp4"] = oracle.quantize_mxfp4(head, None if gather_lists is not None else ids,
                                               rule=mx_scale)

    out = {"rule": "ids equal, or a pick within 1e-3 relative of the max in a near-tie row; "
                   "logits within 2e-3 relative; acceptance equal to the oracle's on the "
                   "GPU argmax",
           "draft_table": table, "draft_source": "gather" if gather_lists is not None else "table"}
    d = {"rows": 0, "exact": 0, "near_tie_rows": 0, "near_tie_diff": 0, "violations": 0,
         "max_logit_rel": 0.0}
    for c, ((gi, gl), h) in enumerate(zip(g_drafts, hiddens)):
        ref, pick = draft_check(c, h)
        r = rows(gi, gl, ref, pick)
        for key in ("rows", "exact", "near_tie_rows", "near_tie_diff", "violations"):
            d[key] += r[key]
        d["max_logit_rel"] = max(d["max_logit_rel"], r["max_logit_rel"])
    out["draft"] = d
    ref = {key: np.asarray(v).reshape(-1) for key, v in orc["verify"].items()
           if key in ("id", "exact", "runner_exact")}
    out["verify"] = rows(g_verify["argmax"].reshape(-1), g_verify["logit"].reshape(-1), ref,
                         lambda m, g: float(oracle.pair_logits(hv, head, np.array([m]),
                                                               np.array([g]))[0])
                         if 0 <= g < wk.V else None)
    exp = oracle.accept(np.asarray(drafts, np.int32).reshape(wk.B, wk.k),
                        g_verify["argmax"].reshape(wk.B, wk.k + 1))
    out["accept_equal"] = bool(np.array_equal(g_verify["accept"].reshape(-1), exp["accept"]) and
                               np.array_equal(g_verify["tokens"].reshape(wk.B, wk.k + 1),
                                              exp["tokens"]))
    out["ok"] = bool(out["accept_equal"] and out["verify"]["violations"] == 0 and
                     out["draft"]["violations"] == 0)
    return out


if __name__ == "__main__":
    sys.exit(main())
