#!/usr/bin/env python3
"""Benchmark of the per-decode-step KV recall path on one MI355X.

A step is one pass of the whole path over one batch: Stage One (probe,
refresh, classify, allocate, link, invalidate) for every request and query
token, then the zero-copy gather of every missed row from pinned host memory
into the device slot buffer.  The default workload is MTP-3, the largest configuration
(batch 16, 4 query tokens per iteration through one shared buffer, context
100000, K = 2048, S = 8192, 1280-byte rows, 131072 lookups per step); its
32 seeded iterations are run in order from an empty buffer (warm-up steps
first, then the timed ones), and a run asking for more than 32 is refused.
Other workloads generate as many distinct steps as the run needs.

Inputs are resident in HBM (selections) and in pinned host memory (the KV
pool, which is where the method keeps it) before the timed region starts.
The headline step latency is the wall time of one replay of a HIP graph
that holds the K timed steps (Stage One + gather each, on that step's
inputs), bracketed by device synchronisation, divided by K: the recall as it
runs inside a captured decode step, where the graph's launch is paid once.
A second pass replays one graph per step; events between those replays give
the per-step spread, and their wall time per step is reported beside the
headline.  A first, eager
pass with an event between the two kernels gives the per-kernel times, the
gather bandwidth and the counters.  A third pass runs Stage One alone, its
launches back to back between two events, for the match rate.  The CPU
oracle is timed on the host cores beside it.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "recall-step latency (us) + effective host->HBM gather GB/s; match Mkeys/s"
PCIE_GEN5_X16_GBPS = 64.0   # published per-direction peak of the host link
HBM_PEAK_GBPS = 8000.0      # MI355X HBM3E


CSRC = os.path.join(ROOT, "recall_step_amd", "csrc")
# The sources each kernel's code comes from: a counter summary is only
# reported while these hash to the value it was taken on.
KERNEL_SOURCES = {"gather_kernel": ("gather.hip", "gather.h"),
                  "stage1_kernel": ("stage_one.hip", "internal.h")}


def source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def profiled_traffic(kernel, workload, key="traffic_bytes_per_launch"):
    """HBM-side bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 PMC summary profiles/<kernel>.<workload>.pmc.txt (FETCH_SIZE and
    WRITE_SIZE, each scaled by what it reads for a plain copy of known size),
    or None when there is no summary or it was taken on other sources.  `key`
    names the figure (the probe sweep's summary holds one per batch size)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line:
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
    recorded = fields.get("source_sha256_16", fields.get("gather_source_sha256_16"))
    if recorded != source_hash(kernel):
        return None
    try:
        return int(fields[key])
    except (KeyError, ValueError):
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=24)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="mtp3",
                    choices=["tiny", "matching", "residency", "mtp3", "imbalanced"])
    ap.add_argument("--gather-blocks", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--stage1-threads", type=int, default=0)
    ap.add_argument("--ratios", action="store_true",
                    help="instead of the step benchmark: the comparison points the "
                         "pages measure against (gather partitions at B=1/25%% and "
                         "B=8/75%% reuse; no-reuse KV Offload on the matching "
                         "workload), one JSON line each")
    ap.add_argument("--layers", type=int, default=0,
                    help="instead of the step benchmark: N layers of the matching "
                         "workload, each with its own cache, stepped (a) layer by "
                         "layer, (b) as one batched launch per stage, (c) with layer "
                         "l+1's matching overlapping layer l's gather on a second stream")
    ap.add_argument("--transfer-sweep", action="store_true",
                    help="instead of the step benchmark: effective host-to-HBM "
                         "bandwidth against row size, zero-copy gather vs one "
                         "hipMemcpyAsync per row vs one bulk copy")
    ap.add_argument("--prefetch", action="store_true",
                    help="instead of the step benchmark: threshold prefetch (ECHO) on "
                         "scored selections: the recall left on the critical path after "
                         "the exact top-K is known, with and without the prefetch")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="instead of the step benchmark: Stage-One latency of one request "
                         "(75%% adjacent reuse) over K in 256..2048 and S in 512..8192")
    ap.add_argument("--lifetime-sweep", action="store_true",
                    help="instead of the step benchmark: hit rate and Stage-One latency "
                         "of the residency shape against the lifetime L")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="instead of the step benchmark: Stage-One throughput on the "
                         "residency request shape (K=2048, S=8192) at B = 32..1024, "
                         "one JSON line per batch size")
    ap.add_argument("--batch", type=int, action="append",
                    help="with --probe-sweep: only these batch sizes (repeatable)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="with --probe-sweep: end with one device copy of exactly "
                         "1 GiB, the reference a counter run scales its byte "
                         "counters by")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    return args


def hip_runtime():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    hip.hipMemcpyAsync.restype = ctypes.c_int
    return hip


def pinned_h2d_peak(r, torch, stream, nbytes=1 << 30, reps=10):
    """Best-of-N pinned hipMemcpyAsync host->device rate, GB/s."""
    hip = hip_runtime()
    pool = r.HostPool(nbytes)
    pool.array[:] = 1
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    best = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = hip.hipMemcpyAsync(dst.data_ptr(), pool.ptr, nbytes, 1, stream.cuda_stream)
        assert rc == 0, rc
        e1.record(stream)
        e1.synchronize()
        best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del dst
    pool.close()
    return best


def hbm_copy_peak(torch, stream, nbytes=1 << 30, reps=5):
    """Best-of-N device-to-device copy of nbytes (torch's copy kernel), as
    HBM GB/s counting the read and the write."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    best = 0.0
    with torch.cuda.stream(stream):
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            e1.synchronize()
            best = max(best, 2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return best


STAGE1_BYTES_MODEL = ("algorithmic bytes of the method's state accesses, wherever "
                      "they are served: per request 2*S*4 B of lifetimes read and "
                      "written, per lookup 9 B (id in, slot out, mask out), per bucket "
                      "visited 8 B (word and cached id; staged in LDS here, so they do "
                      "not reach HBM), per miss 20 B (C, F, Q install and the miss "
                      "list entry), per token 4 B")


def stage1_algorithmic_bytes(B, S, Nq, lookups, visits, misses):
    """Stage-One algorithmic bytes of one step (see STAGE1_BYTES_MODEL):
    lifetimes read and written once per request (2*S*4 B), 4 B id in + 4 B
    slot out + 1 B mask out per lookup, 8 B (word + cached id) per bucket
    visited, 20 B per miss (install 12 B + miss list 8 B), 4 B count per
    token."""
    return B * 2 * S * 4 + lookups * 9 + visits * 8 + misses * 20 + B * Nq * 4


def probe_sweep(args):
    import torch
    import recall_step_amd as r
    from workloads import make

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    # The measured HBM stream peak (a 1 GiB device copy, read plus write),
    # beside the published one; and the counter-measured traffic of the
    # committed summary at each batch size it holds.
    copy_peak = hbm_copy_peak(torch, stream)
    for B in (args.batch or (32, 128, 256, 512, 1024)):
        counted = profiled_traffic("stage1_kernel", "probe-sweep",
                                   f"traffic_bytes_per_launch_B{B}")
        w = make("residency", steps=40, B=B)
        cfg = r.avsg_config_default(w.B, w.Nq, w.K, w.S, w.row_bytes, L=w.L, R=w.R,
                                    a1=w.a1, a2=w.a2, a_fp=w.afp, flags=r.FLAG_SKIP_GATHER,
                                    stage1_threads=args.stage1_threads)
        rs = r.RecallStep(cfg, None, w.host_rows_total, stream=stream)
        topk = torch.from_numpy(np.ascontiguousarray(w.topk)).cuda()
        ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len)).cuda()
        row_base = torch.from_numpy(w.row_base).cuda()
        host_rows = torch.from_numpy(w.host_rows).cuda()
        ios = [rs.io(topk[t], ctx[t], row_base, host_rows) for t in range(w.steps)]
        torch.cuda.synchronize()
        for t in range(8):
            r.avsg_match(rs.handle, ios[t], sh)
        torch.cuda.synchronize()
        cnt0 = rs.CNT.cpu().numpy().astype(np.int64)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        timed = w.steps - 8
        for t in range(8, w.steps):
            r.avsg_match(rs.handle, ios[t], sh)
        e1.record(stream)
        torch.cuda.synchronize()
        d = (rs.CNT.cpu().numpy().astype(np.int64) - cnt0).sum(0)
        us = e0.elapsed_time(e1) * 1e3 / timed
        per_step = stage1_algorithmic_bytes(B, w.S, w.Nq, d[r.CNT_LOOKUPS] / timed,
                                            d[r.CNT_PROBE_VISITS] / timed,
                                            d[r.CNT_MISSES] / timed)
        staged = B * (2 * 3 * w.S * 4 + w.Nq * w.K * 9)  # Q, C, F in and out + ids/outputs
        gbps = per_step / (us * 1e-6) / 1e9
        line = {
            "probe_sweep": "residency request shape, Stage One only",
            "B": B, "K": w.K, "S": w.S, "stage1_us": round(us, 2),
            "match_Mkeys_per_s": round(d[r.CNT_LOOKUPS] / timed / us, 1),
            "algorithmic_bytes_per_step": int(per_step), "bytes_model": STAGE1_BYTES_MODEL,
            "achieved_GBps": round(gbps, 1), "peak_GBps": HBM_PEAK_GBPS,
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "measured_copy_peak_GBps": round(copy_peak, 1),
            "frac_of_measured_peak": round(gbps / copy_peak, 4),
            "state_traffic_GBps": round(staged / (us * 1e-6) / 1e9, 1),
            "hit_rate": round(d[r.CNT_HITS] / d[r.CNT_LOOKUPS], 4)}
        if counted is not None:
            cg = counted / (us * 1e-6) / 1e9
            line["counter_traffic"] = {
                "bytes_per_launch": counted, "source": "profiles/stage1_kernel.probe-sweep.pmc.txt",
                "GBps": round(cg, 1), "frac": round(cg / HBM_PEAK_GBPS, 4),
                "frac_of_measured_peak": round(cg / copy_peak, 4)}
        print(json.dumps(line), flush=True)
        rs.close()
    if args.calibration_copy:
        log(f"[bench] calibration copy: 1 GiB device to device, "
            f"{hbm_copy_peak(torch, stream, reps=1):.0f} GB/s")
    return 0


def stage1_only(r, torch, stream, w, warmup, timed, L=None, B=None):
    """Stage One alone (no host pool) over w's steps: mean launch time from
    events around `timed` launches after `warmup`, and the counter deltas
    of the timed launches."""
    cfg = r.avsg_config_default(w.B, w.Nq, w.K, w.S, w.row_bytes,
                                L=w.L if L is None else L, R=w.R, a1=w.a1, a2=w.a2,
                                a_fp=w.afp, flags=r.FLAG_SKIP_GATHER)
    rs = r.RecallStep(cfg, None, w.host_rows_total, stream=stream)
    topk = torch.from_numpy(np.ascontiguousarray(w.topk)).cuda()
    ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len)).cuda()
    row_base = torch.from_numpy(w.row_base).cuda()
    host_rows = torch.from_numpy(w.host_rows).cuda()
    ios = [rs.io(topk[t], ctx[t], row_base, host_rows) for t in range(w.steps)]
    sh = stream.cuda_stream
    torch.cuda.synchronize()
    for t in range(warmup):
        r.avsg_match(rs.handle, ios[t % w.steps], sh)
    torch.cuda.synchronize()
    cnt0 = rs.CNT.cpu().numpy().astype(np.int64)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for k in range(timed):
        r.avsg_match(rs.handle, ios[(warmup + k) % w.steps], sh)
    e1.record(stream)
    torch.cuda.synchronize()
    d = (rs.CNT.cpu().numpy().astype(np.int64) - cnt0).sum(0)
    rs.close()
    return {"stage1_us": round(e0.elapsed_time(e1) * 1e3 / timed, 2),
            "hit_rate": round(d[r.CNT_HITS] / max(1, d[r.CNT_LOOKUPS]), 4),
            "lost_per_step": round((d[r.CNT_LOST_COLLISION] + d[r.CNT_LOST_EXHAUSTED]) / timed,
                                   1),
            "visits_per_lookup": round(d[r.CNT_PROBE_VISITS] / max(1, d[r.CNT_LOOKUPS]), 3)}


def shape_sweep(args):
    """Stage-One latency of one request against K and S (the in-kind
    analog of the AVSG page's matching-latency sweep, section 4.2)."""
    import torch
    import recall_step_amd as r
    from workloads.synth import gen_reuse

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    for S in (512, 1024, 2048, 4096, 8192):
        row = {}
        for K in (256, 512, 1024, 2048):
            if K > S:
                continue
            w = gen_reuse(1, 0.75, steps=16, K=K, S=S)
            row[str(K)] = stage1_only(r, torch, stream, w, 4, 12)
        print(json.dumps({"shape_sweep": "one request, 75% adjacent reuse, Stage One only",
                          "S": S, "by_K": {k: v["stage1_us"] for k, v in row.items()},
                          "hit_rate_by_K": {k: v["hit_rate"] for k, v in row.items()}}),
              flush=True)
    return 0


def lifetime_sweep(args):
    """Hit rate and Stage-One latency of the residency shape (B=8, K=2048,
    S=8192) against the lifetime L (the in-kind analog of the AVSG page's
    Appendix A)."""
    import torch
    import recall_step_amd as r
    from workloads import make

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    w = make("residency", steps=48, B=8)
    for L in (1, 3, 7, 15, 63, 127):
        res = stage1_only(r, torch, stream, w, 16, 32, L=L)
        print(json.dumps({"lifetime_sweep": "residency shape, B=8, steps 16..47",
                          "L": L, **res}), flush=True)
    return 0


def eager_steps(r, torch, stream, w, host, flags, warmup, steps):
    """Run warmup + steps recall steps with an event between Stage One and
    the gather; returns per-kernel means and the counter deltas.  The dense
    matcher gets a map of one entry per host row of the longest request."""
    cfg = r.avsg_config_default(w.B, w.Nq, w.K, w.S, w.row_bytes, L=w.L, R=w.R,
                                a1=w.a1, a2=w.a2, a_fp=w.afp, flags=flags)
    map_len = int(w.host_rows.max()) if flags & r.FLAG_DENSE_MAP else 0
    rs = r.RecallStep(cfg, host, w.host_rows_total, stream=stream, map_len=map_len)
    topk = torch.from_numpy(np.ascontiguousarray(w.topk)).cuda()
    ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len)).cuda()
    row_base = torch.from_numpy(w.row_base).cuda()
    host_rows = torch.from_numpy(w.host_rows).cuda()
    ios = [rs.io(topk[t], ctx[t], row_base, host_rows) for t in range(w.steps)]
    sh = stream.cuda_stream
    torch.cuda.synchronize()
    for t in range(warmup):
        r.avsg_step(rs.handle, ios[t % w.steps], sh)
    torch.cuda.synchronize()
    cnt0 = rs.CNT.cpu().numpy().astype(np.int64)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        io = ios[(warmup + k) % w.steps]
        ev[k][0].record(stream)
        r.avsg_match(rs.handle, io, sh)
        ev[k][1].record(stream)
        r.avsg_gather(rs.handle, io, sh)
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    d = (rs.CNT.cpu().numpy().astype(np.int64) - cnt0).sum(0)
    s1 = sum(e[0].elapsed_time(e[1]) for e in ev) * 1e3 / steps
    g = sum(e[1].elapsed_time(e[2]) for e in ev) * 1e3 / steps
    rs.close()
    misses = d[r.CNT_MISSES] / steps
    return {"stage1_us": round(s1, 2), "gather_us": round(g, 2),
            "step_us": round(s1 + g, 2), "rows_per_step": round(misses, 1),
            "gather_GBps": round(misses * w.row_bytes / (g * 1e-6) / 1e9, 2),
            "hit_rate": round(d[r.CNT_HITS] / max(1, d[r.CNT_LOOKUPS]), 4),
            "lost_per_step": round((d[r.CNT_LOST_COLLISION] + d[r.CNT_LOST_EXHAUSTED]) / steps,
                                   2)}


def ratios(args):
    """The pages' comparison points, measured in kind on this GPU:
    effective H2D bandwidth of the per-row split against request-level
    assignment (B=1, 25 % reuse) and against equal top-K partitions (B=8,
    75 % reuse), all three partitions under uneven misses per request (the
    imbalanced workload and a B=8 batch with reuse spread over 40-100 %),
    and the recall step without reuse (KV Offload) against the one with it
    on the matching workload."""
    import torch
    import recall_step_amd as r
    from workloads import make

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    parts = {"per_row": 0, "by_request": r.FLAG_GATHER_BY_REQUEST,
             "by_topk": r.FLAG_GATHER_BY_TOPK}
    for name, pct, other in (("reuse25_b1", 25, "by_request"), ("reuse75_b8", 75, "by_topk")):
        w = make(name)
        host = r.HostPool(w.host_bytes)
        w.fill_host_kv(host.array)
        res = {p: eager_steps(r, torch, stream, w, host, f, 4, 12) for p, f in parts.items()}
        host.close()
        print(json.dumps({
            "comparison": f"gather partition, {name} (B={w.B}, K={w.K}, S={w.S}, "
                          f"{pct}% adjacent reuse)",
            "effective_GBps": {p: v["gather_GBps"] for p, v in res.items()},
            "gather_us": {p: v["gather_us"] for p, v in res.items()},
            "rows_per_step": res["per_row"]["rows_per_step"],
            "hit_rate": res["per_row"]["hit_rate"],
            f"per_row_over_{other}": round(res["per_row"]["gather_GBps"] /
                                           res[other]["gather_GBps"], 2)}), flush=True)
    # Uneven misses per request, where the split by missed row should matter:
    # the imbalanced workload (64 requests, per-request miss rates 0-60 %) and
    # 8 requests whose adjacent-step reuse spreads evenly over 40-100 %.
    for name in ("imbalanced", "skew40to100_b8"):
        w = make(name, steps=16)
        host = r.HostPool(w.host_bytes)
        w.fill_host_kv(host.array)
        res = {p: eager_steps(r, torch, stream, w, host, f, 4, 12) for p, f in parts.items()}
        host.close()
        print(json.dumps({
            "comparison": f"gather partition, {name} (B={w.B}, K={w.K}, S={w.S}, uneven "
                          f"misses per request)",
            "effective_GBps": {p: v["gather_GBps"] for p, v in res.items()},
            "gather_us": {p: v["gather_us"] for p, v in res.items()},
            "rows_per_step": res["per_row"]["rows_per_step"],
            "hit_rate": res["per_row"]["hit_rate"],
            "per_row_over_by_request": round(res["per_row"]["gather_GBps"] /
                                             res["by_request"]["gather_GBps"], 2),
            "per_row_over_by_topk": round(res["per_row"]["gather_GBps"] /
                                          res["by_topk"]["gather_GBps"], 2)}), flush=True)
    w = make("matching")
    host = r.HostPool(w.host_bytes)
    w.fill_host_kv(host.array)
    reuse = eager_steps(r, torch, stream, w, host, 0, 4, 30)
    offload = eager_steps(r, torch, stream, w, host, r.FLAG_NO_REUSE, 4, 30)
    merge = eager_steps(r, torch, stream, w, host, r.FLAG_SORT_MERGE, 4, 30)
    dense = eager_steps(r, torch, stream, w, host, r.FLAG_DENSE_MAP, 4, 30)
    host.close()
    print(json.dumps({
        "comparison": "matching latency, hash probe vs sort-merge matcher, matching "
                      "workload (B=8, K=S=2048)",
        "hash_stage1_us": reuse["stage1_us"], "sort_merge_stage1_us": merge["stage1_us"],
        "sort_merge_over_hash": round(merge["stage1_us"] / reuse["stage1_us"], 2),
        "hash_hit_rate": reuse["hit_rate"], "sort_merge_hit_rate": merge["hit_rate"]}),
        flush=True)
    print(json.dumps({
        "comparison": "matching latency, hash probe vs dense id-to-slot map, matching "
                      "workload (B=8, K=S=2048, map of 65536 ids per request)",
        "hash_stage1_us": reuse["stage1_us"], "dense_stage1_us": dense["stage1_us"],
        "dense_over_hash": round(dense["stage1_us"] / reuse["stage1_us"], 2),
        "hash_hit_rate": reuse["hit_rate"], "dense_hit_rate": dense["hit_rate"],
        "hash_lost_per_step": reuse["lost_per_step"],
        "hash_step_us": reuse["step_us"], "dense_step_us": dense["step_us"],
        "hash_rows_per_step": reuse["rows_per_step"],
        "dense_rows_per_step": dense["rows_per_step"],
        "state_bytes_per_request": {"hash": 12 * w.S, "dense": 8 * w.S +
                                    4 * int(w.host_rows.max())}}), flush=True)
    # Matching latency against K at fixed S and against S at fixed K (one
    # request, 75 % adjacent reuse, Stage One only).
    from workloads.synth import gen_reuse
    for label, shapes in (("K x8 at S=2048", [(256, 2048), (2048, 2048)]),
                          ("S x16 at K=256", [(256, 512), (256, 8192)])):
        row = {}
        for K_, S_ in shapes:
            wk = gen_reuse(1, 0.75, steps=16, K=K_, S=S_)
            hk = r.HostPool(wk.host_bytes)
            wk.fill_host_kv(hk.array)
            row[f"K={K_},S={S_}"] = {
                "hash": eager_steps(r, torch, stream, wk, hk, 0, 4, 12)["stage1_us"],
                "sort_merge": eager_steps(r, torch, stream, wk, hk, r.FLAG_SORT_MERGE,
                                          4, 12)["stage1_us"],
                "dense": eager_steps(r, torch, stream, wk, hk, r.FLAG_DENSE_MAP,
                                     4, 12)["stage1_us"]}
            hk.close()
        a, b_ = (row[k] for k in row)
        print(json.dumps({"comparison": f"Stage-One latency scaling, {label}", "us": row,
                          "hash_growth": round(b_["hash"] / a["hash"], 2),
                          "sort_merge_growth": round(b_["sort_merge"] / a["sort_merge"], 2),
                          "dense_growth": round(b_["dense"] / a["dense"], 2)}),
              flush=True)
    print(json.dumps({
        "comparison": "recall step with reuse vs KV Offload (no reuse), matching workload",
        "with_reuse": reuse, "kv_offload": offload,
        "step_ratio_offload_over_reuse": round(offload["step_us"] / reuse["step_us"], 3)}),
        flush=True)
    return 0


def layers_mode(args):
    """N layers of the matching workload through three schedules; all three
    compute the same results (the tests check it), only the overlap differs."""
    import torch
    import recall_step_amd as r
    from workloads.synth import gen_matching, stack_layers

    torch.cuda.set_device(0)
    L, warm, steps = args.layers, 4, 20
    ws = [gen_matching(steps=warm + steps, layer=l) for l in range(L)]
    st = stack_layers(ws)
    B = ws[0].B
    log(f"[bench] {L} layers x B={B}: host pool {st.host_bytes / 1e9:.2f} GB")
    host = r.HostPool(st.host_bytes)
    st.fill_host_kv(host.array)
    sA, sB = torch.cuda.Stream(), torch.cuda.Stream()
    topk = torch.from_numpy(np.ascontiguousarray(st.topk)).cuda()
    ctx = torch.from_numpy(np.ascontiguousarray(st.ctx_len)).cuda()
    row_base = torch.from_numpy(st.row_base).cuda()
    host_rows = torch.from_numpy(st.host_rows).cuda()

    def handle(Bn):
        cfg = r.avsg_config_default(Bn, st.Nq, st.K, st.S, st.row_bytes, L=st.L, R=st.R,
                                    a1=st.a1, a2=st.a2, a_fp=st.afp)
        return r.RecallStep(cfg, host, st.host_rows_total, stream=sA)

    per = [handle(B) for _ in range(L)]
    big = handle(B * L)
    torch.cuda.synchronize()
    sl = [slice(l * B, (l + 1) * B) for l in range(L)]
    ios_per = [[per[l].io(topk[t][sl[l]], ctx[t][sl[l]], row_base[sl[l]], host_rows[sl[l]])
                for t in range(warm + steps)] for l in range(L)]
    ios_big = [big.io(topk[t], ctx[t], row_base, host_rows) for t in range(warm + steps)]

    def run(kind):
        for h in per + [big]:
            h.state_init(stream=sA)
        torch.cuda.synchronize()
        ev = []
        for t in range(warm + steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(sA)
            if kind == "batched":
                r.avsg_step(big.handle, ios_big[t], sA.cuda_stream)
            elif kind == "sequential":
                for l in range(L):
                    r.avsg_step(per[l].handle, ios_per[l][t], sA.cuda_stream)
            else:
                sB.wait_stream(sA)
                for l in range(L):
                    r.avsg_match(per[l].handle, ios_per[l][t], sA.cuda_stream)
                    done = torch.cuda.Event()
                    done.record(sA)
                    sB.wait_event(done)
                    r.avsg_gather(per[l].handle, ios_per[l][t], sB.cuda_stream)
                sA.wait_stream(sB)
            e1.record(sA)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in ev[warm:]) * 1e3 / steps

    res = {k: round(run(k), 1) for k in ("sequential", "batched", "pipelined")}
    for h in per + [big]:
        h.close()
    host.close()
    print(json.dumps({"layers": L, "B_per_layer": B, "workload": "matching per layer",
                      "step_us": res,
                      "batched_over_sequential": round(res["batched"] / res["sequential"], 3),
                      "pipelined_over_sequential": round(res["pipelined"] / res["sequential"],
                                                         3)}), flush=True)
    return 0


def transfer_sweep(args):
    """Effective host-to-HBM bandwidth against the size of one row: the
    zero-copy gather over scattered rows of a 4 GiB pinned pool, one
    hipMemcpyAsync per row for the same rows, and one bulk copy of the same
    total (64 MiB per point)."""
    import torch
    import recall_step_amd as r

    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    hip = hip_runtime()
    pool_bytes = 4 << 30
    pool = r.HostPool(pool_bytes)
    total = 64 << 20
    rng = np.random.default_rng(77)
    for row in (256, 512, 1024, 1280, 2048, 4096, 8192, 16384, 65536):
        M = total // row
        K, S = (4096, 8192) if M >= 4096 else (M, max(16, 1 << (M - 1).bit_length()))
        Bn = (M + K - 1) // K
        pool_rows = pool_bytes // row
        ids = rng.choice(pool_rows, M, replace=False).astype(np.int32)
        cfg = r.avsg_config_default(Bn, 1, K, S, row)
        rs = r.RecallStep(cfg, pool, pool_rows, stream=stream)
        pairs = np.zeros((Bn, 1, K, 2), np.int32)
        n = np.zeros((Bn, 1), np.int32)
        for b in range(Bn):
            chunk = np.sort(ids[b * K:(b + 1) * K])
            n[b, 0] = chunk.size
            pairs[b, 0, :chunk.size, 0] = chunk
            pairs[b, 0, :chunk.size, 1] = np.arange(chunk.size)
        tp = torch.from_numpy(pairs).cuda()
        tn = torch.from_numpy(n).cuda()
        rb = torch.zeros(Bn, dtype=torch.int64, device="cuda")
        hr = torch.full((Bn,), pool_rows, dtype=torch.int32, device="cuda")
        io = r.AvsgStepIO(0, 0, rb.data_ptr(), hr.data_ptr(), rs.slot_table.data_ptr(),
                          rs.hit_mask.data_ptr(), tn.data_ptr(), tp.data_ptr())
        best = 1e9
        for _ in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            r.avsg_gather(rs.handle, io, sh)
            e1.record(stream)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        zero_copy = M * row / (best * 1e-3) / 1e9
        # one DMA copy per row (at most 4096 rows timed)
        m2 = min(M, 4096)
        dst = rs.dev_kv.data_ptr()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(m2):
            rc = hip.hipMemcpyAsync(dst + i * row, pool.ptr + int(ids[i]) * row, row, 1, sh)
            assert rc == 0, rc
        e1.record(stream)
        e1.synchronize()
        per_row = m2 * row / (e0.elapsed_time(e1) * 1e-3) / 1e9
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = hip.hipMemcpyAsync(dst, pool.ptr, M * row, 1, sh)
        assert rc == 0, rc
        e1.record(stream)
        e1.synchronize()
        bulk = M * row / (e0.elapsed_time(e1) * 1e-3) / 1e9
        rs.close()
        print(json.dumps({"transfer_sweep": "scattered rows of a 4 GiB pinned pool, 64 MiB per point",
                          "row_bytes": row, "rows": M,
                          "zero_copy_gather_GBps": round(zero_copy, 2),
                          "memcpy_per_row_GBps": round(per_row, 2),
                          "bulk_memcpy_GBps": round(bulk, 2)}), flush=True)
    pool.close()
    return 0


def prefetch_mode(args):
    """Threshold prefetch ahead of the recall (ECHO decode prefetch) on the
    scored workload (B=8, context 65536, K=2048, S=4096, ~82 % adjacent
    reuse).  Without prefetch the whole recall (Stage One + gather) follows
    the top-K.  With it, candidates above the moving-average threshold are
    matched and copied first (the part that overlaps the indexer), and only
    the exact selection's continuation is left on the critical path."""
    import torch
    import recall_step_amd as r
    from workloads import make

    torch.cuda.set_device(0)
    w = make("scored")
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream
    host = r.HostPool(w.host_bytes)
    w.fill_host_kv(host.array)
    cfg = r.avsg_config_default(w.B, 1, w.K, w.S, w.row_bytes)
    base = r.RecallStep(cfg, host, w.host_rows_total, stream=stream)
    pre = r.RecallStep(cfg, host, w.host_rows_total, stream=stream)
    dev = base.Q.device
    scores = torch.from_numpy(w.extra["scores"]).to(dev)
    kth = torch.from_numpy(w.extra["kth"]).to(dev)
    topk = torch.from_numpy(np.ascontiguousarray(w.topk)).to(dev)
    ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len)).to(dev)
    row_base = torch.from_numpy(w.row_base).to(dev)
    host_rows = torch.from_numpy(w.host_rows).to(dev)
    theta = torch.full((w.B,), float("inf"), dtype=torch.float32, device=dev)
    cap = torch.full((w.B,), w.K, dtype=torch.int32, device=dev)  # min(K, N/32) = K here
    cand = torch.empty((w.B, 1, w.K), dtype=torch.int32, device=dev)
    o1 = [torch.empty_like(x) for x in (pre.slot_table, pre.hit_mask, pre.n_miss,
                                        pre.miss_pairs)]
    io1 = [r.AvsgStepIO(cand.data_ptr(), ctx[t].data_ptr(), row_base.data_ptr(),
                        host_rows.data_ptr(), o1[0].data_ptr(), o1[1].data_ptr(),
                        o1[2].data_ptr(), o1[3].data_ptr()) for t in range(w.steps)]
    iob = [base.io(topk[t], ctx[t], row_base, host_rows) for t in range(w.steps)]
    iop = [pre.io(topk[t], ctx[t], row_base, host_rows) for t in range(w.steps)]
    torch.cuda.synchronize()
    warm = 4
    rec = []
    for t in range(w.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        e[0].record(stream)
        r.avsg_step(base.handle, iob[t], sh)
        e[1].record(stream)
        r.avsg_prefetch_select(pre.handle, scores[t].data_ptr(), scores.shape[2],
                               ctx[t].data_ptr(), theta.data_ptr(), cap.data_ptr(),
                               cand.data_ptr(), sh)
        r.avsg_step(pre.handle, io1[t], sh)
        e[2].record(stream)
        r.avsg_match_continue(pre.handle, iop[t], sh)
        r.avsg_gather(pre.handle, iop[t], sh)
        e[3].record(stream)
        r.avsg_ema_threshold(pre.handle, kth[t].data_ptr(), theta.data_ptr(), 0.5, sh)
        e[4].record(stream)
        torch.cuda.synchronize()
        n_pre = int(o1[2].sum())
        n_cand = int((cand >= 0).sum())
        n_exact = int(pre.n_miss.sum())
        n_base = int(base.n_miss.sum())
        rec.append((e[0].elapsed_time(e[1]) * 1e3, e[1].elapsed_time(e[2]) * 1e3,
                    e[2].elapsed_time(e[3]) * 1e3, n_cand, n_pre, n_exact, n_base))
    a = np.array(rec[warm:], dtype=np.float64)
    sel = w.B * w.K
    out = {
        "prefetch": "ECHO-style threshold prefetch, scored workload (B=8, K=2048, S=4096, "
                    "context 65536, ~82% adjacent reuse), alpha 0.5, cap K",
        "steps": len(a),
        "no_prefetch_recall_us": round(a[:, 0].mean(), 1),
        "prefetch_part_us": round(a[:, 1].mean(), 1),
        "critical_path_recall_us": round(a[:, 2].mean(), 1),
        "critical_path_speedup": round(a[:, 0].mean() / a[:, 2].mean(), 2),
        "candidates_per_step": round(a[:, 3].mean(), 1),
        "rows_prefetched_per_step": round(a[:, 4].mean(), 1),
        "rows_left_for_exact_recall": round(a[:, 5].mean(), 1),
        "rows_without_prefetch": round(a[:, 6].mean(), 1),
        "selected_per_step": sel,
    }
    base.close()
    pre.close()
    host.close()
    print(json.dumps(out), flush=True)
    return 0


def contiguous_gather_peak(r, torch, stream, row_bytes=1280, rows=1 << 19, blocks=0):
    """The gather kernel on a miss list of consecutive host rows: the
    zero-copy streaming rate of the same kernel without scattered reads."""
    B, K = 256, 2048
    S = K
    rows = min(rows, B * K)
    pool = r.HostPool(rows * row_bytes)
    pool.array[:] = 7
    cfg = r.avsg_config_default(B, 1, K, S, row_bytes, gather_blocks=blocks)
    rs = r.RecallStep(cfg, pool, rows, stream=stream)
    per = rows // B
    n = torch.full((B, 1), per, dtype=torch.int32, device="cuda")
    ids = torch.arange(K, dtype=torch.int32, device="cuda").repeat(B, 1)
    pairs = torch.stack([ids, ids], dim=-1).reshape(B, 1, K, 2).contiguous()
    row_base = (torch.arange(B, dtype=torch.int64, device="cuda") * per)
    host_rows = torch.full((B,), per, dtype=torch.int32, device="cuda")
    io = r.AvsgStepIO(0, 0, row_base.data_ptr(), host_rows.data_ptr(),
                      rs.slot_table.data_ptr(), rs.hit_mask.data_ptr(),
                      n.data_ptr(), pairs.data_ptr())
    best = 0.0
    for _ in range(8):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        r.avsg_gather(rs.handle, io, stream.cuda_stream)
        e1.record(stream)
        e1.synchronize()
        best = max(best, per * B * row_bytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    rs.close()
    pool.close()
    return best


def host_cpu_model():
    """The host CPU's model name and logical CPU count, as the OS reports them."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs visible"


def cpu_baseline(w, host_array, warmup, steps, budget_s):
    """The CPU oracle as it stands, single thread, on the same steps."""
    import oracle
    per_pass = []
    t_start = time.perf_counter()
    passes = 0
    while True:
        o = oracle.Oracle.for_workload(w, host_kv=host_array)
        for t in range(warmup):
            k = t % w.steps
            o.step(w.topk[k], w.ctx_len[k], w.row_base, w.host_rows)
        t0 = time.perf_counter()
        for t in range(warmup, warmup + steps):
            k = t % w.steps
            o.step(w.topk[k], w.ctx_len[k], w.row_base, w.host_rows)
        per_pass.append((time.perf_counter() - t0) / steps)
        passes += 1
        if time.perf_counter() - t_start >= budget_s or passes >= 50:
            break
    return statistics.median(per_pass), passes


def adjacent_step_reuse(topk, t0, t1):
    """Mean over requests and steps t in [t0, t1) of the fraction of step t's
    selected ids (all query tokens, padding and repeats dropped) that step
    t - 1 selected too; None when t0 is 0."""
    if t0 < 1:
        return None
    fr = []
    for t in range(t0, t1):
        for b in range(topk.shape[1]):
            cur = np.unique(topk[t, b][topk[t, b] >= 0])
            prev = np.unique(topk[t - 1, b][topk[t - 1, b] >= 0])
            if cur.size:
                fr.append(np.isin(cur, prev, assume_unique=True).mean())
    return float(np.mean(fr)) if fr else None


def host_threads():
    """Worker threads for host-side work: the machine's CPU share (its
    OMP_NUM_THREADS), else the visible cores."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, int(env)) if env.isdigit() else max(1, os.cpu_count() or 1)


def cpu_baseline_all_cores(w, host_array, warmup, steps):
    """The same oracle on all host cores: requests are independent, so each
    request runs in its own single-request oracle on a thread pool (the
    oracle's C calls release the GIL).  Returns the wall time per step of the
    timed steps and the threads used."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    threads = min(w.B, host_threads())
    orcs = [oracle.Oracle(1, w.Nq, w.K, w.S, w.L, w.R, w.a1, w.a2, w.afp, w.row_bytes,
                          w.host_rows_total, host_array) for _ in range(w.B)]

    def run(b, t0, t1):
        rb, hr = w.row_base[b:b + 1], w.host_rows[b:b + 1]
        for t in range(t0, t1):
            k = t % w.steps
            orcs[b].step(w.topk[k][b:b + 1], w.ctx_len[k][b:b + 1], rb, hr)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda b: run(b, 0, warmup), range(w.B)))
        t0 = time.perf_counter()
        list(ex.map(lambda b: run(b, warmup, warmup + steps), range(w.B)))
        wall = time.perf_counter() - t0
    return wall / steps, threads


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the recall path shards by request "
              f"with no exchange between GPUs, and this build measures one GPU's "
              f"share; --gpus {args.gpus} is not supported.", file=sys.stderr)
        return 2
    if args.probe_sweep:
        return probe_sweep(args)
    if args.shape_sweep:
        return shape_sweep(args)
    if args.lifetime_sweep:
        return lifetime_sweep(args)
    if args.ratios:
        return ratios(args)
    if args.layers:
        return layers_mode(args)
    if args.prefetch:
        return prefetch_mode(args)
    if args.transfer_sweep:
        return transfer_sweep(args)
    import torch
    import recall_step_amd as r
    from workloads import make

    # Enough distinct steps for the warm-up and the timed steps, so that no
    # selection is replayed onto a buffer that already holds it.  The MTP-3
    # workload is defined as 32 iterations (its verified length grows by 4
    # per iteration into the end of the host rows), so a run needing more is
    # refused rather than replayed.
    need = args.warmup + args.steps
    if args.workload == "mtp3" and need > 32:
        print(f"bench.py: the MTP-3 workload has 32 iterations; --warmup {args.warmup} "
              f"+ --steps {args.steps} = {need} would replay some of them onto a "
              f"buffer that already holds them.", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    w = make(args.workload)
    if need > w.steps:
        w = make(args.workload, steps=need)
    log(f"[bench] workload {w.name}: B={w.B} Nq={w.Nq} K={w.K} S={w.S} "
        f"row={w.row_bytes} host_bytes={w.host_bytes} steps={args.steps} warmup={args.warmup}")
    stream = torch.cuda.Stream()
    host = r.HostPool(w.host_bytes)
    w.fill_host_kv(host.array)
    cfg = r.avsg_config_default(w.B, w.Nq, w.K, w.S, w.row_bytes, L=w.L, R=w.R,
                                a1=w.a1, a2=w.a2, a_fp=w.afp,
                                gather_blocks=args.gather_blocks,
                                stage1_threads=args.stage1_threads)
    rs = r.RecallStep(cfg, host, w.host_rows_total, stream=stream)
    topk = torch.from_numpy(np.ascontiguousarray(w.topk)).cuda()
    ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len)).cuda()
    row_base = torch.from_numpy(w.row_base).cuda()
    host_rows = torch.from_numpy(w.host_rows).cuda()
    ios = [rs.io(topk[t], ctx[t], row_base, host_rows) for t in range(w.steps)]
    sh = stream.cuda_stream
    torch.cuda.synchronize()

    first_reuse = None
    for t in range(args.warmup):
        rs.step(ios[t % w.steps], stream)
        if t == 0:
            # The first step starts from an empty buffer: whatever it does
            # not copy, its query tokens reused from one another.
            d0 = rs.CNT.cpu().numpy().astype(np.int64).sum(0)
            if d0[r.CNT_LOOKUPS]:
                first_reuse = 1.0 - d0[r.CNT_MISSES] / d0[r.CNT_LOOKUPS]
    torch.cuda.synchronize()
    cnt0 = rs.CNT.cpu().numpy().astype(np.int64)

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        io = ios[(args.warmup + k) % w.steps]
        e = ev[k]
        e[0].record(stream)
        r.avsg_match(rs.handle, io, sh)
        e[1].record(stream)
        r.avsg_gather(rs.handle, io, sh)
        e[2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    cnt1 = rs.CNT.cpu().numpy().astype(np.int64)

    # The same steps from an empty buffer, each step a replay of a graph
    # captured on that step's inputs (Stage One + gather), so no copy sits
    # between steps: the K replays back to back, bracketed by device
    # synchronisation, with events between replays for the per-step spread.
    rs.state_init(stream=stream)
    torch.cuda.synchronize()
    graphs = []
    with torch.cuda.stream(stream):
        for t in range(w.steps):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                rs.step(ios[t], stream=stream)
            graphs.append(g)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for k in range(args.warmup):
            graphs[k % w.steps].replay()
    torch.cuda.synchronize()
    gev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    tg0 = time.perf_counter()
    with torch.cuda.stream(stream):
        gev[0].record(stream)
        for k in range(K):
            graphs[(args.warmup + k) % w.steps].replay()
            gev[k + 1].record(stream)
    torch.cuda.synchronize()
    graph_wall = time.perf_counter() - tg0
    step_ms = [gev[k].elapsed_time(gev[k + 1]) for k in range(K)]

    # Headline: the same timed steps captured together in one graph, as the
    # recall sits inside a captured decode step among other kernels, where
    # the graph's launch is paid once and not once per recall step.
    rs.state_init(stream=stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for k in range(args.warmup):
            graphs[k % w.steps].replay()
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all, stream=stream):
            for k in range(K):
                rs.step(ios[(args.warmup + k) % w.steps], stream=stream)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ta0 = time.perf_counter()
    with torch.cuda.stream(stream):
        a0.record(stream)
        g_all.replay()
        a1.record(stream)
    torch.cuda.synchronize()
    one_graph_wall = time.perf_counter() - ta0
    one_graph_event_us = a0.elapsed_time(a1) * 1e3 / K
    del graphs, g_all

    # Stage One alone over the same steps from an empty buffer (the gather
    # does not change the state), its timed launches back to back between
    # two events: the match rate without the dispatch gap that an event pair
    # around each launch includes.
    rs.state_init(stream=stream)
    for t in range(args.warmup):
        r.avsg_match(rs.handle, ios[t % w.steps], sh)
    m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    m0.record(stream)
    for k in range(K):
        r.avsg_match(rs.handle, ios[(args.warmup + k) % w.steps], sh)
    m1.record(stream)
    torch.cuda.synchronize()
    s1_b2b_s = m0.elapsed_time(m1) * 1e-3 / K
    d = (cnt1 - cnt0).sum(0)
    s1_ms = [e[0].elapsed_time(e[1]) for e in ev]
    g_ms = [e[1].elapsed_time(e[2]) for e in ev]
    misses, lookups, hits = int(d[r.CNT_MISSES]), int(d[r.CNT_LOOKUPS]), int(d[r.CNT_HITS])
    visits = int(d[r.CNT_PROBE_VISITS])
    gather_bytes = misses * w.row_bytes
    s1_avg_s = sum(s1_ms) * 1e-3 / K
    g_avg_s = sum(g_ms) * 1e-3 / K
    step_us = one_graph_wall / K * 1e6
    gather_gbps = gather_bytes / (sum(g_ms) * 1e-3) / 1e9
    mkeys = lookups / K / s1_b2b_s / 1e6

    s1_bytes_step = stage1_algorithmic_bytes(w.B, w.S, w.Nq, lookups / K, visits / K,
                                             misses / K)
    # Over the distinct timed steps (a workload with fewer steps than the run
    # replays them cyclically).
    adj_reuse = adjacent_step_reuse(w.topk, args.warmup, min(args.warmup + K, w.steps))

    result = {
        "metric": METRIC,
        "value": round(step_us, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "N_q": w.Nq, "K": w.K, "S": w.S,
                   "row_bytes": w.row_bytes, "context": int(w.host_rows.max()),
                   "L": w.L, "R": w.R, "parallelism": "single GPU"},
        "step_us_p50_p90": [round(float(np.percentile(step_ms, q)) * 1e3, 2) for q in (50, 90)],
        "value_timing": "wall time of one replay of a graph holding the K timed steps, "
                        "between device synchronisations, divided by K",
        "one_graph_event_us": round(one_graph_event_us, 2),
        "graph_per_step_us": round(graph_wall / K * 1e6, 2),
        "graph_event_mean_us": round(sum(step_ms) * 1e3 / K, 2),
        "eager_wall_us_per_step": round(wall / K * 1e6, 2),
        "gather_GBps": round(gather_gbps, 2),
        "match_Mkeys_per_s": round(mkeys, 1),
        "match_timing": "Stage One alone, the timed launches back to back between two "
                        "events on the launch stream; lookups per step / time per launch",
        "stage1_us": round(s1_b2b_s * 1e6, 2),
        "stage1_event_pair_us": round(s1_avg_s * 1e6, 2),
        "gather_us": round(g_avg_s * 1e6, 2),
        "stage1_us_p50_p90": [round(float(np.percentile(s1_ms, q)) * 1e3, 2) for q in (50, 90)],
        "gather_us_p50_p90": [round(float(np.percentile(g_ms, q)) * 1e3, 2) for q in (50, 90)],
        "misses_per_step": round(misses / K, 1),
        "hit_rate": round(hits / lookups, 4) if lookups else 0.0,
        "lost_mappings_per_step": round(float(d[r.CNT_LOST_COLLISION] + d[r.CNT_LOST_EXHAUSTED]) / K, 1),
        "adjacent_reuse": (None if adj_reuse is None else round(adj_reuse, 4)),
        "first_step_reuse": (None if first_reuse is None else round(float(first_reuse), 4)),
        "roofline": {
            "bound": "pcie",
            "achieved": round(gather_gbps, 2),
            "peak": PCIE_GEN5_X16_GBPS,
            "unit": "GB/s",
            "frac": round(gather_gbps / PCIE_GEN5_X16_GBPS, 4),
            "traffic": profiled_traffic("gather_kernel", w.name),
            "kernel": "gather_kernel",
            "bytes_per_launch": round(gather_bytes / K),
            "timing": "event pair around each launch in the eager pass, on the launch "
                      "stream",
        },
        "roofline_stage1": {
            "bound": "hbm",
            "achieved": round(s1_bytes_step / s1_b2b_s / 1e9, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(s1_bytes_step / s1_b2b_s / 1e9 / HBM_PEAK_GBPS, 5),
            "traffic": profiled_traffic("stage1_kernel", w.name),
            "kernel": "stage1_kernel",
            "bytes_per_launch": round(s1_bytes_step),
            "bytes_model": STAGE1_BYTES_MODEL,
        },
    }

    if not args.no_peaks:
        log("[bench] measuring pinned memcpy and contiguous zero-copy peaks")
        peak = pinned_h2d_peak(r, torch, stream)
        contig = contiguous_gather_peak(r, torch, stream, w.row_bytes,
                                        blocks=args.gather_blocks)
        result["hbm_copy_peak_GBps"] = round(hbm_copy_peak(torch, stream), 1)
        result["pinned_h2d_memcpy_peak_GBps"] = round(peak, 2)
        result["contiguous_gather_GBps"] = round(contig, 2)
        result["gather_frac_of_memcpy_peak"] = round(gather_gbps / peak, 4)

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on the same steps")
        per_step, passes = cpu_baseline(w, host.array, args.warmup, K, args.cpu_seconds)
        cpu = host_cpu_model()
        result["cpu_baseline"] = {
            "value": round(per_step * 1e6, 1), "unit": "us", "cores": 1, "kind": "oracle",
            "sample": f"{w.name} workload, full batch, the same {K} timed steps after "
                      f"{args.warmup} warm-up steps, {passes} passes from an empty "
                      f"buffer, median per-step time (single thread, gcc -O2)",
            "cpu": cpu,
        }
        per_step_mt, threads = cpu_baseline_all_cores(w, host.array, args.warmup, K)
        result["cpu_baseline_all_cores"] = {
            "value": round(per_step_mt * 1e6, 1), "unit": "us", "cores": threads,
            "kind": "oracle", "cpu": cpu,
            "sample": f"{w.name} workload, the same {K} timed steps after {args.warmup} "
                      f"warm-up steps, one pass from an empty buffer; each request in its "
                      f"own single-request oracle, requests spread over {threads} threads",
        }

    rs.close()
    host.close()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
