#!/usr/bin/env python3
"""Benchmark of the MoE expert-parallel dispatch -> combine path on one MI355X.

One step = one pass of the whole path over one batch already resident in
HBM: ep_plan (layout, and the static plan where the workload uses it) ->
ep_dispatch -> ep_combine with identity experts; the training workload adds
ep_combine_bwd -> dispatch backward -> duplicated-expert gradient reduce.

Default workload: prefill, T=4096 tokens, H=7168 bf16, E=256 experts, top-8,
Zipf(1.1)-skewed routing, HT (2D concatenated) layout.

Prints ONE JSON line: tokens/s of the whole step (value), HBM GB/s of the
step's algorithmic bytes, the roofline of the dominant kernel timed with HIP
events on the stream it is launched on, and the CPU oracle's throughput on a
bounded sample of the same workload (a reported baseline, not a target).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8
METRIC = "dispatch+combine tokens/s and HBM GB/s (% of peak), T=4096 H=7168 top-8"


def parse():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="prefill",
                   choices=["prefill", "decode", "tiny", "sweep", "training"])
    p.add_argument("--rho", type=float, default=8.0, help="sweep: max/mean expert load")
    p.add_argument("--fp8", action="store_true",
                   help="FP8 e4m3 dispatch (one fp32 scale per 128 channels); with --gemm the "
                        "grouped GEMM takes the FP8 rows and FP8 weights (roofline against the "
                        "fp8 MFMA peak)")
    p.add_argument("--fp8-scales", choices=("amax", "pow2", "amax_pow2w"), default="amax",
                   help="format of the FP8 scales (the group's fp8_scales): amax/448, or the power "
                        "of two at or above it (then the FP8 GEMM of large groups runs on the "
                        "256 x 256 kernel with the scales applied by the matrix cores), or amax "
                        "rows against power-of-two weight scales (the matrix cores apply the "
                        "weights' scales, the rows' are folded)")
    p.add_argument("--route", action="store_true",
                   help="start the step from router logits (ep_route before ep_plan)")
    p.add_argument("--two-call-dispatch", action="store_true",
                   help="time ep_plan + ep_dispatch as two calls even where ep_plan_dispatch "
                        "runs them as one launch (LL / HT with T*k <= 2048: decode, tiny)")
    p.add_argument("--fused-route", action="store_true",
                   help="start the step from router logits with routing fused into the layout "
                        "launch (ep_route_plan instead of ep_route + ep_plan)")
    p.add_argument("--prefetch", action="store_true",
                   help="STATIC workloads: add the replica-weight prefetch of one [4096, 1536] "
                        "bf16 projection per expert after the plan")
    p.add_argument("--dispatch-stores", choices=("auto", "cached", "streaming"), default="auto",
                   help="how dispatch writes the receive rows (default: cached for 64 MiB to "
                        "512 MiB of rows, non-temporal otherwise)")
    p.add_argument("--combine-stores", choices=("auto", "cached", "streaming"), default=None,
                   help="how combine writes its token rows (default: streaming for the training "
                        "step, whose backward pass streams far more than the Infinity Cache "
                        "holds; the library's default, cached, otherwise)")
    p.add_argument("--slot-mode", choices=("training", "inference"), default="training",
                   help="STATIC workloads: what the plan does past a rank's S-th replica slot")
    p.add_argument("--slots", type=int, default=None,
                   help="STATIC workloads: replica slots per rank (default: the workload's)")
    p.add_argument("--gemm", type=int, default=0, metavar="N",
                   help="add the grouped GEMM of the experts after dispatch: the received "
                        "[rows, H] bf16 tokens times one [N, H] bf16 matrix per expert (through "
                        "the prefetch slots with --prefetch); reported beside the step, its "
                        "roofline against the bf16 MFMA peak")
    p.add_argument("--swiglu", action="store_true",
                   help="with --gemm: the FFN's first GEMM with the SwiGLU store (weight rows "
                        "interleave gate and up; output N/2 columns of silu(gate) * up)")
    p.add_argument("--ffn", action="store_true",
                   help="with --gemm N --swiglu: the whole expert FFN, the second GEMM [E, H, N/2] "
                        "back to H after the activation (with --fp8 the activation quantised by "
                        "ep_quantize_fp8 first, both GEMMs on FP8 operands); combine then gathers "
                        "the FFN output")
    p.add_argument("--microbatches", type=int, default=1, metavar="M",
                   help="one step = M independent micro-batches of the workload (forward chain "
                        "plan -> dispatch -> combine), each with its own inputs, handle, receive "
                        "and output buffers (M-deep buffering); value = M*T tokens per step")
    p.add_argument("--overlap", action="store_true",
                   help="with --microbatches: micro-batch i on stream i, launches interleaved op "
                        "by op, so one micro-batch's plan/dispatch runs beside another's combine "
                        "(without it: all micro-batches in turn on one stream)")
    p.add_argument("--graph", action="store_true",
                   help="time the step as one captured HIP graph (replayed K times) instead of "
                        "K eager launches of each call; per-kernel times stay eager")
    p.add_argument("--cold", action="store_true",
                   help="read a 512 MB buffer before every step (Infinity Cache evicted with "
                        "clean lines); steps are then timed one by one")
    p.add_argument("--no-prepare", action="store_true",
                   help="marshal every call's arguments in Python each time (by default each op is "
                        "prepared once with ep.prepare and replays its C call)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                   help="only run a plain device copy of MB megabytes K times (counter scaling)")
    a = p.parse_args()
    if a.combine_stores is None:
        a.combine_stores = "streaming" if a.workload == "training" else "auto"
    return a


PREFETCH_P = 4096 * 1536   # elements of one expert projection (training shapes)


def median_step_ms(run_step, K, stream):
    """Median of K more steps, each bracketed by events.  An event record
    costs host time (about 3 us here), which a launch-bound step would pay
    inside its own time, so this pass gives the median only; ms_per_step comes
    from K steps back to back between two events."""
    import torch
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(K):
        run_step()
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    lst = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(K))
    return lst[K // 2] if K % 2 else 0.5 * (lst[K // 2 - 1] + lst[K // 2])


def gemm_report(ab, name, us, grows, mats, N, K, n_out, fp8, epilogue):
    """Flops, algorithmic bytes (X, every weight matrix used and Y, once each;
    stored in ab[name]) and the roofline of one grouped GEMM launch."""
    flops = 2.0 * grows * N * K
    if fp8:   # codes (1 byte) plus one fp32 scale per 128 of K, for rows and weights
        el, sc, peak = 1, 4.0 / 128, MFMA_FP8_PEAK_TFLOPS
    else:
        el, sc, peak = 2, 0.0, MFMA_BF16_PEAK_TFLOPS
    ab[name] = int(grows * K * (el + sc) + mats * N * K * (el + sc) + grows * n_out * 2)
    tflops = flops / (us * 1e-6) / 1e12
    info = {"N": N, "K": K, "dtype": "fp8-e4m3" if fp8 else "bf16", "epilogue": epilogue,
            "rows": grows, "weight_matrices": mats, "flops": flops,
            "avg_us": round(us, 2), "tflops": round(tflops, 1)}
    # the binding resource: MFMA time of the flops or HBM time of the bytes
    if flops / (peak * 1e12) >= ab[name] / (HBM_PEAK_GBPS * 1e9):
        info["roofline"] = {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak,
                            "unit": "TFLOP/s", "frac": round(tflops / peak, 4)}
    else:
        gbps = ab[name] / (us * 1e-6) / 1e9
        info["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4)}
    return info


def algorithmic_bytes(c, fp8=False, filled_slots=0, slot_elems=PREFETCH_P, slot_elem_bytes=2):
    """Bytes each kernel must move by definition: x read once, every routed row
    written once and read once, outputs written once, int32/fp32 metadata."""
    N = c.T * c.k
    row = c.H * 2
    b = {
        "route": c.T * c.E * 4 + N * 8,                          # logits read, idx + weights written
        "plan": N * 4 + N * 4,                                   # topk_idx read, dst written
        "dispatch": c.T * row + N * (c.H + c.H // 128 * 4 if fp8 else row) + N * 4,
        "combine": N * row + N * 4 + N * 4 + c.T * row,          # rows, dst, w read; y written
    }
    if c.name == "training":
        b["combine_bwd"] = c.T * row + N * row + N * row + N * 4 * 3 + N * 4   # gy, out rows, grad rows, dst/w, grad_w
        b["dispatch_bwd"] = N * row + N * 4 + c.T * row
        P = 4096 * 1536
        b["dup_reduce"] = 2 * P * 2 + P * 4 * 2                  # 2 bf16 replicas, one fp32 owner r/w
    b["route_plan"] = b["route"] + b["plan"]
    b["plan_dispatch"] = b["plan"] + b["dispatch"]
    b["prefetch"] = filled_slots * slot_elems * slot_elem_bytes * 2   # each filled slot: owner row read, slot written
    b["prefetch_scales"] = filled_slots * (slot_elems // 128) * 4 * 2  # FP8 weights: their fp32 scales
    return b


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "combine_ep_plan_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {"dispatch": ["dispatch.hip", "device.h"], "combine": ["combine.hip", "device.h"],
                  "combine_bwd": ["combine.hip", "device.h"], "dispatch_bwd": ["combine.hip", "device.h"],
                  "plan": ["plan.hip"], "dup_reduce": ["dup_reduce.hip", "device.h"],
                  "plan_dispatch": ["dispatch.hip", "device.h"]}


def traffic_for(workload, kernel):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel source; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    k = d.get("kernels", {}).get(kernel)
    if not k or k.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return k.get("bytes_per_launch")


def cpu_baseline(name, rho, fp8, budget_s):
    """The oracle, as it stands, on the whole batch of the same workload: the
    full layout -> dispatch -> combine chain, repeated for about budget_s
    (three quarters on every host thread, one quarter on one thread)."""
    import numpy as np
    import oracle
    import workloads
    oracle.build(force=False)
    c = workloads.get_config(name, rho)
    Ts = c.T
    inp = workloads.make_inputs(name, 0, rho) if name == "sweep" else workloads.make_inputs(name)
    idx, w, x = inp.topk_idx[:Ts], inp.topk_w[:Ts], inp.x[:Ts]

    def chain():
        L = oracle.layout(idx, c.E, c.layout, cap=c.cap, R=c.R, S=c.S)
        if fp8:
            oracle.dispatch_fp8(x, L.dst, L.rows)
        recv = oracle.dispatch(x, L.dst, L.rows)
        oracle.combine(recv, L.dst, w, out_fp32=c.out_fp32)

    def timed(seconds):
        chain()
        runs, t0 = 0, time.perf_counter()
        while True:
            chain()
            runs += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return runs, el

    cores = oracle.get_threads()
    runs, el = timed(budget_s * 0.75)
    oracle.set_threads(1)
    runs1, el1 = timed(budget_s * 0.25)
    oracle.set_threads(cores)
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": Ts * runs / el, "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{Ts} of {c.T} tokens of the {name} workload (the whole batch), full "
                      f"layout{'+plan' if c.layout == 'static' else ''}+dispatch+combine chain, "
                      f"{runs} runs in {el:.1f} s on {cores} threads",
            "value_1_thread": round(Ts * runs1 / el1, 1), "cpu_model": model}


def run_microbatches(a):
    """Several micro-batches in flight: the one-GPU form of double-buffered
    dispatch/combine ([NCCL-EP] Table II and Figure 2: LL mode overlaps the
    dispatch and combine phases of consecutive batches through double
    buffers).  Every micro-batch has its own handle, receive and output
    buffers; with --overlap each runs on its own stream (default priority) and
    the launches are interleaved op by op, so the GPU sees micro-batch i's
    plan and dispatch beside micro-batch j's combine."""
    import numpy as np
    import torch
    import combine_ep_plan_amd as ep
    import workloads

    name, M = a.workload, a.microbatches
    if name == "training" or a.route or a.fused_route or a.prefetch or a.gemm or a.graph or a.cold:
        print("bench.py: --microbatches times the forward chain only (no training, --route, --fused-route, "
              "--prefetch, --gemm, --graph or --cold)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    main_stream = torch.cuda.current_stream()
    c = workloads.get_config(name, a.rho)
    # overlapped micro-batches are passes in flight together: the library's
    # default store rule counts their receive rows together
    g = ep.Group(c.E, c.R, c.H, c.k, c.T, c.layout, capacity=c.cap, slots_per_rank=c.S,
                 dispatch_stores=a.dispatch_stores, passes_in_flight=M if a.overlap else 1,
                 combine_stores=a.combine_stores)
    streams = [torch.cuda.Stream() for _ in range(M)] if a.overlap else [main_stream] * M
    fused = c.layout in ("ll", "ht") and c.T * c.k <= 2048 and not a.two_call_dispatch
    mbs = []
    for i in range(M):
        inp = workloads.make_inputs(name, i, a.rho)
        h = ep.Handle(g, c.T)
        x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
        idx = torch.from_numpy(inp.topk_idx).to(dev)
        w = torch.from_numpy(inp.topk_w).to(dev)
        recv = torch.empty(g.recv_shape(c.T), dtype=torch.bfloat16, device=dev)
        y = torch.empty((c.T, c.H), dtype=torch.float32 if c.out_fp32 else torch.bfloat16, device=dev)
        ep.ep_plan(h.ptr, idx, main_stream)
        ep.ep_dispatch(h.ptr, x, None, recv, None, None, None, main_stream)   # bf16 rows feed combine
        rq = rs = None
        if a.fp8:
            rq = torch.empty(g.recv_shape(c.T), dtype=torch.float8_e4m3fn, device=dev)
            rs = torch.empty((h.recv_rows, c.H // 128), dtype=torch.float32, device=dev)
        st = streams[i]

        def ops_for(h=h, x=x, idx=idx, w=w, recv=recv, y=y, rq=rq, rs=rs, st=st):
            out, out_s = (rq, rs) if a.fp8 else (recv, None)
            if fused:   # layout and dispatch in one launch
                lead = [("plan_dispatch",
                         lambda: ep.ep_plan_dispatch(h.ptr, idx, x, None, out, out_s, None, None, st))]
            else:
                lead = [("plan", lambda: ep.ep_plan(h.ptr, idx, st)),
                        ("dispatch", lambda: ep.ep_dispatch(h.ptr, x, None, out, out_s, None, None, st))]
            ops = lead + [("combine", lambda: ep.ep_combine(h.ptr, recv, w, y, st))]
            return ops if a.no_prepare else [(nm, ep.prepare(f)) for nm, f in ops]
        mbs.append((h, ops_for()))
    n_ops = len(mbs[0][1])
    start = torch.cuda.Event()
    ends = [torch.cuda.Event() for _ in range(M)]

    def step():
        # one pass over every micro-batch; with --overlap the streams are not
        # joined between steps (micro-batch i's next step depends only on its
        # own previous one), only around the timed region
        if a.overlap:
            for j in range(n_ops):
                for _, ops in mbs:
                    ops[j][1]()
        else:
            for _, ops in mbs:
                for _, f in ops:
                    f()

    def fork():
        start.record(main_stream)
        for st in streams:
            st.wait_event(start)

    def join():
        for st, e in zip(streams, ends):
            e.record(st)
            main_stream.wait_event(e)

    if a.overlap:
        fork()
    for _ in range(a.warmup):
        step()
    if a.overlap:
        join()
    torch.cuda.synchronize()
    for h, _ in mbs:
        assert h.status() == 0, "device flags raised on the benchmark input"
    K = a.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(main_stream)
    if a.overlap:
        fork()
    for i in range(K):
        step()
    if a.overlap:
        join()
    e1.record(main_stream)
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / K
    if a.overlap:
        median_ms = None   # the streams run free between the fork and the join
    else:
        median_ms = median_step_ms(step, K, main_stream)

    # per-kernel durations: micro-batch 0's launches one by one on the main
    # stream (nothing beside them), for the roofline of the dominant kernel
    h0, _ = mbs[0]
    inp0 = workloads.make_inputs(name, 0, a.rho)
    x0 = torch.from_numpy(inp0.x.view(np.int16)).to(dev).view(torch.bfloat16)
    idx0 = torch.from_numpy(inp0.topk_idx).to(dev)
    w0 = torch.from_numpy(inp0.topk_w).to(dev)
    recv0 = torch.empty(g.recv_shape(c.T), dtype=torch.bfloat16, device=dev)
    y0 = torch.empty((c.T, c.H), dtype=torch.float32 if c.out_fp32 else torch.bfloat16, device=dev)
    rq0 = torch.empty(g.recv_shape(c.T), dtype=torch.float8_e4m3fn, device=dev) if a.fp8 else None
    rs0 = torch.empty((h0.recv_rows, c.H // 128), dtype=torch.float32, device=dev) if a.fp8 else None
    serial = [("plan", lambda: ep.ep_plan(h0.ptr, idx0, main_stream)),
              ("dispatch", (lambda: ep.ep_dispatch(h0.ptr, x0, None, rq0, rs0, None, None, main_stream)) if a.fp8
               else (lambda: ep.ep_dispatch(h0.ptr, x0, None, recv0, None, None, None, main_stream))),
              ("combine", lambda: ep.ep_combine(h0.ptr, recv0, w0, y0, main_stream))]
    ep.ep_plan(h0.ptr, idx0, main_stream)
    ep.ep_dispatch(h0.ptr, x0, None, recv0, None, None, None, main_stream)
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in serial]
           for _ in range(K)]
    for sidx in range(K):
        for (b, e), (_, f) in zip(evs[sidx], serial):
            b.record(main_stream)
            f()
            e.record(main_stream)
    torch.cuda.synchronize()
    per_us = {nm: 1000.0 * sum(evs[sidx][i][0].elapsed_time(evs[sidx][i][1]) for sidx in range(K)) / K
              for i, (nm, _) in enumerate(serial)}
    ab = algorithmic_bytes(c, a.fp8)
    dom = max(("dispatch", "combine"), key=lambda nm: per_us[nm])
    dom_gbps = ab[dom] / (per_us[dom] * 1e-6) / 1e9
    step_s = step_ms / 1000.0
    chain_bytes = M * sum(ab[nm] for nm, _ in serial)
    out = {
        "metric": METRIC,
        "value": round(M * c.T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(step_ms, 4),
        "median_ms_per_step": None if median_ms is None else round(median_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{name} {c.layout.upper()} T={c.T} H={c.H} E={c.E} top-{c.k}"
                               f"{' fp8' if a.fp8 else ''}, {M} micro-batches "
                               f"{'overlapped on ' + str(M) + ' streams' if a.overlap else 'in turn on one stream'}",
                   "T": c.T, "H": c.H, "E": c.E, "top_k": c.k, "layout": c.layout,
                   "microbatches": M, "overlap": a.overlap, "dispatch_stores": a.dispatch_stores,
                   "combine_stores": a.combine_stores,
                   "step": " -> ".join(nm for nm, _ in mbs[0][1]) + f" (x{M})",
                   "prepared_calls": not a.no_prepare},
        "hbm_gbps": round(chain_bytes / step_s / 1e9, 1),
        "hbm_frac_of_peak": round(chain_bytes / step_s / 1e9 / HBM_PEAK_GBPS, 4),
        "step_algorithmic_bytes": chain_bytes,
        "kernels_us_alone": {k: round(v, 2) for k, v in per_us.items()},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                     "bytes_per_launch": ab[dom], "avg_us": round(per_us[dom], 2)},
    }
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(name, a.rho, a.fp8, a.cpu_seconds)
    print(json.dumps(out), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (got --gpus {a.gpus}); logical "
              "expert-parallel ranks are regions of that GPU's HBM.", file=sys.stderr)
        sys.exit(2)
    if a.microbatches > 1 or a.overlap:
        if a.microbatches < 2:
            print("bench.py: --overlap needs --microbatches M with M >= 2", file=sys.stderr)
            sys.exit(2)
        return run_microbatches(a)
    import numpy as np
    import torch
    import combine_ep_plan_amd as ep
    import workloads

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    if a.copy_calibration:
        n = a.copy_calibration * (1 << 20)
        src = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(a.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        for _ in range(a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": a.steps + a.warmup}))
        return

    name = a.workload
    inp = workloads.make_inputs(name, 0, a.rho) if name == "sweep" else workloads.make_inputs(name)
    c = inp.cfg
    S = c.S if a.slots is None else a.slots
    if a.swiglu and (not a.gemm or a.gemm % 16):
        print("bench.py: --swiglu needs --gemm N with N a multiple of 16", file=sys.stderr)
        sys.exit(2)
    if a.ffn and (not a.swiglu or (a.fp8 and a.gemm % 256)):
        print("bench.py: --ffn needs --gemm N --swiglu (with --fp8: N a multiple of 256, so that "
              "the activation is whole 128-blocks)", file=sys.stderr)
        sys.exit(2)
    if (a.prefetch or a.slots is not None or a.slot_mode != "training") and c.layout != "static":
        print("bench.py: --prefetch, --slots and --slot-mode need a STATIC workload (sweep, training)",
              file=sys.stderr)
        sys.exit(2)
    g = ep.Group(c.E, c.R, c.H, c.k, c.T, c.layout, capacity=c.cap, slots_per_rank=S,
                 slot_mode=a.slot_mode, dispatch_stores=a.dispatch_stores, fp8_scales=a.fp8_scales,
                 combine_stores=a.combine_stores)
    h = ep.Handle(g, c.T)
    x = torch.from_numpy(inp.x.view(np.int16)).to(dev).view(torch.bfloat16)
    idx = torch.from_numpy(inp.topk_idx).to(dev)
    w = torch.from_numpy(inp.topk_w).to(dev)
    shape = g.recv_shape(c.T)
    recv = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    rq = rs = None
    if a.fp8:
        rq = torch.empty(shape, dtype=torch.float8_e4m3fn, device=dev)
        rs = torch.empty((h.recv_rows, c.H // 128), dtype=torch.float32, device=dev)
    y = torch.empty((c.T, c.H), dtype=torch.float32 if c.out_fp32 else torch.bfloat16, device=dev)
    train = name == "training"
    if train:
        gy = torch.from_numpy(workloads.make_grad(c, 0, (c.T, c.H), 1).view(np.int16)).to(dev).view(torch.bfloat16)
        gout = torch.empty_like(recv)
        gw = torch.empty_like(w)
        gx = torch.empty((c.T, c.H), dtype=torch.bfloat16, device=dev)
        rep = torch.from_numpy(workloads.make_grad(c, 0, (2, 4096, 1536), 2).view(np.int16)).to(dev).view(torch.bfloat16)
        owner = torch.zeros((c.E, 4096, 1536), dtype=torch.float32, device=dev)
        rep_e = torch.zeros(2, dtype=torch.int32, device=dev)   # replicas of expert 0, same owner
    flush = torch.ones(512 << 20, dtype=torch.uint8, device=dev) if a.cold else None

    def evict():
        # Reading twice the Infinity Cache's 256 MB leaves it holding clean lines
        # of another buffer: the step then misses in it without paying for the
        # write-back of dirty lines, which a flush by writing would add.
        flush.view(torch.int32).sum()

    LS = {"s": stream}   # the stream the library calls launch on (a capture stream under --graph)
    ops = []
    if a.route or a.fused_route:   # the pass starts from router logits: plan and combine use the routed outputs
        logits = torch.from_numpy(inp.logits).to(dev)
        idx, w = torch.empty_like(idx), torch.empty_like(w)
    # small LL / HT batches: the layout runs inside the dispatch launch (ep_plan_dispatch)
    fused_pd = (c.layout in ("ll", "ht") and c.T * c.k <= 2048 and not a.fused_route
                and not a.two_call_dispatch)
    if a.fused_route:
        ops.append(("route_plan", lambda: ep.ep_route_plan(h.ptr, logits, idx, w, LS["s"])))
    else:
        if a.route:
            ops.append(("route", lambda: ep.ep_route(h.ptr, logits, idx, w, LS["s"])))
        if not fused_pd:
            ops.append(("plan", lambda: ep.ep_plan(h.ptr, idx, LS["s"])))
    slot_elems = a.gemm * c.H if a.gemm else PREFETCH_P
    slots = None
    if a.gemm:   # one [N, H] projection per expert, the GEMM's weights
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 * 5 + 7)
        wts = (torch.randn((c.E, a.gemm, c.H), generator=gen, device=dev) * c.H ** -0.5).to(torch.bfloat16)
    elif a.prefetch:
        wts = torch.empty((c.E, PREFETCH_P), dtype=torch.bfloat16, device=dev).fill_(0.5)
    gemm_fp8 = bool(a.gemm and a.fp8)
    pow2 = a.fp8_scales in ("pow2", "amax_pow2w")   # the weights' scale format
    row_pow2 = a.fp8_scales == "pow2"                # the rows' (the FFN's activation)
    if gemm_fp8:   # the weights quantised like the rows (the library's quantiser, the group's format)
        wts, wsc = ep.Buffer.quantize_fp8(wts, pow2=pow2)
        torch.cuda.synchronize()
    if a.prefetch:
        slots = torch.empty((c.R, S) + tuple(wts.shape[1:]), dtype=wts.dtype, device=dev)
        ops.append(("prefetch", lambda: ep.ep_prefetch_replicas(h.ptr, wts, slots, LS["s"])))
        slot_sc = None
        if gemm_fp8:
            slot_sc = torch.empty((c.R, S) + tuple(wsc.shape[1:]), dtype=torch.float32, device=dev)
            ops.append(("prefetch_scales",
                        lambda: ep.ep_prefetch_replicas(h.ptr, wsc, slot_sc, LS["s"], scales=True)))
    if a.fp8:
        # the experts' bf16 outputs (identity experts: the bf16 rows) feed combine
        ep.ep_plan(h.ptr, idx, stream)
        ep.ep_dispatch(h.ptr, x, None, recv, None, None, None, stream)
        if fused_pd:
            ops.append(("plan_dispatch", lambda: ep.ep_plan_dispatch(h.ptr, idx, x, None, rq, rs, None, None,
                                                                     LS["s"])))
        else:
            ops.append(("dispatch", lambda: ep.ep_dispatch(h.ptr, x, None, rq, rs, None, None, LS["s"])))
    elif fused_pd:
        ops.append(("plan_dispatch", lambda: ep.ep_plan_dispatch(h.ptr, idx, x, None, recv, None, None, None,
                                                                 LS["s"])))
    else:
        ops.append(("dispatch", lambda: ep.ep_dispatch(h.ptr, x, None, recv, None, None, None, LS["s"])))
    comb_in = recv
    if a.gemm:
        gy_out = torch.empty((h.recv_rows, a.gemm // 2 if a.swiglu else a.gemm), dtype=torch.bfloat16,
                             device=dev)
        if gemm_fp8:   # straight from the FP8 dispatch output
            rq2d = rq.view(h.recv_rows, c.H)
            ops.append(("gemm", lambda: ep.ep_expert_gemm_fp8(
                h.ptr, rq2d, rs, wts, wsc, slots, slot_sc if a.prefetch else None, gy_out, LS["s"],
                swiglu=a.swiglu)))
        else:
            recv2d = recv.view(h.recv_rows, c.H)
            ops.append(("gemm", lambda: ep.ep_expert_gemm(h.ptr, recv2d, wts, slots, gy_out, LS["s"],
                                                          swiglu=a.swiglu)))
    if a.ffn:   # down projection [E, H, I] back to H; combine gathers its output
        I = a.gemm // 2
        gen2 = torch.Generator(device=dev)
        gen2.manual_seed(1000 * 5 + 11)
        w2 = (torch.randn((c.E, c.H, I), generator=gen2, device=dev) * I ** -0.5).to(torch.bfloat16)
        ffn_out = torch.empty((h.recv_rows, c.H), dtype=torch.bfloat16, device=dev)
        comb_in = ffn_out.view(shape)
        if gemm_fp8:
            w2c, w2s = ep.Buffer.quantize_fp8(w2, pow2=pow2)
            aq = torch.empty((h.recv_rows, I), dtype=torch.float8_e4m3fn, device=dev)
            asc = torch.empty((h.recv_rows, I // 128), dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            del w2
            ops.append(("quantize", lambda: ep.ep_quantize_fp8(gy_out, aq, asc, LS["s"], pow2=row_pow2)))
            ops.append(("gemm2", lambda: ep.ep_expert_gemm_fp8(h.ptr, aq, asc, w2c, w2s, None, None,
                                                               ffn_out, LS["s"])))
        else:
            ops.append(("gemm2", lambda: ep.ep_expert_gemm(h.ptr, gy_out, w2, None, ffn_out, LS["s"])))
    ops.append(("combine", lambda: ep.ep_combine(h.ptr, comb_in, w, y, LS["s"])))
    if train:
        ops.append(("combine_bwd", lambda: ep.ep_combine_bwd(h.ptr, gy, recv, w, gout, gw, LS["s"])))
        ops.append(("dispatch_bwd", lambda: ep.ep_combine(h.ptr, gout, None, gx, LS["s"])))
        ops.append(("dup_reduce", lambda: ep.ep_dup_grad_reduce(h.ptr, rep, rep_e, owner, LS["s"])))

    if not a.graph and not a.no_prepare:
        # each op's C call marshalled once (the library still validates and
        # launches on every call); a graph capture needs the capture stream
        ops = [(nm, ep.prepare(f)) for nm, f in ops]

    def step():
        for _, f in ops:
            f()

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    assert h.status() == 0, "device flags raised on the benchmark input"

    graph = None
    if a.graph:   # the whole step as one HIP graph, replayed (no host launch cost per kernel)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            LS["s"] = torch.cuda.current_stream()
            step()
        LS["s"] = stream
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert h.status() == 0, "device flags raised on the benchmark input (graph replay)"

    def run_step():
        if graph is not None:
            graph.replay()
        else:
            step()

    # timed region 1: the whole step, back to back (or one by one when --cold)
    K = a.steps
    if not a.cold:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_host = time.perf_counter()
        e0.record(stream)
        for i in range(K):
            run_step()
        e1.record(stream)
        torch.cuda.synchronize()
        t_host = time.perf_counter() - t_host
        step_ms = e0.elapsed_time(e1) / K
        median_ms = median_step_ms(run_step, K, stream)
    else:
        tot = 0.0
        steps_cold = []
        t_host = time.perf_counter()
        for _ in range(K):
            evict()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_step()
            e1.record(stream)
            torch.cuda.synchronize()
            tot += e0.elapsed_time(e1)
            steps_cold.append(e0.elapsed_time(e1))
        t_host = time.perf_counter() - t_host
        step_ms = tot / K
        step_list = sorted(steps_cold)
        median_ms = step_list[K // 2] if K % 2 else 0.5 * (step_list[K // 2 - 1] + step_list[K // 2])

    # timed region 2: the same steps with an event pair around every launch
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in ops] for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        if a.cold:
            evict()
        for (nm, f), (b, e) in zip(ops, evs[s]):
            b.record(stream)
            f()
            e.record(stream)
    torch.cuda.synchronize()
    per_us = {nm: 1000.0 * sum(evs[s][i][0].elapsed_time(evs[s][i][1]) for s in range(K)) / K
              for i, (nm, _) in enumerate(ops)}

    filled = int((h.tables()["replica"] >= 0).sum()) if c.layout == "static" and S > 0 else 0
    ab = algorithmic_bytes(c, a.fp8, filled, slot_elems, 1 if gemm_fp8 else 2)
    gemm_info = gemm2_info = None
    if a.gemm:
        tb = h.tables()
        if c.layout == "ll":
            grows = int(torch.clamp(tb["counts"], max=c.cap).sum())
        else:
            grows = int(tb["offsets"][-1])   # every routed entry is one row of some group
        # every weight matrix some row uses (experts with rows, plus the
        # prefetch slots the segments read)
        mats = int((tb["counts"] > 0).sum()) + (filled if a.prefetch else 0)
        n_out = a.gemm // 2 if a.swiglu else a.gemm
        gemm_info = gemm_report(ab, "gemm", per_us["gemm"], grows, mats, a.gemm, c.H, n_out, gemm_fp8,
                                "swiglu" if a.swiglu else "plain")
        if a.ffn:   # the second GEMM reads no prefetch slots
            I = a.gemm // 2
            mats2 = int((tb["counts"] > 0).sum())
            gemm2_info = gemm_report(ab, "gemm2", per_us["gemm2"], grows, mats2, c.H, I, c.H, gemm_fp8,
                                     "plain")
            if gemm_fp8:   # bf16 activation read, codes and scales written
                ab["quantize"] = int(h.recv_rows * I * (2 + 1) + h.recv_rows * (I // 128) * 4)
    chain_bytes = sum(ab[nm] for nm, _ in ops)
    step_s = step_ms / 1000.0
    dom = max((nm for nm in ("dispatch", "plan_dispatch", "combine", "combine_bwd") if nm in per_us),
              key=lambda nm: per_us[nm])
    dom_gbps = ab[dom] / (per_us[dom] * 1e-6) / 1e9
    traffic = traffic_for(f"{name}{'_fp8' if a.fp8 else ''}", dom)
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic, "bytes_per_launch": ab[dom], "avg_us": round(per_us[dom], 2)}

    wl = {"prefill": f"prefill HT T={c.T} H={c.H} E={c.E} top-{c.k} zipf(1.1) bf16",
          "decode": f"decode LL T={c.T} H={c.H} E={c.E} top-{c.k} cap={c.cap}{' fp8' if a.fp8 else ' bf16'}",
          "tiny": f"tiny LL T={c.T} H={c.H} E={c.E} top-{c.k} cap={c.cap} fp32 combine",
          "sweep": f"imbalance sweep STATIC T={c.T} H={c.H} E={c.E} top-{c.k} R={c.R} S={c.S} rho={c.rho:g}",
          "training": f"training fwd+bwd STATIC T={c.T} H={c.H} E={c.E} top-{c.k} R={c.R} S={c.S}"}[name]
    out = {
        "metric": METRIC,
        "value": round(c.T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": a.warmup,
        "ms_per_step": round(step_ms, 4),
        "median_ms_per_step": round(median_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl, "T": c.T, "H": c.H, "E": c.E, "top_k": c.k,
                   "layout": c.layout, "ranks": c.R, "cold_cache": a.cold,
                   "dispatch_stores": a.dispatch_stores, "combine_stores": a.combine_stores,
                   "step": " -> ".join(nm for nm, _ in ops), "from_logits": a.route or a.fused_route,
                   "hip_graph": a.graph, "prepared_calls": not a.graph and not a.no_prepare,
                   "fp8_scales": a.fp8_scales if a.fp8 else None},
        **({"prefetch": {"filled_slots": filled, "slot_bytes": slot_elems * 2}} if a.prefetch else {}),
        **({"gemm": gemm_info} if gemm_info else {}),
        **({"gemm2": gemm2_info} if gemm2_info else {}),
        "hbm_gbps": round(chain_bytes / step_s / 1e9, 1),
        "hbm_frac_of_peak": round(chain_bytes / step_s / 1e9 / HBM_PEAK_GBPS, 4),
        "step_algorithmic_bytes": chain_bytes,
        "kernels_us": {k: round(v, 2) for k, v in per_us.items()},
        "kernels_gbps": {k: round(ab[k] / (per_us[k] * 1e-6) / 1e9, 1) for k in per_us if k in ab},
        "host_wall_s": round(t_host, 6),
        "kernels_algorithmic_bytes": {k: int(ab[k]) for k in per_us if k in ab},
        "roofline": roof,
    }
    if name == "sweep":
        out["config"]["rho"] = c.rho
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(name, a.rho, a.fp8, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
