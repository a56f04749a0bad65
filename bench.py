#!/usr/bin/env python3
"""Benchmark of the MoE dispatch+combine hot path on one MI355X.

One step = one moe_dispatch (routing ordinals, receive-count scan, quantize+scatter) followed
by one moe_combine (top-K weighted gather) over the whole workload, with every input already
resident in HBM.  The expert FFN between them is not part of the path: combine reads a
pre-built expert-output buffer (bf16, or fp16 for a binary16-token workload), one row per
received row.

Prints ONE JSON line.  `value` is whole-job tokens/s: W*BS source tokens per step divided
by the measured time per step.  The `roofline` object is for the dominant kernel (the
combine gather) with its algorithmic bytes per launch divided by its average duration from
HIP events recorded on the launch stream; `traffic` is the measured HBM bytes per launch from
the committed rocprofv3 counter summary when it still matches the kernel source.  The
`cpu_baseline` object times the CPU oracle (single-threaded C) on the same inputs.

Modes (`--mode`): bench (default), copy-calib (a plain device copy of known size, for
scaling the HBM byte counters), ceilings (the dispatch scatter's and the combine gather's
access patterns with their arithmetic taken out, timed beside the library's own dispatch and
combine on the same buffers: the rates those patterns allow on this chip).
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

import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD's published peak
METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (H=7168, K=8, 256 experts)"
DEFAULT_WORKLOAD = "c4_w16_int8_roundtrip"
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "combine_kernel_c4_hbm_traffic.md")
COMBINE_SOURCES = [os.path.join(ROOT, "combine_quant_amd", "csrc", f)
                   for f in ("combine.hip", "dc_device.h")]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sets", type=int, default=3,
                    help="input/output buffer sets rotated across steps (each set is far "
                         "larger than the 256 MB Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-passes", type=int, default=3)
    ap.add_argument("--mode", default="bench", choices=["bench", "copy-calib", "ceilings"])
    ap.add_argument("--graph", action="store_true",
                    help="also capture one step per buffer set into a HIP graph and report the "
                         "replayed step time as the headline (launch gaps removed)")
    return ap.parse_args()


# -- algorithmic bytes (what the method must move; no staging) -----------------------------

def algorithmic_bytes(wl, inp, routed_rows, copy_picks, active_tokens):
    """Bytes dispatch and combine must move for this input (see the design notes).

    dispatch: read x of every token with a routed pick, ids (and mask, smooth table once),
    write each routed row's codes + scales + source triple, expand_idx, ep_recv_count,
    expert_token_nums, recv_offsets.
    combine: read each routed expert-output row once, ids + expand_idx + weights, the
    receive counts (and mask, and ori_x for copy picks), write y."""
    W, E, H, K, T = wl.W, wl.E, wl.H, wl.K, wl.T
    b = 2 if wl.quant_mode == 0 else 0.5 if wl.out_dtype == 4 else 1
    S = scale_bytes_per_row(wl)
    m = 0 if inp.get("mask") is None else inp["mask"].nbytes
    smooth = 0 if inp.get("scales") is None else inp["scales"].nbytes
    P = routed_rows
    dispatch = (2 * H * active_tokens + 4 * T * K + m + smooth + P * (int(b * H) + S + 12)
                + 4 * T * K + 4 * E * W + 8 * E + 8 * (W + 1))
    row = 2 * H if wl.combine_quant == 0 else H + 4 * ((H + 7) // 8)
    if wl.combine_path == "scatter":
        # each routed row and its source triple once, ids + weights, the shared output, y
        combine = (2 * H + 12) * P + 8 * T * K + 8 * (W + 1) + m + 2 * H * copy_picks \
            + 2 * H * T + 2 * H * T
    else:
        combine = row * P + 12 * T * K + 4 * E * W + 8 * (W + 1) + m + 2 * H * copy_picks \
            + 2 * H * T
    return dispatch, combine


def quantize_bytes(wl, routed_rows):
    """Expert-side int8 block quantization: read each routed bf16 row, write its codes and
    Ceil(H, 8) fp32 scales, read recv_offsets."""
    H = wl.H
    return routed_rows * (2 * H + H + 4 * ((H + 7) // 8)) + 8 * (wl.W + 1)


def mx_scales_per_row(H):
    nb = (H + 31) // 32
    return nb + (nb & 1)


def scale_bytes_per_row(wl):
    """dynamic_scales bytes per expand_x row: none (modes 0, 1), one fp32 (mode 2), one fp32
    per 128-group (mode 3), one fp32 or E8M0 byte per 32-block, Align2 (modes 4, 5)."""
    if wl.quant_mode <= 1:
        return 0
    if wl.quant_mode == 2:
        return 4
    if wl.quant_mode == 3:
        return 4 * ((wl.H + 127) // 128)
    return (1 if wl.scale_format == 1 else 4) * mx_scales_per_row(wl.H)


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def combine_kernel_name(wl):
    """The kernel(s) the combine timing of workload `wl` covers."""
    if wl.combine_quant:
        return ("combine_int8_wide_kernel" if wl.H % 16 == 0 and wl.K <= 8
                else "combine_wave_kernel")
    if wl.combine_path == "scatter":
        return "scatter_back_index_kernel + combine_wave_kernel"
    return "combine_wave_kernel"


def committed_traffic():
    """HBM bytes per combine launch from the committed counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None
    text = open(TRAFFIC_SUMMARY).read()
    mh = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    mb = re.search(r"hbm_bytes_per_launch:\s*([0-9]+)", text)
    if not mh or not mb or mh.group(1) != source_hash(COMBINE_SOURCES):
        return None
    return int(mb.group(1))


# -- CPU baseline: the oracle, as it stands ---------------------------------------------

def cpu_baseline(wl, inp, expert_out_host, passes, shared_host=None):
    import oracle
    cfg = oracle.make_cfg(wl.W, wl.E, wl.BS, wl.H, wl.K, quant_mode=wl.quant_mode,
                          zero_expert_num=wl.zero_expert_num,
                          copy_expert_num=wl.copy_expert_num,
                          expert_token_nums_type=wl.expert_token_nums_type,
                          mask_kind=wl.mask_kind, out_dtype=wl.out_dtype,
                          scales_kind=wl.scales_kind, scale_format=wl.scale_format,
                          token_dtype=wl.token_dtype)
    cpus = sorted(os.sched_getaffinity(0))
    os.sched_setaffinity(0, {cpus[0]})          # the oracle is single-threaded; pin it
    times = []
    try:
        for _ in range(passes):
            t0 = time.perf_counter()
            d = oracle.dispatch(cfg, inp["x"], inp["expert_ids"], scales=inp.get("scales"),
                                mask=inp.get("mask"))
            if wl.combine_path == "scatter":
                oracle.combine_scatter(cfg, expert_out_host, d["assist_info"],
                                       d["recv_offsets"], inp["expert_ids"],
                                       inp["expert_scales"], mask=inp.get("mask"),
                                       ori_x=inp["x"], shared_x=shared_host)
            elif wl.combine_quant:
                codes, bsc = oracle.combine_quantize(cfg, expert_out_host, d["recv_offsets"])
                oracle.combine_int8(cfg, codes, bsc, inp["expert_ids"], d["expand_idx"],
                                    inp["expert_scales"], d["ep_recv_count"],
                                    d["recv_offsets"], mask=inp.get("mask"), ori_x=inp["x"])
                del codes, bsc
            else:
                oracle.combine(cfg, expert_out_host, inp["expert_ids"], d["expand_idx"],
                               inp["expert_scales"], d["ep_recv_count"], d["recv_offsets"],
                               mask=inp.get("mask"), ori_x=inp["x"])
            times.append(time.perf_counter() - t0)
            del d
    finally:
        os.sched_setaffinity(0, set(cpus))
    t = statistics.median(times)
    return {"value": round(wl.T / t, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the whole {wl.name} workload ({wl.T} source tokens, dispatch+combine), "
                      f"{passes} passes, median {t:.2f} s; one core of {len(cpus)} available",
            "seconds_per_pass": [round(x, 3) for x in times]}


# -- modes --------------------------------------------------------------------------------

def run_copy_calib(args):
    """A plain device-to-device copy of known size (1 GiB), for scaling HBM counters."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(max(1, args.steps)):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"mode": "copy-calib", "bytes_read_per_launch": n,
                      "bytes_written_per_launch": n, "launches": max(1, args.steps)}))


def _median_us(fn, stream, steps, warmup):
    """Median duration of fn() in microseconds, each call between two events on `stream`."""
    import torch
    for n in range(warmup):
        fn(n)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for n in range(steps):
        evs[n][0].record(stream)
        fn(n)
        evs[n][1].record(stream)
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)


def run_ceilings(args):
    """The scatter's and the gather's access patterns without their arithmetic, from
    libmoe_dc_ceiling.so, next to the library's dispatch and combine (same buffers, same
    rotation of buffer sets).  Prints one JSON line."""
    import ctypes
    import torch
    import combine_quant_amd as cq
    from combine_quant_amd.build import CEILING_LIB

    wl = workloads.WORKLOADS[args.workload]
    if wl.H % 1024 != 0 or wl.quant_mode == 0 or wl.combine_path != "gather":
        sys.exit("ceilings: needs a quantized gather workload with H a multiple of 1024")
    lib = ctypes.CDLL(CEILING_LIB)
    P_, i64, i32 = ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int
    lib.ceiling_scatter_copy.argtypes = [P_, P_, P_, i64, i32, i32, P_]
    lib.ceiling_write_rows.argtypes = [P_, P_, i64, i32, P_]
    lib.ceiling_gather_sum.argtypes = [P_, P_, P_, i64, i32, i32, P_]
    lib.ceiling_write_chunks.argtypes = [P_, i64, i32, P_]
    lib.ceiling_read_chunks.argtypes = [P_, P_, i64, i32, P_]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    inp = workloads.generate(wl, seed=args.seed)
    cfg = cq.make_config(wl.W, wl.E, wl.BS, wl.H, wl.K, wl.quant_mode,
                         zero_expert_num=wl.zero_expert_num, copy_expert_num=wl.copy_expert_num,
                         expert_token_nums_type=wl.expert_token_nums_type,
                         mask_kind=wl.mask_kind, out_dtype=wl.out_dtype,
                         scales_kind=wl.scales_kind, scale_format=wl.scale_format,
                         token_dtype=wl.token_dtype)
    tdt = cq.token_torch_dtype(cfg)

    def dev_t(a, dtype=None):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(dtype) if dtype is not None else t).to(dev)

    ids, mask, smooth = dev_t(inp["expert_ids"]), dev_t(inp.get("mask")), dev_t(inp.get("scales"))
    w = dev_t(inp["expert_scales"])
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    sets = []
    for k in range(args.sets):
        x = dev_t(inp["x"], tdt) if k == 0 else sets[0]["x"].clone()
        st = dict(x=x, eo=workloads.expert_out_torch(wl, wl.cap, seed=args.seed, device=dev),
                  y=torch.empty((wl.W, wl.BS, wl.H), dtype=tdt, device=dev),
                  raw=torch.empty((wl.cap, wl.H), dtype=torch.uint8, device=dev))
        st["dispatch"], st["out"] = cq.prepare_dispatch(cfg, x, ids, smooth, mask)
        o = st["out"]
        st["combine"], _ = cq.prepare_combine(cfg, st["eo"], ids, o["expand_idx"], w,
                                              o["ep_recv_count"], o["recv_offsets"], mask, x,
                                              st["y"])
        sets.append(st)
    for st in sets:
        st["dispatch"]()
    torch.cuda.synchronize()
    o = sets[0]["out"]
    P = int(o["recv_offsets"][-1].item())
    ai = o["assist_info"][:P].long()
    pick = (ai[:, 0] * wl.BS + ai[:, 1]) * wl.K + ai[:, 2]
    dest = torch.full((wl.T * wl.K,), -1, dtype=torch.int32, device=dev)
    dest[pick] = torch.arange(P, dtype=torch.int32, device=dev)       # row of each pick
    order = dest[dest >= 0].contiguous()                              # rows, token-major
    active = int((dest.view(wl.T, wl.K) >= 0).any(dim=1).sum().item())
    ns = len(sets)
    H, T, K = wl.H, wl.T, wl.K
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"ceiling kernel launch failed ({rc})")

    runs = {
        "library_dispatch": (lambda n: sets[n % ns]["dispatch"](), None),
        "scatter_copy": (lambda n: check(lib.ceiling_scatter_copy(
            sets[n % ns]["x"].data_ptr(), dest.data_ptr(), sets[n % ns]["raw"].data_ptr(), T, H,
            K, sp)), 2 * H * active + H * P + 4 * T * K),
        "write_rows_scatter_order": (lambda n: check(lib.ceiling_write_rows(
            sets[n % ns]["raw"].data_ptr(), order.data_ptr(), P, H, sp)), H * P),
        "write_rows_in_sequence": (lambda n: check(lib.ceiling_write_rows(
            sets[n % ns]["raw"].data_ptr(), None, P, H, sp)), H * P),
        # the same bytes in address order, one chunk per one-shot workgroup: 4 KiB is the
        # fastest write shape on this chip; the other sizes show how much the shape matters
        **{f"write_chunks_{c // 1024}k_in_sequence": (lambda n, c=c: check(lib.ceiling_write_chunks(
            sets[n % ns]["raw"].data_ptr(), H * P, c, sp)), H * P)
           for c in (2048, 4096, 7168, 8192, 16384)},
        "library_combine": (lambda n: sets[n % ns]["combine"](), None),
        # the gather's row bytes read in address order, 16 KiB per one-shot workgroup
        "read_chunks_16k_in_sequence": (lambda n: check(lib.ceiling_read_chunks(
            sets[n % ns]["eo"].data_ptr(), sink.data_ptr(), 2 * H * P, 16384, sp)), 2 * H * P),
        "gather_sum": (lambda n: check(lib.ceiling_gather_sum(
            sets[n % ns]["eo"].data_ptr(), dest.data_ptr(), sets[n % ns]["y"].data_ptr(), T, H,
            K, sp)), 2 * H * P + 2 * H * T + 4 * T * K),
    }
    res = {}
    for name, (fn, nbytes) in runs.items():
        us = _median_us(fn, stream, args.steps, args.warmup)
        res[name] = {"median_us": round(us, 2)}
        if nbytes is not None:
            res[name]["bytes"] = nbytes
            res[name]["gbps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    print(json.dumps({"mode": "ceilings", "workload": wl.name, "routed_rows": P,
                      "active_tokens": active, "steps": args.steps, "sets": args.sets,
                      "results": res}), flush=True)


class _NoEvent:
    """Stands in for a timing event inside graph capture, where none is recorded."""

    def record(self, stream=None):
        pass


def run_bench(args):
    import torch
    import combine_quant_amd as cq

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    print(f"[bench] generating {wl.name}", file=sys.stderr, flush=True)
    inp = workloads.generate(wl, seed=args.seed)
    cfg = cq.make_config(wl.W, wl.E, wl.BS, wl.H, wl.K, wl.quant_mode,
                         zero_expert_num=wl.zero_expert_num, copy_expert_num=wl.copy_expert_num,
                         expert_token_nums_type=wl.expert_token_nums_type,
                         mask_kind=wl.mask_kind, out_dtype=wl.out_dtype,
                         scales_kind=wl.scales_kind, scale_format=wl.scale_format,
                         token_dtype=wl.token_dtype)
    tok_dtype = cq.token_torch_dtype(cfg)

    def dev_t(a, dtype=None):
        if a is None:
            return None
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(dtype) if dtype is not None else t).to(dev)

    ids = dev_t(inp["expert_ids"])
    mask = dev_t(inp.get("mask"))
    smooth = dev_t(inp.get("scales"))
    w = dev_t(inp["expert_scales"])
    sets = []
    for k in range(args.sets):
        x = dev_t(inp["x"], tok_dtype) if k == 0 else sets[0]["x"].clone()
        eo = workloads.expert_out_torch(wl, wl.cap, seed=args.seed, device=dev)
        sets.append(dict(x=x, eo=eo, out=cq.alloc_dispatch_outputs(cfg, dev),
                         y=torch.empty((wl.W, wl.BS, wl.H), dtype=tok_dtype, device=dev)))
        if wl.combine_path == "scatter":
            sets[-1]["shared"] = workloads.expert_out_torch(wl, wl.T, seed=args.seed + 1,
                                                            device=dev).view(wl.W, wl.BS, wl.H)
            sets[-1]["sws"] = torch.empty((cq.moe_dc_combine_scatter_workspace_bytes(cfg),),
                                          dtype=torch.uint8, device=dev)
        if wl.combine_quant:
            sets[-1]["codes"] = torch.empty((wl.cap, wl.H), dtype=torch.int8, device=dev)
            sets[-1]["bscales"] = torch.empty((wl.cap, (wl.H + 7) // 8), dtype=torch.float32,
                                              device=dev)
    stream = torch.cuda.current_stream(dev)

    # launch plans: every call's arguments are checked and marshalled once per buffer set
    for st in sets:
        o = st["out"]
        st["dispatch"], _ = cq.prepare_dispatch(cfg, st["x"], ids, smooth, mask, out=o)
        st["quantize"] = None
        if wl.combine_path == "scatter":
            st["combine"], _ = cq.prepare_combine_scatter(
                cfg, st["eo"], o["assist_info"], o["recv_offsets"], ids, w, mask, st["x"],
                st["shared"], st["y"], st["sws"])
        elif wl.combine_quant == 0:
            st["combine"], _ = cq.prepare_combine(cfg, st["eo"], ids, o["expand_idx"], w,
                                                  o["ep_recv_count"], o["recv_offsets"], mask,
                                                  st["x"], st["y"])
        else:
            st["quantize"], _ = cq.prepare_combine_quantize(cfg, st["eo"], o["recv_offsets"],
                                                            (st["codes"], st["bscales"]))
            st["combine"], _ = cq.prepare_combine_int8(cfg, st["codes"], st["bscales"], ids,
                                                       o["expand_idx"], w, o["ep_recv_count"],
                                                       o["recv_offsets"], mask, st["x"],
                                                       st["y"])

    # events made before the timed region, so that the host's per-step work is the launches
    no_events = tuple(_NoEvent() for _ in range(4))
    events = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4))
              for _ in range(max(args.steps, args.warmup))]

    def step(n, stream=stream, timed=True):
        st = sets[n % len(sets)]
        ev = events[n] if timed else no_events
        ev[0].record(stream)
        st["dispatch"](stream)
        ev[1].record(stream)
        if st["quantize"] is not None:
            st["quantize"](stream)
        ev[2].record(stream)
        st["combine"](stream)
        ev[3].record(stream)
        return ev

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for n in range(args.warmup):
        step(n, timed=False)
    torch.cuda.synchronize()
    # 1. the step time: K steps with nothing but their launches between two events
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for n in range(args.steps):
        step(n, timed=False)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    eager_ms_per_step = total_ms / args.steps
    # 2. per-kernel times: the same K steps again, with events around every launch
    evs = [step(n) for n in range(args.steps)]
    torch.cuda.synchronize()

    if args.graph:
        # one graph per buffer set, each holding one whole step; the warm-up above ran every
        # kernel once outside capture
        graphs = []
        for k in range(len(sets)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(k, torch.cuda.current_stream(dev), timed=False)
            graphs.append(g)
        torch.cuda.synchronize()
        for n in range(args.warmup):
            graphs[n % len(graphs)].replay()
        torch.cuda.synchronize()
        print(f"[bench] timing {args.steps} graph replays", file=sys.stderr, flush=True)
        wall0 = time.perf_counter()
        t_start.record(stream)
        for n in range(args.steps):
            graphs[n % len(graphs)].replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        total_ms = t_start.elapsed_time(t_end)
    disp_ms = [e[0].elapsed_time(e[1]) for e in evs]
    quant_ms = [e[1].elapsed_time(e[2]) for e in evs]      # 0 without combine quantization
    comb_ms = [e[2].elapsed_time(e[3]) for e in evs]
    ms_per_step = total_ms / args.steps

    # routed rows etc. of this input, read back from the library's own outputs
    o = sets[0]["out"]
    P = int(o["recv_offsets"][-1].item())
    ids_np = inp["expert_ids"]
    act = np.ones(ids_np.shape, bool) if inp.get("mask") is None else (
        inp["mask"].astype(bool) if inp["mask"].ndim == 3 else
        np.repeat(inp["mask"].astype(bool)[:, :, None], wl.K, axis=2))
    copy_picks = int(((ids_np >= wl.E + wl.zero_expert_num) &
                      (ids_np < wl.n_ids) & act).sum())
    active_tokens = int(((o["expand_idx"] >= 0).any(dim=2)).sum().item())
    d_bytes, c_bytes = algorithmic_bytes(wl, inp, P, copy_picks, active_tokens)
    d_avg = statistics.mean(disp_ms)
    c_avg = statistics.mean(comb_ms)

    def pct(v, q):
        return float(np.percentile(np.asarray(v), q)) * 1e3
    comb_gbps = c_bytes / (c_avg * 1e-3) / 1e9
    disp_gbps = d_bytes / (d_avg * 1e-3) / 1e9
    q_bytes = quantize_bytes(wl, P) if wl.combine_quant else 0
    total_gbps = (d_bytes + q_bytes + c_bytes) / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = wl.T / (ms_per_step * 1e-3)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline ({args.cpu_passes} oracle passes)", file=sys.stderr,
              flush=True)
        eo_host = sets[0]["eo"].view(torch.int16).cpu().numpy().view(np.uint16)
        shared_host = (sets[0]["shared"].view(torch.int16).cpu().numpy().view(np.uint16)
                       if wl.combine_path == "scatter" else None)
        cpu = cpu_baseline(wl, inp, eo_host, args.cpu_passes, shared_host)

    line = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "W": wl.W, "E": wl.E, "BS_per_rank": wl.BS,
                   "H": wl.H, "K": wl.K, "quant_mode": wl.quant_mode,
                   "out_dtype": wl.out_dtype, "scales_kind": wl.scales_kind,
                   "scale_format": wl.scale_format, "token_dtype": wl.token_dtype,
                   "combine_quant": wl.combine_quant,
                   "combine_path": wl.combine_path,
                   "routing": wl.routing, "tokens_per_step": wl.T, "routed_rows": P,
                   "description": wl.description},
        "hbm_gbps": round(total_gbps, 1),
        "hbm_frac": round(total_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(comb_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(comb_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": committed_traffic() if wl.name == DEFAULT_WORKLOAD else None,
                     "kernel": combine_kernel_name(wl),
                     "algorithmic_bytes_per_launch": c_bytes,
                     "avg_launch_us": round(c_avg * 1e3, 2)},
        "dispatch": {"avg_us": round(d_avg * 1e3, 2), "median_us": round(pct(disp_ms, 50), 2),
                     "p90_us": round(pct(disp_ms, 90), 2), "algorithmic_bytes": d_bytes,
                     "gbps": round(disp_gbps, 1), "frac": round(disp_gbps / HBM_PEAK_GBPS, 4)},
        "combine": {"avg_us": round(c_avg * 1e3, 2), "median_us": round(pct(comb_ms, 50), 2),
                    "p90_us": round(pct(comb_ms, 90), 2), "algorithmic_bytes": c_bytes,
                    "gbps": round(comb_gbps, 1)},
        "combine_quantize": None if not wl.combine_quant else {
            "avg_us": round(statistics.mean(quant_ms) * 1e3, 2),
            "algorithmic_bytes": q_bytes,
            "gbps": round(q_bytes / (statistics.mean(quant_ms) * 1e-3) / 1e9, 1)},
        "launch": "hip_graph" if args.graph else "eager",
        "eager_ms_per_step": round(eager_ms_per_step, 4),
        "wall_s_timed": round(wall, 4),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not "
              "supported (how the path would shard across GPUs is described in the design "
              "notes)", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy-calib":
        run_copy_calib(args)
    elif args.mode == "ceilings":
        run_ceilings(args)
    else:
        run_bench(args)


if __name__ == "__main__":
    main()
