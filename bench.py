#!/usr/bin/env python3
"""Benchmark of absorbed-MLA tree-verify attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q9_p16384]

One step = one full verify call (split-KV MFMA kernel + combine kernel) over one
batch of synthetic bf16 inputs already resident in HBM. Prints one JSON line:
value = algorithmic TFLOP/s of the whole call, measured on rotating input
copies (more bytes than the 256 MB MALL, so every call reads its KV from HBM);
the warm figure (same inputs every call) is reported beside it. `roofline`
covers the split kernel, timed alone with HIP events on its stream;
`cpu_baseline` times the fp64 oracle on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
SRC = os.path.join(ROOT, "mla_tree_verify_amd", "csrc", "mla_verify.hip")
PROFILES = os.path.join(ROOT, "profiles")
# the pages' final sm_120 kernel at q_len 9, prefix 16384 (fp32, RTX PRO 6000): 4782.6 us
PAGES_US_Q9_P16384 = 4782.6


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-ms", type=float, default=400.0,
                    help="keep warming up (untimed) until this much GPU time has passed, so clocks settle")
    ap.add_argument("--workload", default="q9_p16384")
    ap.add_argument("--rotate-mb", type=float, default=768.0, help="bytes of rotating input copies (cold run)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target host time of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--copy-calib-mb", type=float, default=0.0,
                    help="after timing, run one device copy of this size (counter calibration)")
    ap.add_argument("--pv-mode", type=int, default=0)
    ap.add_argument("--partials", type=int, default=0, help="0: int16 split partials (default), 1: fp32")
    ap.add_argument("--paged", action="store_true",
                    help="read the KV through a page table (one token per page): the rows scattered over a pool "
                         "by a seeded random permutation, through mla_verify_paged")
    ap.add_argument("--pool-extra", type=int, default=0, help="paged: pool rows beyond the workload's KV rows")
    ap.add_argument("--nsplit", type=int, default=0, help="force the KV split count (0: the planner's)")
    ap.add_argument("--merge", type=int, default=0,
                    help="0: the combine kernel (default), 1: plans of 2..4 splits merge in the split kernel")
    ap.add_argument("--prefix", type=int, default=-1, help="override the workload's prefix length")
    ap.add_argument("--heads", type=int, default=64,
                    help="query heads per token (the workload's shape with this head count; 64 is the metric's)")
    return ap.parse_args()


def source_digest() -> str:
    """sha256[:16] of the kernel source without comments and blank space, so
    that counters stay attached to the code they were taken on across
    comment-only edits."""
    text = open(SRC, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def read_counters(workload: str, paged: bool = False):
    """HBM bytes per split-kernel launch and its MFMA-busy fraction from the
    committed counter summary, or (None, None) when there is none or the
    kernel source changed since."""
    path = os.path.join(PROFILES, f"split_mfma_kernel_{workload}{'_paged' if paged else ''}_counters.txt")
    if not os.path.exists(path):
        return None, None
    kv = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != source_digest():
        return None, None
    try:
        traffic = int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        traffic = None
    try:
        busy = float(kv["mfma_busy_fraction"])
    except (KeyError, ValueError):
        busy = None
    return traffic, busy


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return os.cpu_count() or 1


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the verify operator has no "
                          "multi-GPU path: sharded, each GPU would run the same call on its own heads or "
                          "sequences with no communication",
                          "n_gpus": args.gpus}))
        return 2

    import ctypes

    import numpy as np
    import torch

    import oracle.mla_verify_oracle as orc
    from mla_tree_verify_amd import _lib, api, gen

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = gen.WORKLOADS[args.workload]
    if spec["kind"] != "single":
        print(json.dumps({"error": "bench.py times single-sequence workloads"}))
        return 2
    if args.heads == 64 and args.prefix < 0:
        case = gen.make_workload(args.workload)
    else:
        kw = dict(gen.WORKLOADS[args.workload])
        kw.pop("kind")
        if args.prefix >= 0:
            kw["prefix_len"] = args.prefix
        case = gen.make_case(num_heads=args.heads, **kw)
    q, p = case.q_len, case.prefix_len
    n = p + q
    H = args.heads
    flops = orc.algorithmic_flops(case.tree_parent, p, num_heads=H)
    alg_bytes = orc.algorithmic_bytes(q, n, num_heads=H)
    plan = api.device_plan(q, 1, n, n, nsplit=args.nsplit, pv_mode=args.pv_mode, num_heads=H,
                           partials=args.partials, merge=args.merge)
    lib = _lib.load()
    ws_bytes = _lib.workspace_size(q, H, 1, n, n, nsplit=args.nsplit, pv_mode=args.pv_mode, partials=args.partials,
                                   merge=args.merge)

    host = {k: getattr(case, k) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}
    if args.paged:
        pg = gen.make_paged(case, seed=1234, extra_rows=args.pool_extra)
        host["kv_latent"], host["k_rope"] = pg.pool_latent, pg.pool_rope
        host["kv_index"] = pg.kv_index
    per_copy = sum(t.numel() * t.element_size() for t in host.values()) + ws_bytes + q * H * 513 * 4
    ncopy = max(2, math.ceil(args.rotate_mb * 2**20 / per_copy))
    copies = []
    for _ in range(ncopy):
        d = {k: v.to(dev) for k, v in host.items()}
        d["out"] = torch.empty(q, H, 512, dtype=torch.float32, device=dev)
        d["lse"] = torch.empty(q, H, dtype=torch.float32, device=dev)
        d["ws"] = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        copies.append(d)
    stream = torch.cuda.current_stream(dev)
    # Each timed call goes straight to the C ABI with prebuilt arguments, so
    # that host-side argument handling does not gap the back-to-back launches.
    # phase 0 = the whole call, 1 = the split kernel alone, 2 = the combine
    # kernel alone (on the workspace phase 1 filled; nothing when the split
    # kernel merges the splits itself).
    opts = [_lib.options(args.nsplit, args.pv_mode, 0, args.partials, ph, args.merge) for ph in range(3)]
    entry = lib.mla_verify_paged if args.paged else lib.mla_verify_ex
    for d in copies:
        if args.paged:
            d["args"] = [(d["q_nope"].data_ptr(), d["q_rope"].data_ptr(), d["kv_latent"].data_ptr(),
                          d["k_rope"].data_ptr(), d["kv_index"].data_ptr(), int(d["kv_latent"].shape[0]),
                          d["tree_parent"].data_ptr(), None, 1, n, n, ctypes.c_float(case.scale),
                          d["out"].data_ptr(), d["lse"].data_ptr(), q, H, d["ws"].data_ptr(), ws_bytes,
                          stream.cuda_stream, ctypes.byref(opts[ph])) for ph in range(3)]
        else:
            d["args"] = [(d["q_nope"].data_ptr(), d["q_rope"].data_ptr(), d["kv_latent"].data_ptr(),
                          d["k_rope"].data_ptr(), d["tree_parent"].data_ptr(), p, ctypes.c_float(case.scale),
                          d["out"].data_ptr(), d["lse"].data_ptr(), q, H, d["ws"].data_ptr(), ws_bytes,
                          stream.cuda_stream, ctypes.byref(opts[ph])) for ph in range(3)]
    for ph in range(3):
        rc = entry(*copies[0]["args"][ph])
        if rc != _lib.MLAV_OK:
            raise _lib.MLAVError(rc, f"verify call (phase {ph})")

    def call(d):
        entry(*d["args"][0])

    def warm(fn, rotate: bool = True) -> None:
        # W untimed steps, then more until warmup_ms of wall time has passed
        t0 = time.perf_counter()
        i = 0
        while i < args.warmup or (time.perf_counter() - t0) * 1e3 < args.warmup_ms:
            fn(copies[i % ncopy] if rotate else copies[0])
            i += 1
            if i % 50 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()

    def timed(rotate: bool) -> float:
        warm(call, rotate)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            call(copies[i % ncopy] if rotate else copies[0])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps  # us per call

    us_warm = timed(rotate=False)
    us_cold = timed(rotate=True)

    # each kernel alone: K back-to-back launches (rotating inputs) between two
    # events recorded on the stream the library launches on
    def split(d):
        entry(*d["args"][1])

    def merge(d):
        entry(*d["args"][2])

    def batch_us(fn) -> float:
        warm(fn)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(args.steps):
            fn(copies[i % ncopy])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / args.steps

    split_us = batch_us(split)
    combine_us = batch_us(merge) if plan.combine == 1 else 0.0

    # The whole call replayed from a HIP graph, as a serving loop would issue
    # it: one graph makes the call on every input copy in turn (cold, like
    # us_cold). Inside the capture the launches go to the capture stream, so
    # the arguments carry that stream. The replayed output must equal the
    # eager output bit for bit (the kernels are deterministic).
    graph_us = graph_equal = None
    if not args.no_graph:
        d0 = copies[0]
        call(d0)
        torch.cuda.synchronize()
        eager = (d0["out"].clone(), d0["lse"].clone())
        d0["out"].zero_()
        d0["lse"].zero_()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        with torch.cuda.graph(g, stream=cap):
            for d in copies:
                a = list(d["args"][0])
                a[-2] = cap.cuda_stream
                rc = entry(*a)
                if rc != _lib.MLAV_OK:
                    raise _lib.MLAVError(rc, "verify call under graph capture")
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < 100.0:
            g.replay()
            torch.cuda.synchronize()
        reps = max(1, args.steps // ncopy)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_us = e0.elapsed_time(e1) * 1e3 / (reps * ncopy)
        graph_equal = bool(torch.equal(d0["out"], eager[0]) and torch.equal(d0["lse"], eager[1]))
        del g

    if args.copy_calib_mb > 0:
        nb = int(args.copy_calib_mb * 2**20) // 4 * 4
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    # parity of the benchmarked output against the oracle (also the CPU baseline)
    d0 = copies[0]
    call(d0)
    torch.cuda.synchronize()
    out = d0["out"].cpu().double().numpy()
    lse = d0["lse"].cpu().double().numpy()
    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        reps, t_cpu = 0, 0.0
        ro = rl = None
        t_start = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            ro, rl = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent, p,
                                    case.scale)
            t_cpu += time.perf_counter() - t0
            reps += 1
            if t_cpu >= args.cpu_seconds or time.perf_counter() - t_start > 30.0:
                break
        cpu = {"value": flops * reps / t_cpu / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"the full {args.workload} workload, {reps} oracle call(s), fp64 numpy, "
                         f"{t_cpu:.1f} s; us/call {t_cpu / reps * 1e6:.0f}"}
        err = np.abs(out - ro)
        parity = {"max_abs_err": float(err.max()),
                  "worst_err_over_tol": float((err / (2e-3 + 1e-2 * np.abs(ro))).max()),
                  "lse_max_abs_err": float(np.abs(lse - rl).max())}

    tflops = flops / (us_cold * 1e-6) / 1e12
    tflops_warm = flops / (us_warm * 1e-6) / 1e12
    achieved = flops / (split_us * 1e-6) / 1e12
    traffic, mfma_busy = read_counters(args.workload, args.paged) if H == 64 else (None, None)
    res = {
        "metric": "MLA verify attention us/call + TFLOP/s (% MFMA peak), H=64 q_len=9, prefix 16k",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_cold / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / (flops / (PAGES_US_Q9_P16384 * 1e-6) / 1e12), 2)
        if args.workload == "q9_p16384" and H == 64 and not args.paged and args.prefix < 0 else None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "q_len": q, "prefix": p, "kv_len": n, "heads": H, "dl": 512,
                   "dr": 64, "tree": case.meta["tree"], "scale": case.scale, "nsplit": plan.nsplit,
                   "chunk": plan.chunk, "pv_mode": args.pv_mode, "partials": "int16" if args.partials == 0 else "fp32",
                   "merge": ["none (one split)", "combine kernel", "in the split kernel"][plan.combine],
                   "kv_layout": (f"paged, one token per page, pool {n + args.pool_extra} rows" if args.paged
                                 else "contiguous"),
                   "parallelism": "single GPU"},
        "us_per_call": round(us_cold, 2),
        "us_per_call_warm": round(us_warm, 2),
        "us_per_call_graph": None if graph_us is None else round(graph_us, 2),
        "graph_replay_equals_eager": graph_equal,
        "tflops_warm": round(tflops_warm, 2),
        "pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "hbm_gbs_algorithmic": round(alg_bytes / (us_cold * 1e-6) / 1e9, 1),
        "pct_hbm_peak": round(100 * alg_bytes / (us_cold * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
        "split_kernel_us": round(split_us, 2),
        "combine_kernel_us": round(combine_us, 2),
        "algorithmic_gflop": round(flops / 1e9, 3),
        "algorithmic_mb": round(alg_bytes / 1e6, 3),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "split_mfma_kernel", "algorithmic_flop_per_launch": flops,
                     "mfma_busy_counter": mfma_busy},
        "cpu_baseline": cpu,
        "parity": parity,
        "baseline_note": "vs_baseline divides by the pages' final sm_120 kernel at q9/16k (4782.6 us, fp32, RTX PRO "
                         "6000): context from other hardware, not a target",
    }
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
