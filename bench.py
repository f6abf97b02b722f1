#!/usr/bin/env python3
"""Benchmark of absorbed-MLA tree-verify attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload q9_p16384]

One step = one full verify call (split-KV MFMA kernel + combine kernel) over one
batch of synthetic bf16 inputs already resident in HBM. Prints one JSON line:
value = algorithmic TFLOP/s of the whole call on the headline workload,
measured on rotating input copies (more bytes than the 256 MB MALL, so every
call reads its KV from HBM); the warm figure (same inputs every call) is
reported beside it. `roofline` covers the split kernel, timed alone with HIP
events on its stream; `cpu_baseline` times the fp64 oracle on the host cores.
`configs` times the other workloads (cold whole call, warm, split kernel
alone) in the same run, and `measured_peaks` gives the bf16 MFMA throughput
this GPU sustains under a pure MFMA load and a device-to-device copy rate.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
SRC = os.path.join(ROOT, "mla_tree_verify_amd", "csrc", "mla_verify.hip")
PROFILES = os.path.join(ROOT, "profiles")
PROBE_LIB = os.path.join(ROOT, "mla_tree_verify_amd", "libmla_verify_probe.so")
# the pages' final sm_120 kernel at q_len 9, prefix 16384 (fp32, RTX PRO 6000): 4782.6 us
PAGES_US_Q9_P16384 = 4782.6
# the other workloads timed in the same run (the headline one is --workload)
EXTRA_WORKLOADS = ("q9_p256", "q9_p4096", "q33_p16384_peaky", "q9_p65536_chain", "b8_ragged_q33")


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
    ap.add_argument("--no-extra-configs", action="store_true", help="time the headline workload only")
    ap.add_argument("--no-peaks", action="store_true", help="skip the MFMA and copy peak measurements")
    ap.add_argument("--peaks-only", action="store_true",
                    help="print the measured MFMA and copy peaks as one JSON line and exit")
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
    """HBM bytes per split-kernel launch and its MFMA-busy fractions from the
    committed counter summary, or (None, None) when there is none or the
    kernel source changed since. The fractions: MFMA busy cycles over the SIMD
    cycles of the CUs while they held a workgroup, and over all SIMDs in the
    dispatch's GPU-active window (a lower bound: for a short dispatch that
    window also holds the profiler's launch and drain)."""
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
        busy = {"on_occupied_cus": float(kv["mfma_busy_fraction"]),
                "gpu_window_lower_bound": float(kv["mfma_busy_fraction_gpu_window"])}
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


class Runner:
    """One workload on the GPU: rotating input copies, prebuilt C-ABI
    argument tuples for phase 0 (the whole call), 1 (split kernel alone) and
    2 (combine kernel alone), and HIP-event timing on the library's stream.
    Each timed call goes straight to the C ABI with prebuilt arguments, so that
    host-side argument handling does not gap the back-to-back launches."""

    def __init__(self, case, args, dev, heads, paged=False, pool_extra=0):
        import torch

        import oracle.mla_verify_oracle as orc
        from mla_tree_verify_amd import _lib, api, gen

        self.torch, self.case, self.args, self.dev = torch, case, args, dev
        self.lib = _lib.load()
        self._lib = _lib
        q, H = case.q_len, heads
        self.q, self.H = q, H
        if case.batched:
            offs = case.kv_offsets.tolist()
            lens = [offs[b + 1] - offs[b] for b in range(len(offs) - 1)]
            self.batch, self.total, self.max_kv = len(lens), offs[-1], max(lens)
            parents = case.tree_parent.tolist()
            self.flops = sum(orc.algorithmic_flops(parents[b], lens[b] - q, num_heads=H) for b in range(self.batch))
            self.alg_bytes = sum(orc.algorithmic_bytes(q, lens[b], num_heads=H) for b in range(self.batch))
        else:
            n = case.prefix_len + q
            self.batch, self.total, self.max_kv = 1, n, n
            self.flops = orc.algorithmic_flops(case.tree_parent, case.prefix_len, num_heads=H)
            self.alg_bytes = orc.algorithmic_bytes(q, n, num_heads=H)
        self.plan = api.device_plan(q, self.batch, self.total, self.max_kv, nsplit=args.nsplit, pv_mode=args.pv_mode,
                                    num_heads=H, partials=args.partials, merge=args.merge)
        self.ws_bytes = _lib.workspace_size(q, H, self.batch, self.total, self.max_kv, nsplit=args.nsplit,
                                            pv_mode=args.pv_mode, partials=args.partials, merge=args.merge)
        host = {k: getattr(case, k) for k in ("q_nope", "q_rope", "kv_latent", "k_rope", "tree_parent")}
        if case.batched:
            host["kv_offsets"] = case.kv_offsets
        self.paged = paged
        if paged:
            pg = gen.make_paged(case, seed=1234, extra_rows=pool_extra)
            host["kv_latent"], host["k_rope"] = pg.pool_latent, pg.pool_rope
            host["kv_index"] = pg.kv_index
        out_shape = tuple(case.q_nope.shape[:-1]) + (512,)
        lse_shape = tuple(case.q_nope.shape[:-1])
        per_copy = (sum(t.numel() * t.element_size() for t in host.values()) + self.ws_bytes
                    + self.batch * q * H * 513 * 4)
        self.ncopy = max(2, math.ceil(args.rotate_mb * 2**20 / per_copy))
        self.copies = []
        for _ in range(self.ncopy):
            d = {k: v.to(dev) for k, v in host.items()}
            d["out"] = torch.empty(out_shape, dtype=torch.float32, device=dev)
            d["lse"] = torch.empty(lse_shape, dtype=torch.float32, device=dev)
            d["ws"] = torch.empty(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)
            self.copies.append(d)
        self.stream = torch.cuda.current_stream(dev)
        opts = [_lib.options(args.nsplit, args.pv_mode, 0, args.partials, ph, args.merge) for ph in range(3)]
        self.opts = opts  # the tuples below hold pointers into these
        sc = ctypes.c_float(case.scale)
        if paged:
            self.entry = self.lib.mla_verify_paged
        elif case.batched:
            self.entry = self.lib.mla_verify_batched
        else:
            self.entry = self.lib.mla_verify_ex
        for d in self.copies:
            if paged:
                offs_ptr = d["kv_offsets"].data_ptr() if case.batched else None
                d["args"] = [(d["q_nope"].data_ptr(), d["q_rope"].data_ptr(), d["kv_latent"].data_ptr(),
                              d["k_rope"].data_ptr(), d["kv_index"].data_ptr(), int(d["kv_latent"].shape[0]),
                              d["tree_parent"].data_ptr(), offs_ptr, self.batch, self.total, self.max_kv, sc,
                              d["out"].data_ptr(), d["lse"].data_ptr(), q, H, d["ws"].data_ptr(), self.ws_bytes,
                              self.stream.cuda_stream, ctypes.byref(opts[ph])) for ph in range(3)]
            elif case.batched:
                d["args"] = [(d["q_nope"].data_ptr(), d["q_rope"].data_ptr(), d["kv_latent"].data_ptr(),
                              d["k_rope"].data_ptr(), d["tree_parent"].data_ptr(), d["kv_offsets"].data_ptr(),
                              self.batch, self.total, self.max_kv, sc, d["out"].data_ptr(), d["lse"].data_ptr(), q,
                              H, d["ws"].data_ptr(), self.ws_bytes, self.stream.cuda_stream,
                              ctypes.byref(opts[ph])) for ph in range(3)]
            else:
                d["args"] = [(d["q_nope"].data_ptr(), d["q_rope"].data_ptr(), d["kv_latent"].data_ptr(),
                              d["k_rope"].data_ptr(), d["tree_parent"].data_ptr(), case.prefix_len, sc,
                              d["out"].data_ptr(), d["lse"].data_ptr(), q, H, d["ws"].data_ptr(), self.ws_bytes,
                              self.stream.cuda_stream, ctypes.byref(opts[ph])) for ph in range(3)]
        for ph in range(3):
            rc = self.entry(*self.copies[0]["args"][ph])
            if rc != _lib.MLAV_OK:
                raise _lib.MLAVError(rc, f"verify call (phase {ph})")

    def call(self, d, phase=0):
        self.entry(*d["args"][phase])

    def warm(self, phase=0, rotate=True):
        # W untimed steps, then more until warmup_ms of wall time has passed
        t0 = time.perf_counter()
        i = 0
        while i < self.args.warmup or (time.perf_counter() - t0) * 1e3 < self.args.warmup_ms:
            self.call(self.copies[i % self.ncopy] if rotate else self.copies[0], phase)
            i += 1
            if i % 50 == 0:
                self.torch.cuda.synchronize()
        self.torch.cuda.synchronize()

    def timed(self, phase=0, rotate=True) -> float:
        """us per call: K back-to-back launches between two events on the library's stream."""
        torch = self.torch
        self.warm(phase, rotate)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for i in range(self.args.steps):
            self.call(self.copies[i % self.ncopy] if rotate else self.copies[0], phase)
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / self.args.steps

    def graph_us(self):
        """The whole call replayed from a HIP graph (one graph makes the call on
        every input copy in turn: cold, like the eager figure), and whether
        the replayed output equals the eager one bit for bit."""
        torch, _lib = self.torch, self._lib
        d0 = self.copies[0]
        self.call(d0)
        torch.cuda.synchronize()
        eager = (d0["out"].clone(), d0["lse"].clone())
        d0["out"].zero_()
        d0["lse"].zero_()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(self.dev)
        with torch.cuda.graph(g, stream=cap):
            for d in self.copies:
                a = list(d["args"][0])
                a[-2] = cap.cuda_stream  # inside the capture the launches go to the capture stream
                rc = self.entry(*a)
                if rc != _lib.MLAV_OK:
                    raise _lib.MLAVError(rc, "verify call under graph capture")
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < 100.0:
            g.replay()
            torch.cuda.synchronize()
        reps = max(1, self.args.steps // self.ncopy)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(reps):
            g.replay()
        e1.record(self.stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * self.ncopy)
        equal = bool(torch.equal(d0["out"], eager[0]) and torch.equal(d0["lse"], eager[1]))
        del g
        return us, equal

    def release(self):
        self.copies = []
        self.torch.cuda.empty_cache()


def measured_peaks(torch, dev, num_cus: int) -> dict:
    """bf16 MFMA throughput under a pure MFMA load (the probe library: one
    wave per SIMD on every CU issuing independent 32x32x16 MFMAs) and the
    rate of a 1 GiB device-to-device copy (bytes read + written)."""
    res = {}
    if os.path.exists(PROBE_LIB):
        probe = ctypes.CDLL(PROBE_LIB)
        probe.mlav_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p]
        probe.mlav_probe_mfma.restype = ctypes.c_int32
        probe.mlav_probe_mfma_per_wave.restype = ctypes.c_int32
        grid, iters = num_cus, 4000
        out = torch.empty(grid * 256, dtype=torch.float32, device=dev)
        cyc = torch.empty(grid * 4, dtype=torch.int64, device=dev)
        stream = torch.cuda.current_stream(dev)
        for _ in range(3):
            if probe.mlav_probe_mfma(grid, iters, out.data_ptr(), cyc.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("MFMA probe launch failed")
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        probe.mlav_probe_mfma(grid, iters, out.data_ptr(), cyc.data_ptr(), stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        per_wave = probe.mlav_probe_mfma_per_wave()
        mfmas = grid * 4 * iters * per_wave
        cycles = float(cyc.double().mean().item())
        res["mfma_bf16_tflops"] = round(mfmas * 32768 / (ms * 1e-3) / 1e12, 1)
        res["mfma_clock_ghz"] = round(cycles / (ms * 1e-3) / 1e9, 3)  # shader clock under the MFMA load
        res["mfma_cycles_per_instruction"] = round(cycles / (iters * per_wave), 2)
        res["mfma_probe"] = (f"{grid} workgroups x 4 waves (one per SIMD), {iters * per_wave} independent "
                             "v_mfma_f32_32x32x16_bf16 per wave over 8 accumulators")
        # the split kernel's loop step as a bare data flow: cycles per step with
        # each part added to its 50 MFMAs per wave (1600 cycles at 32 per MFMA)
        probe.mlav_probe_step_mix.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        probe.mlav_probe_step_mix.restype = ctypes.c_int32
        probe.mlav_probe_steps_per_iteration.restype = ctypes.c_int32
        src = torch.zeros(64 << 20, dtype=torch.uint8, device=dev)  # MLAV_MIX_SRC_BYTES
        mix_iters = 250
        steps = mix_iters * probe.mlav_probe_steps_per_iteration()
        mix = {}
        for name, parts in (("mfma", 0), ("mfma+lds", 1), ("mfma+dma", 2), ("mfma+lds+dma", 3),
                            ("mfma+lds+dma+barriers", 7)):
            for _ in range(2):
                if probe.mlav_probe_step_mix(grid, mix_iters, parts, src.data_ptr(), out.data_ptr(), cyc.data_ptr(),
                                             stream.cuda_stream) != 0:
                    raise RuntimeError("step-mix probe launch failed")
            torch.cuda.synchronize()
            mix[name] = round(float(cyc.double().mean().item()) / steps, 1)
        res["step_mix_cycles"] = mix
        res["step_mix_probe"] = ("the split kernel's loop step without its data dependencies, cycles per 32-key "
                                 "step: 50 MFMAs per wave, plus its LDS operand reads (136 KB per CU), its nine 1 KB "
                                 "direct-to-LDS tile loads per wave and its two barriers")
        del src
    nb = 1 << 30
    src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    res["hbm_copy_gbs"] = round(2 * nb / (ms * 1e-3) / 1e9, 1)
    res["hbm_copy"] = "1 GiB fp32 device-to-device copy (torch copy_), read + written bytes"
    del src, dst
    torch.cuda.empty_cache()
    return res


def config_summary(r: Runner, us: float, us_warm: float, split_us: float, peaks: dict) -> dict:
    tf = r.flops / (us * 1e-6) / 1e12
    d = {"us_per_call": round(us, 2), "us_per_call_warm": round(us_warm, 2), "split_kernel_us": round(split_us, 2),
         "tflops": round(tf, 2), "pct_mfma_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
         "split_kernel_tflops": round(r.flops / (split_us * 1e-6) / 1e12, 2),
         "split_kernel_frac": round(r.flops / (split_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
         "hbm_gbs_algorithmic": round(r.alg_bytes / (us * 1e-6) / 1e9, 1),
         "pct_hbm_peak": round(100 * r.alg_bytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 2),
         "algorithmic_gflop": round(r.flops / 1e9, 3), "algorithmic_mb": round(r.alg_bytes / 1e6, 3),
         "nsplit": int(r.plan.nsplit), "chunk": int(r.plan.chunk), "batch": r.batch, "q_len": r.q,
         "kv_rows": r.total}
    if peaks.get("mfma_bf16_tflops"):
        d["pct_measured_mfma_peak"] = round(100 * tf / peaks["mfma_bf16_tflops"], 2)
    if r.case.batched:
        d["prefixes"] = list(r.case.prefix_lens)
    return d


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the verify operator has no "
                          "multi-GPU path: sharded, each GPU would run the same call on its own heads or "
                          "sequences with no communication",
                          "n_gpus": args.gpus}))
        return 2

    import numpy as np
    import torch

    import oracle.mla_verify_oracle as orc
    from mla_tree_verify_amd import _lib, gen

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    num_cus = torch.cuda.get_device_properties(dev).multi_processor_count
    _lib.load()
    peaks = {} if args.no_peaks else measured_peaks(torch, dev, num_cus)
    if args.peaks_only:
        print(json.dumps({"measured_peaks": peaks}))
        return 0

    spec = gen.WORKLOADS[args.workload]
    H = args.heads
    if spec["kind"] != "single" and (args.heads != 64 or args.prefix >= 0):
        print(json.dumps({"error": "--heads and --prefix apply to single-sequence workloads"}))
        return 2
    if args.heads == 64 and args.prefix < 0:
        case = gen.make_workload(args.workload)
    else:
        kw = dict(spec)
        kw.pop("kind")
        if args.prefix >= 0:
            kw["prefix_len"] = args.prefix
        case = gen.make_case(num_heads=args.heads, **kw)
    run = Runner(case, args, dev, H, paged=args.paged, pool_extra=args.pool_extra)
    q, p = case.q_len, case.prefix_len
    plan = run.plan

    us_warm = run.timed(0, rotate=False)
    us_cold = run.timed(0, rotate=True)
    split_us = run.timed(1)
    combine_us = run.timed(2) if plan.combine == 1 else 0.0
    graph_us = graph_equal = None
    if not args.no_graph:
        graph_us, graph_equal = run.graph_us()

    if args.copy_calib_mb > 0:
        nb = int(args.copy_calib_mb * 2**20) // 4 * 4
        src = torch.empty(nb // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()

    # parity of the benchmarked output against the oracle (also the CPU baseline)
    d0 = run.copies[0]
    run.call(d0)
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
            if case.batched:
                ro, rl = orc.mla_verify_batched(case.q_nope, case.q_rope, case.kv_latent, case.k_rope,
                                                case.tree_parent, case.kv_offsets, case.scale)
            else:
                ro, rl = orc.mla_verify(case.q_nope, case.q_rope, case.kv_latent, case.k_rope, case.tree_parent,
                                        p, case.scale)
            t_cpu += time.perf_counter() - t0
            reps += 1
            if t_cpu >= args.cpu_seconds or time.perf_counter() - t_start > 30.0:
                break
        try:
            affinity = len(os.sched_getaffinity(0))
        except AttributeError:
            affinity = None
        cpu = {"value": run.flops * reps / t_cpu / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
               "sample": f"the full {args.workload} workload, {reps} oracle call(s), fp64 numpy, "
                         f"{t_cpu:.1f} s; us/call {t_cpu / reps * 1e6:.0f}",
               "blas_threads": blas_threads(), "os_cpu_count": os.cpu_count(), "sched_affinity_cores": affinity}
        err = np.abs(out - ro)
        parity = {"max_abs_err": float(err.max()),
                  "worst_err_over_tol": float((err / (2e-3 + 1e-2 * np.abs(ro))).max()),
                  "lse_max_abs_err": float(np.abs(lse - rl).max())}

    flops, alg_bytes = run.flops, run.alg_bytes
    tflops = flops / (us_cold * 1e-6) / 1e12
    tflops_warm = flops / (us_warm * 1e-6) / 1e12
    achieved = flops / (split_us * 1e-6) / 1e12
    traffic, mfma_busy = read_counters(args.workload, args.paged) if H == 64 else (None, None)
    headline_plain = (args.workload == "q9_p16384" and H == 64 and not args.paged and args.prefix < 0)
    run.release()

    # the other workloads, same run: cold whole call, warm, split kernel alone
    configs = {}
    if not args.no_extra_configs:
        for name in EXTRA_WORKLOADS:
            if name == args.workload:
                continue
            r = Runner(gen.make_workload(name), args, dev, 64)
            u_cold = r.timed(0, rotate=True)
            u_warm = r.timed(0, rotate=False)
            u_split = r.timed(1)
            configs[name] = config_summary(r, u_cold, u_warm, u_split, peaks)
            c_traffic, c_busy = read_counters(name)
            if c_traffic is not None:
                configs[name]["split_kernel_hbm_bytes"] = c_traffic
            if c_busy is not None:
                configs[name]["split_kernel_mfma_busy"] = c_busy
            r.release()

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
        "vs_baseline": round(tflops / (flops / (PAGES_US_Q9_P16384 * 1e-6) / 1e12), 2) if headline_plain else None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "q_len": q, "prefix": p, "kv_len": run.total, "heads": H, "dl": 512,
                   "dr": 64, "tree": case.meta["tree"], "scale": case.scale, "nsplit": plan.nsplit,
                   "chunk": plan.chunk, "pv_mode": args.pv_mode, "partials": "int16" if args.partials == 0 else "fp32",
                   "merge": ["none (one split)", "combine kernel", "in the split kernel"][plan.combine],
                   "kv_layout": (f"paged, one token per page, pool {run.total + args.pool_extra} rows" if args.paged
                                 else "contiguous"),
                   "parallelism": "single GPU"},
        "us_per_call": round(us_cold, 2),
        "us_per_call_warm": round(us_warm, 2),
        "us_per_call_graph": None if graph_us is None else round(graph_us, 2),
        "graph_replay_equals_eager": graph_equal,
        "tflops_warm": round(tflops_warm, 2),
        "pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "pct_measured_mfma_peak": (round(100 * tflops / peaks["mfma_bf16_tflops"], 2)
                                   if peaks.get("mfma_bf16_tflops") else None),
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
        "measured_peaks": peaks or None,
        "configs": configs or None,
        "baseline_note": "vs_baseline divides by the pages' final sm_120 kernel at q9/16k (4782.6 us, fp32, RTX PRO "
                         "6000): context from other hardware, not a target",
    }
    print(json.dumps(res))
    return 0


if __name__ == "__main__":
    sys.exit(main())
