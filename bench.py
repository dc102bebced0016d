#!/usr/bin/env python3
"""Benchmark of the fused exact-attention hot path on one MI355X.

Default run (one JSON line on stdout): the training-step workload — B=2,
H=16, N=16384, d=128, bf16, causal, Q/K/V/dO ~ N(0,1) from seed 5 — where a
step is fa_fwd followed by fa_bwd (every stage of the path). Throughput is
attention TFLOP/s by the usual convention: forward 4·B·H·N²·d, halved for
causal; backward 2.5× the forward.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --sweep     # forward TFLOP/s for every forward workload, one line each
    python bench.py --fp8-sweep # fa_fwd vs fa_fwd_fp8 on the d = 128 forward workloads
    python bench.py --workload decode_llama   # decode over a KV cache: HBM GB/s, one line
    python bench.py --pmc-step  # one calibration copy + one step, for rocprofv3 --pmc runs
    python bench.py --pmc-summary FETCH_DIR WRITE_DIR   # counters -> profiles/traffic_<workload>.json
    python bench.py --split-sweep decode_llama_fp8,16-32-8-4-8192-e4m3-128   # decode: every split count

HBM traffic (roofline.traffic) comes from two rocprofv3 --pmc runs of
--pmc-step, one collecting FETCH_SIZE and one WRITE_SIZE. Both counters are
scaled by what they read for a plain copy of known size in the same process
(torch.neg over a 256 MiB bf16 tensor: 256 MiB read, 256 MiB written).
--pmc-summary stores the result with a hash of the kernel sources; the step
bench reports it only while the sources still hash the same, else null.

Inputs are resident in device memory before the timed region starts. The
timed region is exactly K steps through the entry points (fa_fwd + fa_bwd, or
fa_fwd_kvcache) bracketed by device synchronisation, timed with HIP events on
the stream the kernels are launched on; `value` and `ms_per_step` come from
it. A second pass of K steps calls the stages one by one with an event after
every launch, for each kernel's average duration (`kernel_ms`, the roofline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_FP8_TFLOPS = 5033.2    # dense fp8 (e4m3) MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="train_16k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--smi", metavar="PATH",
                   help="with --sweep: read amd-smi (clock, power, temperature) while each "
                        "workload of >= 1 ms per call runs, into PATH as JSON")
    p.add_argument("--sweep", action="store_true",
                   help="time fa_fwd on every forward workload (10 warmup, 100 timed calls)")
    p.add_argument("--fp8-sweep", action="store_true",
                   help="time fa_fwd and fa_fwd_fp8 on the d = 128 forward workloads")
    p.add_argument("--names", default=None,
                   help="comma-separated workload names for --sweep / --fp8-sweep")
    p.add_argument("--pmc-step", action="store_true",
                   help="one calibration copy and one fa_fwd + fa_bwd step (for counter runs)")
    p.add_argument("--split-sweep", metavar="SHAPES", default=None,
                   help="decode: time every key-range count on each shape, one JSON line per shape; "
                        "SHAPES is a comma-separated list of decode workload names or "
                        "B-Hq-Hkv-Nq-Nk-cache-d specs (cache: same or e4m3; bf16 queries, causal)")
    p.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn FETCH_SIZE / WRITE_SIZE counter runs into profiles/traffic_<workload>.json")
    return p.parse_args()


CALIB_BYTES = 256 << 20   # bytes read (and written) by the calibration copy
KERNELS = ("fwd_kernel", "fwd8_kernel", "delta_kernel", "dkdv_kernel", "dq_kernel", "decode_combine_kernel",
           "decode_kernel")


def source_hash() -> str:
    """sha256 over the HIP sources and the public header (what the counters describe)."""
    import glob
    import hashlib
    files = sorted(glob.glob(os.path.join(ROOT, "exact_io_aware_12_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "fa.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{workload}.json")


def load_traffic(workload: str, kernel: str):
    """Calibrated HBM bytes per launch of `kernel`, or None if absent or stale."""
    try:
        with open(traffic_path(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != source_hash() or kernel not in t.get("kernels", {}):
        return None
    k = t["kernels"][kernel]
    return k["fetch_bytes"] + k["write_bytes"]


class Bound:
    """Device buffers and raw C-ABI calls for one workload (nothing allocated per call)."""

    def __init__(self, w, with_bwd: bool):
        import torch
        import exact_io_aware_12_amd as fa
        import workloads as W
        self.fa, self.w, self.torch = fa, w, torch
        td = {"fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        a = W.generate(w, with_grad=with_bwd)
        dev = "cuda"
        self.t = {n: torch.from_numpy(a[n]).to(td).to(dev) for n in a if n != "cu_seqlens"}
        self.cu = torch.from_numpy(a["cu_seqlens"]).to(dev) if w.varlen else None
        del a
        T = w.T
        self.o = torch.empty_like(self.t["q"])
        self.lse = torch.empty((w.Hq, T), dtype=torch.float32, device=dev)
        if with_bwd:
            self.dq = torch.empty_like(self.t["q"])
            self.dk = torch.empty_like(self.t["k"])
            self.dv = torch.empty_like(self.t["v"])
            nws = fa.fa_bwd_workspace_size(w.B, w.Hq, w.Hkv, w.N, w.d)
            self.ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
        self.code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
        self.cu_ptr = self.cu.data_ptr() if self.cu is not None else None
        self.stream = torch.cuda.current_stream().cuda_stream

    def _mask(self):
        """The mask arguments: (causal,), (left, right) for a window workload, or
        (causal, softcap) for a soft-capped one, (causal, p, seed) with dropout."""
        w = self.w
        if w.dropout_p:
            return (int(w.causal), w.dropout_p, w.dropout_seed)
        if w.softcap:
            return (int(w.causal), w.softcap)
        if w.window is None:
            return (int(w.causal),)
        wl, wr = w.window
        return (wl, (0 if wr < 0 else min(wr, 0)) if w.causal else wr)

    def fwd(self):
        w, t = self.w, self.t
        if w.dropout_p:
            st = self.fa.fa_fwd_dropout(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                        self.o.data_ptr(), self.lse.data_ptr(), w.B, w.Hq, w.Hkv,
                                        w.N, w.d, w.scale, int(w.causal), w.dropout_p,
                                        w.dropout_seed, self.cu_ptr, self.code, self.stream)
            if st != self.fa.FA_OK:
                raise self.fa.FaError(st, "fa_fwd_dropout")
            return
        if w.softcap:
            st = self.fa.fa_fwd_softcap(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                        self.o.data_ptr(), self.lse.data_ptr(), w.B, w.Hq, w.Hkv,
                                        w.N, w.d, w.scale, int(w.causal), w.softcap, self.cu_ptr,
                                        self.code, self.stream)
            if st != self.fa.FA_OK:
                raise self.fa.FaError(st, "fa_fwd_softcap")
            return
        fn = self.fa.fa_fwd if w.window is None else self.fa.fa_fwd_window
        st = fn(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), self.o.data_ptr(),
                self.lse.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d, w.scale, *self._mask(),
                self.cu_ptr, self.code, self.stream)
        if st != self.fa.FA_OK:
            raise self.fa.FaError(st, "fa_fwd")

    def _bwd_args(self):
        w, t = self.w, self.t
        return (t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), self.o.data_ptr(),
                t["do"].data_ptr(), self.lse.data_ptr(), self.dq.data_ptr(), self.dk.data_ptr(),
                self.dv.data_ptr(), w.B, w.Hq, w.Hkv, w.N, w.d, w.scale, *self._mask(),
                self.cu_ptr, self.code, self.ws.data_ptr(), self.ws.numel(), self.stream)

    def bwd(self):
        fn = (self.fa.fa_bwd_dropout if self.w.dropout_p else
              self.fa.fa_bwd_softcap if self.w.softcap else
              self.fa.fa_bwd if self.w.window is None else self.fa.fa_bwd_window)
        st = fn(*self._bwd_args())
        if st != self.fa.FA_OK:
            raise self.fa.FaError(st, "fa_bwd")

    def bwd_stage(self, stage):
        if self.w.dropout_p:
            st = self.fa.fa_bwd_dropout_stage(stage, *self._bwd_args())
        elif self.w.softcap:
            st = self.fa.fa_bwd_softcap_stage(stage, *self._bwd_args())
        elif self.w.window is None:
            st = self.fa.fa_bwd_stage(stage, *self._bwd_args())
        else:
            st = self.fa.fa_bwd_window_stage(stage, *self._bwd_args())
        if st != self.fa.FA_OK:
            raise self.fa.FaError(st, "fa_bwd_stage")

    def step(self):
        self.fwd()
        self.bwd()


class Fp8Bound:
    """Device buffers and the raw fa_fwd_fp8 call for one workload: the
    workload's normal draws quantised per tensor to e4m3fn (descale = max|x| / 448)."""

    def __init__(self, w):
        import torch
        import exact_io_aware_12_amd as fa
        import workloads as W
        self.fa, self.w = fa, w
        f8 = W.quantize_e4m3(W.generate(w, with_grad=False))
        self.t = {n: torch.from_numpy(f8[n]).to("cuda") for n in ("q", "k", "v")}
        self.ds = tuple(float(f8["descale_" + n]) for n in ("q", "k", "v"))
        self.cu = torch.from_numpy(f8["cu_seqlens"]).to("cuda") if w.varlen else None
        self.cu_ptr = self.cu.data_ptr() if self.cu is not None else None
        self.o = torch.empty(self.t["q"].shape, dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((w.Hq, w.T), dtype=torch.float32, device="cuda")
        self.stream = torch.cuda.current_stream().cuda_stream

    def fwd(self):
        w, t = self.w, self.t
        st = self.fa.fa_fwd_fp8(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                self.o.data_ptr(), self.lse.data_ptr(), w.B, w.Hq, w.Hkv, w.N,
                                w.d, w.scale, int(w.causal), self.cu_ptr, *self.ds,
                                self.fa.FA_BF16, self.stream)
        if st != self.fa.FA_OK:
            raise self.fa.FaError(st, "fa_fwd_fp8")


def time_calls(torch, fn, iters, warmup, min_warm_s=0.0):
    """Average ms per call with HIP events on the current stream, after `warmup`
    calls and then more until at least `min_warm_s` seconds of back-to-back
    calls have run (a short kernel's first milliseconds run below the clock the
    part settles at under load)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def time_calls_dist(torch, fn, iters, warmup, scratch=None):
    """Per-call HIP event pairs on the current stream: (median, min) ms per call.

    With `scratch` (a device buffer larger than the 256 MB last-level cache), the
    buffer is overwritten before each call, outside its event pair: every call
    then starts with its inputs evicted from L2 and the cache (cold inputs)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(iters)]
    for a, b in ev:
        if scratch is not None:
            scratch.zero_()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    n = len(ts)
    med = ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2])
    return med, ts[0]


def smi_sample(torch, fn, ms_per_call, seconds=8.0):
    """Clock, power and temperature while the GPU runs `fn` back to back: calls
    for about `seconds` are enqueued, amd-smi is read once while they run, and
    its JSON (or its error text) is returned."""
    import subprocess
    n = max(1, int(seconds * 1e3 / max(ms_per_call, 1e-3)))
    for _ in range(n):
        fn()
    try:
        r = subprocess.run(["amd-smi", "metric", "-g", "0", "--power", "--clock",
                            "--temperature", "--json"], capture_output=True, text=True,
                           timeout=30)
        out = r.stdout.strip() or r.stderr.strip()
        try:
            out = json.loads(out)
        except ValueError:
            pass
    except Exception as e:  # the tool missing or hanging must not fail the sweep
        out = f"amd-smi unavailable: {e}"
    torch.cuda.synchronize()
    return out


def cpu_baseline(w, min_seconds=10.0, max_units=4):
    """The float64 oracle, untouched, on (sequence, head) units of the workload.

    Units are run one after another until at least `min_seconds` of wall time
    (at most `max_units`); throughput = their algorithmic FLOP / wall time.
    """
    import numpy as np
    import oracle.attention as O
    try:
        from threadpoolctl import threadpool_info
        cores = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    rng = np.random.default_rng(w.seed)
    L = w.seq_lens[0]
    units = w.B * w.Hq if not w.varlen else None
    flop_unit = (w.fwd_flop() + (w.bwd_flop() if w.backward else 0)) / units
    done, dt = 0, 0.0
    while done < max_units and (done == 0 or dt < min_seconds):
        q, k, v, do = (rng.standard_normal((L, w.d), dtype=np.float32) for _ in range(4))
        t0 = time.perf_counter()
        if w.dropout_p:   # one (sequence, head) unit through the dropout oracle
            import oracle.dropout as OD
            u = [x[:, None, :] for x in (q, k, v, do)]
            OD.attention_fwd_dropout(*u[:3], w.scale, w.causal, None, w.dropout_p,
                                     w.dropout_seed)
            if w.backward:
                OD.attention_bwd_dropout(*u, w.scale, w.causal, None, w.dropout_p,
                                         w.dropout_seed)
        else:
            O.head_fwd(q, k, v, w.scale, w.causal, window=w.window, softcap=w.softcap or None)
            if w.backward:
                O.head_bwd(q, k, v, do, w.scale, w.causal, window=w.window,
                           softcap=w.softcap or None)
        dt += time.perf_counter() - t0
        done += 1
    return {"value": round(done * flop_unit / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done} of {units} (sequence, head) units, N={L}, forward + backward, "
                      f"{dt:.1f} s wall; algorithmic FLOP of those units / wall time"}


class KvlenBound:
    """Device buffers and the raw fa_fwd_kvlen call of one chunked-prefill workload."""

    def __init__(self, w):
        import torch
        import exact_io_aware_12_amd as fa
        import workloads as W
        self.fa, self.w = fa, w
        td = {"fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        a = W.generate_kvlen(w)
        self.t = {n: torch.from_numpy(a[n]).to(td).cuda() for n in ("q", "k", "v")}
        del a
        self.o = torch.empty_like(self.t["q"])
        self.lse = torch.empty((w.Hq, w.B * w.Nq), dtype=torch.float32, device="cuda")
        self.code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
        self.stream = torch.cuda.current_stream().cuda_stream

    def fwd(self):
        w, t = self.w, self.t
        st = self.fa.fa_fwd_kvlen(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                  self.o.data_ptr(), self.lse.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq,
                                  w.Nk, w.d, w.scale, int(w.causal), None, None, self.code,
                                  self.stream)
        if st != self.fa.FA_OK:
            raise self.fa.FaError(st, "fa_fwd_kvlen")


class DecodeBound:
    """Device buffers and raw C-ABI calls of one decode workload."""

    def __init__(self, w):
        import torch
        import exact_io_aware_12_amd as fa
        import workloads as W
        self.fa, self.w, self.torch = fa, w, torch
        td = {"fp16": torch.float16, "bf16": torch.bfloat16}[w.dtype]
        self.kv8 = w.kv_cache == "e4m3"
        a = W.decode_fp8_inputs(w) if self.kv8 else W.generate_decode(w)
        self.q = torch.from_numpy(a["q"]).to(td).cuda()
        ct = torch.uint8 if self.kv8 else td
        self.k = torch.from_numpy(a["k"]).to(ct).cuda()
        self.v = torch.from_numpy(a["v"]).to(ct).cuda()
        self.descales = (a["descale_k"], a["descale_v"]) if self.kv8 else None
        self.lens = torch.from_numpy(a["cache_seqlens"]).cuda()
        del a
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((w.Hq, w.B * w.Nq), dtype=torch.float32, device="cuda")
        ns = fa.fa_kvcache_fp8_num_splits if self.kv8 else fa.fa_kvcache_num_splits
        self.splits = ns(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
        nws = fa.fa_fwd_kvcache_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, self.splits)
        self.ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        self.code = fa.FA_BF16 if w.dtype == "bf16" else fa.FA_FP16
        self.stream = torch.cuda.current_stream().cuda_stream

    def _args(self):
        w = self.w
        desc = self.descales if self.kv8 else ()
        return (self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), self.lens.data_ptr(),
                self.o.data_ptr(), self.lse.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, w.scale,
                int(w.causal), *desc, self.splits, self.code, self.ws.data_ptr(), self.ws.numel(),
                self.stream)

    def call(self):
        fn = "fa_fwd_kvcache_fp8" if self.kv8 else "fa_fwd_kvcache"
        st = getattr(self.fa, fn)(*self._args())
        if st != self.fa.FA_OK:
            raise self.fa.FaError(st, fn)

    def stage(self, i):
        fn = "fa_fwd_kvcache_fp8_stage" if self.kv8 else "fa_fwd_kvcache_stage"
        st = getattr(self.fa, fn)(i, *self._args())
        if st != self.fa.FA_OK:
            raise self.fa.FaError(st, fn)


def cpu_baseline_decode(w, min_seconds=10.0, max_rounds=50):
    """The float64 decode oracle, untouched, over the whole workload, repeated to >= 10 s."""
    import numpy as np
    import oracle.decode as OD
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        cores = 1
    if w.kv_cache == "e4m3":   # the oracle on the decoded cache (decoding is inside the timing)
        import oracle.fp8 as O8
        a = W.decode_fp8_inputs(w)

        def run():
            OD.kvcache_fwd(a["q"], O8.dequantize(a["k"], a["descale_k"]),
                           O8.dequantize(a["v"], a["descale_v"]), a["cache_seqlens"], w.scale,
                           w.causal)
    else:
        a = W.generate_decode(w)

        def run():
            OD.kvcache_fwd(a["q"], a["k"], a["v"], a["cache_seqlens"], w.scale, w.causal)
    rounds, dt = 0, 0.0
    while rounds < max_rounds and (rounds == 0 or dt < min_seconds):
        t0 = time.perf_counter()
        run()
        dt += time.perf_counter() - t0
        rounds += 1
    return {"value": round(rounds * w.io_bytes() / dt / 1e9, 4), "unit": "GB/s",
            "cores": int(cores), "kind": "oracle",
            "sample": f"the whole workload {rounds} times, {dt:.1f} s wall; compulsory bytes of "
                      f"one call (valid K/V, q, o, lse) x calls / wall time"}


def run_decode_bench(args):
    import torch
    import workloads as W
    w = W.DECODE_WORKLOADS[args.workload]
    b = DecodeBound(w)
    nst = b.fa.fa_fwd_kvcache_num_stages()
    names = ["decode_kernel", "decode_combine_kernel"][:nst]
    for _ in range(args.warmup):
        b.call()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        for st in range(nst):
            b.stage(st)
            ev[k][st + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0][0].elapsed_time(ev[-1][-1]) / args.steps
    kern = {n: sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)) / args.steps
            for i, n in enumerate(names)}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        b.call()
    e1.record()
    torch.cuda.synchronize()
    ms_entry = e0.elapsed_time(e1) / args.steps
    value = w.io_bytes() / (ms_entry * 1e-3) / 1e9
    # dominant kernel: the range pass; its algorithmic bytes are the valid K/V and q it must read
    dom = max(kern, key=kern.get)
    alg = {"decode_kernel": w.kv_bytes() + 2 * w.B * w.Nq * w.Hq * w.d,
           "decode_combine_kernel": 2 * w.B * w.Nq * w.Hq * w.d + 4 * w.B * w.Nq * w.Hq}[dom]
    ach = alg / (kern[dom] * 1e-3) / 1e9
    out = {
        "metric": "decode attention over a KV cache: HBM GB/s (compulsory bytes / time)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_entry, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: " + ("fa_fwd_kvcache_fp8" if b.kv8 else "fa_fwd_kvcache"),
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "seed": w.seed, "splits": b.splits,
                   "kv_cache": w.dtype if not b.kv8 else "e4m3fn",
                   "cache_lens": w.cache_lens()},
        "pct_of_hbm_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "attention_tflops": round(w.flop() / (ms_entry * 1e-3) / 1e12, 3),
        "kernel_ms": {k: round(v, 5) for k, v in kern.items()},
        "ms_per_step_staged": round(ms, 5),
        "wall_s_timed": round(wall, 3),
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": load_traffic(w.name, dom), "avg_launch_ms": round(kern[dom], 5)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w)
    print(json.dumps(out), flush=True)


def run_split_sweep(args):
    """Decode: per shape, the median µs per call (8 rounds of 50 calls, rounds
    interleaved over the counts) at every key-range count from 1 to 64 that the
    shape allows, beside the automatic count the library picks."""
    import statistics
    import torch
    import workloads as W
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for spec in args.split_sweep.split(","):
        if spec in W.DECODE_WORKLOADS:
            w = W.DECODE_WORKLOADS[spec]
        else:
            B, Hq, Hkv, Nq, Nk, cache, d = spec.split("-")
            w = W.decode_custom(int(B), int(Hq), int(Hkv), int(Nq), int(Nk), int(d), dtype="bf16",
                                causal=True, seed=3, kv_cache=cache)
        b = DecodeBound(w)
        fa, auto = b.fa, b.splits
        most = max(1, (w.Nk + 255) // 256)
        counts = sorted({n for n in (1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, auto, 2 * auto)
                         if n <= min(most, 256)} | {auto})
        ws = {}
        for n in counts:
            nb = fa.fa_fwd_kvcache_workspace_size(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, n)
            ws[n] = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")

        def run(n):
            b.splits, b.ws = n, ws[n]
            b.call()

        for n in counts:
            for _ in range(20):
                run(n)
        torch.cuda.synchronize()
        res = {n: [] for n in counts}
        for _ in range(8):
            for n in counts:
                ev[0].record()
                for _ in range(50):
                    run(n)
                ev[1].record()
                torch.cuda.synchronize()
                res[n].append(ev[0].elapsed_time(ev[1]) / 50 * 1000)
        med = {n: round(statistics.median(v), 2) for n, v in res.items()}
        best = min(med, key=med.get)
        print(json.dumps({"shape": spec, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk,
                          "d": w.d, "cache": "e4m3fn" if b.kv8 else w.dtype, "auto_splits": auto,
                          "us_auto": med[auto], "best_splits": best, "us_best": med[best],
                          "us_by_splits": {str(n): med[n] for n in counts}}), flush=True)


def run_pmc_step(args):
    """Calibration copy of known size, then one fa_fwd + fa_bwd step (no timing)."""
    import torch
    import workloads as W
    w = W.WORKLOADS.get(args.workload)
    n = CALIB_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)            # reads CALIB_BYTES, writes CALIB_BYTES
    torch.cuda.synchronize()
    del src, dst
    if args.workload in W.DECODE_WORKLOADS:
        DecodeBound(W.DECODE_WORKLOADS[args.workload]).call()
    else:
        b = Bound(w, with_bwd=w.backward)
        b.fwd()
        if w.backward:
            b.bwd()
    torch.cuda.synchronize()
    print("pmc step done", flush=True)


def _counter_means(d, counter):
    """Mean per-dispatch value of `counter` per kernel (short name) in a rocprofv3 csv run."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                name = r["Kernel_Name"]
                short = next((k for k in KERNELS if k in name), None)
                if short is None and "neg" in name.lower():
                    short = "calibration_copy"
                if short is not None:
                    vals.setdefault(short, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def run_pmc_summary(args):
    fetch = _counter_means(args.pmc_summary[0], "FETCH_SIZE")
    write = _counter_means(args.pmc_summary[1], "WRITE_SIZE")
    if "calibration_copy" not in fetch or "calibration_copy" not in write:
        raise SystemExit("no calibration copy dispatch found in the counter runs")
    f_scale = fetch["calibration_copy"] * 1024 / CALIB_BYTES   # counter bytes per real byte
    w_scale = write["calibration_copy"] * 1024 / CALIB_BYTES
    out = {"workload": args.workload, "source_sha256": source_hash(),
           "calibration": {"bytes_each_way": CALIB_BYTES,
                           "fetch_size_kib": fetch["calibration_copy"],
                           "write_size_kib": write["calibration_copy"],
                           "fetch_scale": f_scale, "write_scale": w_scale},
           "kernels": {}}
    for k in KERNELS:
        if k in fetch and k in write:
            out["kernels"][k] = {"fetch_size_kib": fetch[k], "write_size_kib": write[k],
                                 "fetch_bytes": fetch[k] * 1024 / f_scale,
                                 "write_bytes": write[k] * 1024 / w_scale}
    os.makedirs(os.path.dirname(traffic_path(args.workload)), exist_ok=True)
    with open(traffic_path(args.workload), "w") as f:
        json.dump(out, f, indent=1)
    print(f"| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |")
    print(f"|---|---|---|---|---|")
    print(f"| calibration copy ({CALIB_BYTES >> 20} MiB each way) | {fetch['calibration_copy']:.0f} | "
          f"{write['calibration_copy']:.0f} | {CALIB_BYTES / 1e6:.1f} | {CALIB_BYTES / 1e6:.1f} |")
    for k, v in out["kernels"].items():
        print(f"| {k} | {v['fetch_size_kib']:.0f} | {v['write_size_kib']:.0f} | "
              f"{v['fetch_bytes'] / 1e6:.1f} | {v['write_bytes'] / 1e6:.1f} |")


def run_step_bench(args):
    import torch
    import workloads as W
    w = W.WORKLOADS[args.workload]
    if not w.backward:
        raise SystemExit(f"{w.name} has no backward; the step bench needs the training workload")
    b = Bound(w, with_bwd=True)
    flop = w.fwd_flop() + w.bwd_flop()
    nst = b.fa.fa_bwd_num_stages()
    names = ["fwd_kernel", "delta_kernel", "dkdv_kernel", "dq_kernel"][: 1 + nst]

    def step_staged():   # fa_fwd, then fa_bwd's stages one call each (the same launches)
        b.fwd()
        for st in range(nst):
            b.bwd_stage(st)

    for _ in range(args.warmup):
        b.step()
    # K steps with fa_bwd's stages called one by one and an event after every
    # launch: each kernel's duration inside the steps, on the launch stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        b.fwd()
        ev[k][1].record()
        for st in range(nst):
            b.bwd_stage(st)
            ev[k][2 + st].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev[0][0].elapsed_time(ev[-1][-1]) / args.steps
    kern = {n: sum(ev[k][i].elapsed_time(ev[k][i + 1]) for k in range(args.steps)) / args.steps
            for i, n in enumerate(names)}
    # the steps through the entry points: fa_fwd, fa_bwd (what `value` reports)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        b.step()
    e1.record()
    torch.cuda.synchronize()
    ms_entry = e0.elapsed_time(e1) / args.steps
    bwd_ms = sum(kern[n] for n in names[1:])
    alg = {  # algorithmic work per launch
        "fwd_kernel": ("mfma", w.fwd_flop()),
        "dkdv_kernel": ("mfma", 0.8 * w.bwd_flop()),    # S, dP, dV, dK: 4 of the 5 counted GEMMs
        "dq_kernel": ("mfma", 0.2 * w.bwd_flop()),      # dQ: the 5th counted GEMM
        "delta_kernel": ("hbm", 2 * w.T * w.Hq * w.d * 2 + 4 * w.T * w.Hq),
    }
    dom = max(kern, key=kern.get)
    bound, work = alg[dom]
    if bound == "mfma":
        ach = work / (kern[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(w.name, dom), "avg_launch_ms": round(kern[dom], 4)}
    else:
        ach = work / (kern[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": load_traffic(w.name, dom), "avg_launch_ms": round(kern[dom], 4)}

    value = flop / (ms_entry * 1e-3) / 1e12
    out = {
        "metric": "attention TFLOP/s (fwd+bwd training step) and % of MFMA bf16 dense peak",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_entry, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": (f"{w.name}: fa_fwd_dropout + fa_bwd_dropout" if w.dropout_p else
                                f"{w.name}: fa_fwd_softcap + fa_bwd_softcap" if w.softcap else
                                f"{w.name}: fa_fwd + fa_bwd" if w.window is None else
                                f"{w.name}: fa_fwd_window + fa_bwd_window"),
                   "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "N": w.N, "d": w.d, "causal": w.causal, "seed": w.seed,
                   **({"window": list(w.window)} if w.window is not None else {}),
                   **({"softcap": w.softcap} if w.softcap else {}),
                   **({"dropout_p": w.dropout_p, "dropout_seed": w.dropout_seed}
                      if w.dropout_p else {})},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": round(w.fwd_flop() / (kern["fwd_kernel"] * 1e-3) / 1e12, 2),
        "bwd_tflops": round(w.bwd_flop() / (bwd_ms * 1e-3) / 1e12, 2),
        "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
        "ms_per_step_staged": round(ms, 4),
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


def run_sweep(args):
    import torch
    import workloads as W
    names = ["tiny", "causal_d64"] + [f"sweep_N{N}_{c}" for N in (512, 1024, 2048, 4096, 8192)
                                      for c in ("full", "causal")] + ["gqa_varlen", "train_16k",
                                                                      "fwd_d256_N4096",
                                                                      "window_16k",
                                                                      "softcap_16k",
                                                                      "dropout_16k",
                                                                      "prefill_chunk"]
    if args.names:
        names = args.names.split(",")
    # inputs and outputs smaller than twice the 256 MB last-level cache also get a
    # cold-input timing (a 1 GiB scratch buffer overwritten between calls)
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    smi = {}
    for n in names:
        if n in W.KVLEN_WORKLOADS:   # queries and keys of different lengths
            w = W.KVLEN_WORKLOADS[n]
            b = KvlenBound(w)
            ms = time_calls(torch, b.fwd, 100, 10, min_warm_s=0.2)
            med, mn = time_calls_dist(torch, b.fwd, 100, 0)
            tf = w.fwd_flop() / (ms * 1e-3) / 1e12
            print(json.dumps({"workload": n, "Nq": w.Nq, "Nk": w.Nk, "d": w.d, "dtype": w.dtype,
                              "causal": w.causal, "fwd_ms": round(ms, 4),
                              "fwd_tflops": round(tf, 2),
                              "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                              "fwd_ms_median": round(med, 4), "fwd_ms_min": round(mn, 4)}),
                  flush=True)
            del b
            torch.cuda.empty_cache()
            continue
        w = W.WORKLOADS[n]
        b = Bound(w, with_bwd=False)
        ms = time_calls(torch, b.fwd, 100, 10, min_warm_s=0.2)
        med, mn = time_calls_dist(torch, b.fwd, 100, 0)
        tf = w.fwd_flop() / (ms * 1e-3) / 1e12
        io = sum(x.numel() * x.element_size() for x in (b.t["q"], b.t["k"], b.t["v"], b.o, b.lse))
        line = {"workload": n, "N": w.N, "d": w.d, "dtype": w.dtype, "causal": w.causal,
                "fwd_ms": round(ms, 4), "fwd_tflops": round(tf, 2),
                "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                "fwd_ms_median": round(med, 4), "fwd_ms_min": round(mn, 4),
                "io_mb": round(io / 1e6, 2)}
        if io < 512e6:
            cmed, cmn = time_calls_dist(torch, b.fwd, 100, 0, scratch=scratch)
            line.update({"cold_fwd_ms_median": round(cmed, 4), "cold_fwd_ms_min": round(cmn, 4),
                         "cold_tflops": round(w.fwd_flop() / (cmed * 1e-3) / 1e12, 2)})
        if args.smi and ms >= 1.0:
            smi[n] = smi_sample(torch, b.fwd, ms)
        print(json.dumps(line), flush=True)
        del b
        torch.cuda.empty_cache()
    if args.smi:
        with open(args.smi, "w") as f:
            json.dump(smi, f, indent=1)


def run_fp8_sweep(args):
    """fa_fwd (bf16) and fa_fwd_fp8 (e4m3 in, bf16 out) on the d = 128 forward
    workloads (--names picks others, d = 64 and 256 included), one line each:
    TFLOP/s by the forward convention, against the dense peak of each
    instruction's input type."""
    import torch
    import workloads as W
    names = [f"sweep_N{N}_{c}" for N in (1024, 4096, 8192) for c in ("full", "causal")] + \
        ["gqa_varlen", "train_16k"]
    if args.names:
        names = args.names.split(",")
    for n in names:
        w = W.WORKLOADS[n]
        b16 = Bound(w, with_bwd=False)
        ms16 = time_calls(torch, b16.fwd, 100, 10, min_warm_s=0.2)
        del b16
        torch.cuda.empty_cache()
        b8 = Fp8Bound(w)
        ms8 = time_calls(torch, b8.fwd, 100, 10, min_warm_s=0.2)
        del b8
        torch.cuda.empty_cache()
        tf16 = w.fwd_flop() / (ms16 * 1e-3) / 1e12
        tf8 = w.fwd_flop() / (ms8 * 1e-3) / 1e12
        print(json.dumps({"workload": n, "N": w.N, "d": w.d, "causal": w.causal,
                          "bf16_fwd_ms": round(ms16, 4), "bf16_tflops": round(tf16, 2),
                          "bf16_pct_of_peak": round(100 * tf16 / PEAK_BF16_TFLOPS, 2),
                          "fp8_fwd_ms": round(ms8, 4), "fp8_tflops": round(tf8, 2),
                          "fp8_pct_of_peak": round(100 * tf8 / PEAK_FP8_TFLOPS, 2),
                          "fp8_speedup": round(ms16 / ms8, 3)}), flush=True)


def main():
    args = parse()
    if args.pmc_summary:   # host-only: reads counter files
        run_pmc_summary(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the (sequence, head) units are independent; see the sharding notes). "
              "Run with --gpus 1.", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.fp8_sweep:
        run_fp8_sweep(args)
        return
    if args.split_sweep:
        run_split_sweep(args)
        return
    if args.sweep:
        run_sweep(args)
    elif args.pmc_step:
        run_pmc_step(args)
    elif args.workload in __import__("workloads").DECODE_WORKLOADS:
        run_decode_bench(args)
    else:
        run_step_bench(args)


if __name__ == "__main__":
    main()
