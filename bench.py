"""Benchmark: causal attention fwd + bwd through libfa.so on one MI355X.

One step = fa_fwd then fa_bwd (forward kernel, row-dot kernel, dK/dV kernel,
dQ kernel) over the long-context GQA workload (B=1, Hq=32, Hkv=8, S=16384,
D=128, bf16, causal) with every input already resident in HBM.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-memory] [--no-decode] [--no-sweep]
                    [--no-configs] [--sweep-ms MS] [--calibrate-copy-mib MIB]

Prints one JSON line.  ``value`` is causal fwd+bwd TFLOP/s: 4*D flops per
visited (query, key) pair for the forward and 10*D for the backward, pairs =
B*Hq*S*(S+1)/2, divided by the measured time per step.  Per-kernel durations
come from HIP events the library records around each of its kernel launches
(fa_profile_events) during the same timed steps.

Per-kernel and per-step times are reported as mean, median and minimum over
the timed steps.  ``gfx_clock`` holds the GPU's graphics clock (amdsmi GPU
metrics, mean over the XCDs) sampled while the same step, and then the forward
alone, run back to back for about a second each, right after the timed steps;
``pct_of_clock_peak`` prices the throughput against 256 CUs x that clock x 4096
flop/clk/CU instead of the 2.4 GHz figure.

Also reported, outside the timed steps: ``configs`` (forward and backward of
each of the five workloads, timed call by call), ``forward_sweep`` (the forward
alone at S = 4096, 8192, 16384 with 32/8 heads, D = 128), ``decode`` (one
split-KV decode step of 16 sequences x 8192 cached keys, as GB/s against HBM,
beside the plain forward on the same inputs), ``memory`` and ``cpu_baseline``.
Counter figures (HBM bytes, MFMA busy cycles, clock under load) come from the
committed rocprofv3 profiles of this workload when they were taken on the
current kernel sources.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import statistics
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import LONG_CONTEXT, WORKLOADS, workload_inputs  # noqa: E402

METRIC = "attention fwd+bwd TFLOP/s (causal) and % of bf16 MFMA peak at 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6      # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_FP32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
CUS = 256                      # MI355X compute units
BF16_FLOP_PER_CLK_CU = 4096    # dense bf16 / fp16 matrix flops per clock per CU
KERNELS = ("fwd", "rowdot", "dkdv", "dq")


def stats(xs):
    """mean / median / min of a list of milliseconds."""
    return {"mean_ms": round(sum(xs) / len(xs), 4), "median_ms": round(statistics.median(xs), 4),
            "min_ms": round(min(xs), 4)}


class ClockSampler:
    """Samples the GPU's graphics clock (MHz, the mean over its XCDs) and socket
    power from a side thread through amdsmi's GPU metrics.  Telemetry only: it
    reads what the driver reports and changes nothing.  The driver refreshes
    these metrics only every few hundred milliseconds, so the clock is sampled
    over a window of about a second of continuous work (``clock_window``), not
    over the short timed steps.  ``summary()`` says why when there are no
    samples."""

    def __init__(self, period_s=0.01):
        self.period = period_s
        self.clk, self.power = [], []
        self.max_clk = None
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._h = None

    def _handle(self):
        import amdsmi
        hs = amdsmi.amdsmi_get_processor_handles()
        if len(hs) == 1:
            return hs[0]
        import torch
        props = torch.cuda.get_device_properties(0)
        bus = getattr(props, "pci_bus_id", None)
        for h in hs:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)      # "dddd:bb:dd.f"
            if bus is not None and int(bdf.split(":")[1], 16) == bus:
                return h
        raise RuntimeError(f"{len(hs)} GPUs visible to amdsmi and none matched cuda:0")

    def _read(self):
        import amdsmi
        m = amdsmi.amdsmi_get_gpu_metrics_info(self._h)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float))]
        clk = sum(clks) / len(clks) if clks else m.get("current_gfxclk")
        w = m.get("current_socket_power")
        return (float(clk) if isinstance(clk, (int, float)) else None,
                float(w) if isinstance(w, (int, float)) else None)

    def __enter__(self):
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._h = self._handle()
            self.max_clk = amdsmi.amdsmi_get_clock_info(self._h, amdsmi.AmdSmiClkType.GFX).get("max_clk")
            self._read()
        except Exception as e:  # telemetry is optional
            self.error = f"{type(e).__name__}: {e}"
            self._h = None
            return self

        def loop():
            while not self._stop.is_set():
                try:
                    c, w = self._read()
                    if c is not None:
                        self.clk.append(c)
                    if w is not None:
                        self.power.append(w)
                except Exception as e:
                    self.error = f"{type(e).__name__}: {e}"
                    return
                time.sleep(self.period)

        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
        try:
            import amdsmi
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass
        return False

    def summary(self):
        # the first third of the window covers the clock's ramp from idle
        clk, pw = self.clk[len(self.clk) // 3:], self.power[len(self.power) // 3:]
        if not clk:
            return {"samples": 0, "note": self.error or "no samples"}
        out = {"samples": len(clk), "median_mhz": round(statistics.median(clk), 1), "min_mhz": round(min(clk), 1),
               "max_mhz": round(max(clk), 1), "max_clk_mhz": self.max_clk}
        if pw:
            out["socket_power_w_median"] = round(statistics.median(pw), 1)
        return out


def clock_window(fn, seconds):
    """The graphics clock while fn() runs back to back for `seconds`."""
    import torch
    torch.cuda.synchronize()
    with ClockSampler() as cs:
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    out = cs.summary()
    out["seconds"] = seconds
    out["calls"] = n
    return out


class Hip:
    """The few HIP runtime calls bench needs (events), via ctypes."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        vp = ctypes.c_void_p
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(vp)]
        self.h.hipEventRecord.argtypes = [vp, vp]
        self.h.hipEventSynchronize.argtypes = [vp]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        self.h.hipEventDestroy.argtypes = [vp]

    def _ok(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def event(self):
        e = ctypes.c_void_p()
        self._ok(self.h.hipEventCreate(ctypes.byref(e)), "hipEventCreate")
        return e

    def record(self, e, stream):
        self._ok(self.h.hipEventRecord(e, stream), "hipEventRecord")

    def ms(self, a, b):
        out = ctypes.c_float()
        self._ok(self.h.hipEventElapsedTime(ctypes.byref(out), a, b), "hipEventElapsedTime")
        return float(out.value)

    def destroy(self, e):
        self.h.hipEventDestroy(e)


def algorithmic_work(w):
    """Per-kernel algorithmic work of one step (flops, or bytes for the row-dot kernel)."""
    pairs = w.causal_pairs()
    D = w.D
    elem = {"bf16": 2, "f16": 2, "f32": 4}[w.dtype]
    rows = w.B * w.Hq * w.S
    return {
        "fwd": 4.0 * D * pairs,            # Q K^T and P V
        "dkdv": 8.0 * D * pairs,           # S and dP (recomputed), dV, dK
        "dq": 2.0 * D * pairs,             # dQ (its S / dP recompute is overhead of the split)
        "rowdot": 2.0 * rows * D * elem + 4.0 * rows,   # read O and dO, write D (bytes)
    }


def committed_counters(w):
    """Per-kernel MFMA and clock figures from the committed counter profile of this
    workload, if it was taken on exactly the current kernel sources (else None)."""
    from causal_attention_fa_amd.build import source_fingerprint
    path = os.path.join(ROOT, "profiles", f"mfma_util_{w.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    if prof.get("source_sha256") != source_fingerprint():
        return None
    return prof


def committed_traffic(w):
    """Per-launch HBM bytes of each kernel from the committed counter profile of this workload,
    if it was taken on exactly the current kernel sources (else None: the kernels changed)."""
    from causal_attention_fa_amd.build import source_fingerprint
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{w.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    if prof.get("source_sha256") != source_fingerprint():
        return None
    return prof


def run_gpu(w, steps, warmup):
    import numpy as np  # noqa: F401
    import torch

    import causal_attention_fa_amd as fa

    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    code = {"bf16": fa.FA_BF16, "f16": fa.FA_F16, "f32": fa.FA_F32}[w.dtype]
    inp = workload_inputs(w)
    t = {n: torch.from_numpy(x).to(dev).to(tdt).contiguous() for n, x in inp.items()}
    del inp
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws_bytes = fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.D)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream
    hip = Hip()
    args = (w.B, w.Hq, w.Hkv, w.S, w.D, w.scale, int(w.causal), code)

    def step():
        st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), *args, sh)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_fwd")
        st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *args, ws.data_ptr(), ws.numel(), sh)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_bwd")

    torch.cuda.synchronize()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # per step: fwd before/after (2) and bwd rowdot/dkdv/dq boundaries (4)
    evs = [[hip.event() for _ in range(6)] for _ in range(steps)]
    arrays = [((ctypes.c_void_p * 2)(evs[s][0].value, evs[s][1].value),
               (ctypes.c_void_p * 4)(*[e.value for e in evs[s][2:]])) for s in range(steps)]
    start, end = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(start, sh)
    for s in range(steps):
        fa.fa_profile_events(ctypes.addressof(arrays[s][0]), 2)
        st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), *args, sh)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_fwd")
        fa.fa_profile_events(ctypes.addressof(arrays[s][1]), 4)
        st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                       dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *args, ws.data_ptr(), ws.numel(), sh)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_bwd")
    fa.fa_profile_events(None, 0)
    hip.record(end, sh)
    torch.cuda.synchronize()
    total_ms = hip.ms(start, end)
    per = {n: [] for n in KERNELS}
    per["step"] = []
    for s in range(steps):
        e = evs[s]
        per["fwd"].append(hip.ms(e[0], e[1]))
        per["rowdot"].append(hip.ms(e[2], e[3]))
        per["dkdv"].append(hip.ms(e[3], e[4]))
        per["dq"].append(hip.ms(e[4], e[5]))
        per["step"].append(hip.ms(e[0], e[5]))
    for row in evs:
        for e in row:
            hip.destroy(e)
    hip.destroy(start)
    hip.destroy(end)
    def fwd():
        st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), *args, sh)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_fwd")

    # the graphics clock under this work, outside the timed steps
    clock = {"fwd_bwd": clock_window(step, 1.5), "forward": clock_window(fwd, 1.0)}
    del t, q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return total_ms / steps, per, clock


def _time_calls(fn, steps, warmup, stream, hip, nev=0):
    """Mean ms of fn(events) over `steps` calls after `warmup`; with nev > 0 each
    call gets nev fresh events (fa_profile_events) and their gaps are averaged."""
    import torch

    import causal_attention_fa_amd as fa
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [[hip.event() for _ in range(nev)] for _ in range(steps)] if nev else []
    arrays = [(ctypes.c_void_p * nev)(*[e.value for e in row]) for row in evs]
    start, end = hip.event(), hip.event()
    hip.record(start, stream)
    for s in range(steps):
        if nev:
            fa.fa_profile_events(ctypes.addressof(arrays[s]), nev)
        fn()
    fa.fa_profile_events(None, 0)
    hip.record(end, stream)
    torch.cuda.synchronize()
    total = hip.ms(start, end) / steps
    gaps = [sum(hip.ms(row[i], row[i + 1]) for row in evs) / steps for i in range(nev - 1)] if nev else []
    for row in evs:
        for e in row:
            hip.destroy(e)
    hip.destroy(start)
    hip.destroy(end)
    return total, gaps


def _time_each(fn, n, warmup, stream, hip):
    """Milliseconds of each of n calls of fn, from events recorded around every call."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(hip.event(), hip.event()) for _ in range(n)]
    for a, b in evs:
        hip.record(a, stream)
        fn()
        hip.record(b, stream)
    torch.cuda.synchronize()
    out = [hip.ms(a, b) for a, b in evs]
    for a, b in evs:
        hip.destroy(a)
        hip.destroy(b)
    return out


def config_table(skip):
    """Forward and backward of every workload, each timed call by call on resident
    inputs: median / min / mean ms, TFLOP/s at the median and % of the dtype's
    matrix peak (bf16 / fp16 2516.6, fp32 157.3 TFLOP/s)."""
    import torch

    import causal_attention_fa_amd as fa
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream
    hip = Hip()
    rows = []
    for w in WORKLOADS.values():
        if w.name in skip:
            continue
        tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
        code = {"bf16": fa.FA_BF16, "f16": fa.FA_F16, "f32": fa.FA_F32}[w.dtype]
        inp = workload_inputs(w)
        t = {n: torch.from_numpy(x).to(dev).to(tdt).contiguous() for n, x in inp.items()}
        del inp
        q, k, v = t["q"], t["k"], t["v"]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.S), dtype=torch.float32, device=dev)
        args = (w.B, w.Hq, w.Hkv, w.S, w.D, w.scale, int(w.causal), code)
        peak = PEAK_FP32_MATRIX_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS

        def fwd():
            st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), *args, sh)
            if st != fa.FA_OK:
                raise fa.FAError(st, "fa_fwd")

        # 200 calls after at least 50 warm-ups: long enough for the clock to settle
        # (every workload here runs 0.02-0.2 ms per call)
        n, warm = 200, 50
        row = {"workload": w.name, "dtype": w.dtype, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D,
               "peak_tflops": peak}
        ms = _time_each(fwd, n, warm, sh, hip)
        row["fwd"] = dict(stats(ms), calls=n)
        tf = w.fwd_flops() / (statistics.median(ms) * 1e-3) / 1e12
        row["fwd"].update(tflops=round(tf, 2), pct_of_peak=round(100 * tf / peak, 2))
        if w.backward:
            fwd()
            do = t["do"]
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            nb = fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.D)
            ws = torch.empty(max(nb, 256), dtype=torch.uint8, device=dev)

            def bwd():
                st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), *args, ws.data_ptr(),
                               ws.numel(), sh)
                if st != fa.FA_OK:
                    raise fa.FAError(st, "fa_bwd")

            ms = _time_each(bwd, n, warm, sh, hip)
            row["bwd"] = dict(stats(ms), calls=n)
            tf = w.bwd_flops() / (statistics.median(ms) * 1e-3) / 1e12
            row["bwd"].update(tflops=round(tf, 2), pct_of_peak=round(100 * tf / peak, 2))
            del do, dq, dk, dv, ws
        rows.append(row)
        del t, q, k, v, o, lse
        torch.cuda.empty_cache()
    return rows


def decode_bench(steps, warmup):
    """One decode step (split-KV forward) of the decode workload, and the plain
    forward on the same inputs for comparison.  HBM-bound: reported as GB/s of
    the bytes the step must move (K and V once per KV head, Q, O, L)."""
    import torch

    import causal_attention_fa_amd as fa
    from workloads import DECODE, decode_inputs
    w = DECODE
    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    code = {"bf16": fa.FA_BF16, "f16": fa.FA_F16, "f32": fa.FA_F32}[w.dtype]
    t = {n: torch.from_numpy(x).to(dev).to(tdt).contiguous() for n, x in decode_inputs(w).items()}
    q, k, v = t["q"], t["k"], t["v"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
    p = fa.params(w.B, w.Hq, w.Hkv, w.Sq, w.Skv, w.D, w.scale, True, None, code)
    nbytes = fa.fa_fwd_splitkv_workspace_bytes(p, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream
    hip = Hip()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr())

    def split():
        st = fa.fa_fwd_splitkv(*ptrs, p, 0, ws.data_ptr(), nbytes, sh)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_fwd_splitkv")

    def plain():
        st = fa.fa_fwd_ex(*ptrs, p, sh)
        if st != fa.FA_OK:
            raise fa.FAError(st, "fa_fwd_ex")

    ms, (split_ms, merge_ms) = _time_calls(split, steps, warmup, sh, hip, nev=3)
    plain_ms, _ = _time_calls(plain, steps, warmup, sh, hip)
    gbs = w.min_bytes() / (ms * 1e-3) / 1e9
    nsplit = nbytes // (w.B * w.Hq * w.Sq * (w.D + 1) * 4)
    del t, q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return {"workload": w.name, "ms": round(ms, 4), "split_kernel_ms": round(split_ms, 4),
            "merge_kernel_ms": round(merge_ms, 4), "num_splits": int(nsplit),
            "bytes": w.min_bytes(), "achieved": round(gbs, 1), "unit": "GB/s", "bound": "hbm",
            "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
            "plain_forward_ms": round(plain_ms, 4), "speedup_vs_plain_forward": round(plain_ms / ms, 2)}


def forward_sweep(steps, warmup, span_ms=200.0):
    """Forward alone at S = 4096, 8192, 16384 (B=1, Hq=32, Hkv=8, D=128, bf16, causal)."""
    import torch

    import causal_attention_fa_amd as fa
    out = []
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    sh = stream.cuda_stream
    hip = Hip()
    for S in (4096, 8192, 16384):
        B, Hq, Hkv, D = 1, 32, 8, 128
        g = torch.Generator(device=dev).manual_seed(S)
        q = (3 * torch.randn(B, Hq, S, D, device=dev, generator=g)).to(torch.bfloat16)
        k = torch.randn(B, Hkv, S, D, device=dev, generator=g).to(torch.bfloat16)
        v = torch.randn(B, Hkv, S, D, device=dev, generator=g).to(torch.bfloat16)
        o = torch.empty_like(q)
        lse = torch.empty(B, Hq, S, device=dev)

        def fwd():
            st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, S, D,
                           1 / math.sqrt(D), 1, fa.FA_BF16, sh)
            if st != fa.FA_OK:
                raise fa.FAError(st, "fa_fwd")

        # short kernels: warm up and time for a fixed span (span_ms / 2, span_ms),
        # so that the clock has settled and one launch's overhead does not count
        est, _ = _time_calls(fwd, 3, 1, sh, hip)
        ms, _ = _time_calls(fwd, max(steps, int(span_ms / est)), max(warmup, int(span_ms / 2 / est)), sh, hip)
        tf = 4.0 * D * B * Hq * S * (S + 1) / 2 / (ms * 1e-3) / 1e12
        out.append({"S": S, "ms": round(ms, 4), "tflops": round(tf, 1),
                    "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)})
        del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"config": "B=1 Hq=32 Hkv=8 D=128 bf16 causal, forward only", "points": out}


def peak_memory(w):
    """Peak device memory of fa fwd+bwd above the inputs, vs materialised [B,Hq,S,S] scores
    (allocator protocol: baseline after inputs, reset peak, run, read peak)."""
    import torch

    import causal_attention_fa_amd as fa

    dev = torch.device("cuda:0")
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
    elem = {"bf16": 2, "f16": 2, "f32": 4}[w.dtype]
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    q = torch.randn((w.B, w.Hq, w.S, w.D), device=dev, dtype=tdt, generator=g)
    k = torch.randn((w.B, w.Hkv, w.S, w.D), device=dev, dtype=tdt, generator=g)
    v = torch.randn((w.B, w.Hkv, w.S, w.D), device=dev, dtype=tdt, generator=g)
    do = torch.randn((w.B, w.Hq, w.S, w.D), device=dev, dtype=tdt, generator=g)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    o, lse = fa.forward(q, k, v, scale=w.scale, causal=w.causal)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev)
    live = sum(x.numel() * x.element_size() for x in (o, lse, dq, dk, dv))
    scores = w.B * w.Hq * w.S * w.S * elem
    out = {
        "workload": w.name,
        "baseline_MiB": round(base / 2**20, 2),
        "peak_MiB": round(peak / 2**20, 2),
        "above_baseline_MiB": round((peak - base) / 2**20, 2),
        "live_outputs_MiB": round(live / 2**20, 2),
        "bwd_workspace_MiB": round(fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.S, w.D) / 2**20, 2),
        "materialised_scores_one_matrix_MiB": round(scores / 2**20, 2),
        "materialised_fwd_bwd_MiB": round(4 * scores / 2**20, 2),
        "note": "materialised baseline = [B,Hq,S,S] in dtype per matrix; fwd keeps scores and probs, "
                "bwd adds dP and dS (4 matrices); fa keeps O(S*D) outputs plus an fp32 [B*Hq*S] workspace",
    }
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, min_seconds=12.0):
    """The fp64 oracle (dense form) timed on the host on whole KV groups of the
    workload, one after another until at least ``min_seconds`` have passed."""
    import numpy as np  # noqa: F401

    import oracle

    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"),
                      default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    inp = workload_inputs(w)
    G = w.group
    per_head = w.S * (w.S + 1) // 2 if w.causal else w.S * w.S
    done, dt = 0, 0.0
    for g in range(w.Hkv):
        sl = {"q": inp["q"][:1, g * G:(g + 1) * G], "k": inp["k"][:1, g:g + 1], "v": inp["v"][:1, g:g + 1],
              "do": inp["do"][:1, g * G:(g + 1) * G]}
        t0 = time.perf_counter()
        oracle.sdpa_backward(sl["q"], sl["k"], sl["v"], sl["do"], w.scale, w.causal)
        dt += time.perf_counter() - t0
        done += 1
        if dt >= min_seconds:
            break
    flops = 14.0 * w.D * per_head * G * done
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"dense fp64 oracle fwd+bwd of {done} whole KV group(s) (batch 0, KV heads 0..{done - 1}, "
                  f"{G} query heads each, all {w.S} rows) = {flops:.3e} causal flops in {dt:.1f} s; "
                  f"same flop count per pair as the GPU line",
        "seconds": round(dt, 2),
        "host_cpus": len(os.sched_getaffinity(0)),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=LONG_CONTEXT, choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-memory", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the split-KV decode measurement")
    ap.add_argument("--no-sweep", action="store_true", help="skip the forward sweep over S")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload table")
    ap.add_argument("--sweep-ms", type=float, default=200.0,
                    help="time span of each forward-sweep point (shorter for counter runs)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device-to-device copy of this many MiB (a reference "
                         "dispatch for scaling HBM byte counters); not part of the timed steps")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): this build has no "
              f"multi-GPU path; the attention shards by (batch, KV head) with no communication.",
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy_mib > 0:
        import torch
        n = args.calibrate_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
    w = WORKLOADS[args.workload]
    if not w.backward:
        raise SystemExit(f"{w.name} is a forward-only workload; bench times fwd+bwd")

    ms_step, per, clock = run_gpu(w, args.steps, args.warmup)
    kms = {n: sum(per[n]) / len(per[n]) for n in KERNELS}
    work = algorithmic_work(w)
    flops_step = w.fwd_flops() + w.bwd_flops()
    tflops = flops_step / (ms_step * 1e-3) / 1e12
    peak = PEAK_FP32_MATRIX_TFLOPS if w.dtype == "f32" else PEAK_BF16_TFLOPS

    kernels = {}
    for n in KERNELS:
        t_s = kms[n] * 1e-3
        if n == "rowdot":
            a = work[n] / t_s / 1e9
            kernels[n] = {"bound": "hbm", "achieved": round(a, 1), "unit": "GB/s", "frac": round(a / PEAK_HBM_GBS, 4)}
        else:
            a = work[n] / t_s / 1e12
            kernels[n] = {"bound": "mfma", "achieved": round(a, 1), "unit": "TFLOP/s", "frac": round(a / peak, 4)}
        kernels[n].update(ms=round(kms[n], 4), **{k: v for k, v in stats(per[n]).items() if k != "mean_ms"})
    dom = max(KERNELS, key=lambda n: kms[n])
    kd = kernels[dom]
    prof = committed_traffic(w)
    traffic = None
    if prof is not None:
        for n in KERNELS:
            t = prof["kernels"].get(n)
            if t is not None:
                kernels[n]["hbm_bytes"] = t["fetch_bytes"] + t["write_bytes"]
        if dom in prof["kernels"]:
            traffic = prof["kernels"][dom]["fetch_bytes"] + prof["kernels"][dom]["write_bytes"]
    ctr = committed_counters(w)
    if ctr is not None:
        for n in KERNELS:
            c = ctr["kernels"].get(n)
            if c is not None:
                kernels[n]["counters"] = c
    roofline = {"kernel": dom, "bound": kd["bound"], "achieved": kd["achieved"],
                "peak": PEAK_HBM_GBS if kd["bound"] == "hbm" else peak, "unit": kd["unit"], "frac": kd["frac"],
                "traffic": traffic,
                "traffic_note": ("HBM bytes per launch: rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by the "
                                 "ratio a plain copy of known size reads on the same counter; from "
                                 f"profiles/hbm_traffic_{w.name}.json, taken on these exact kernel sources")
                if traffic is not None else "no counter profile for the current kernel sources",
                "work_per_launch": work[dom],
                "work_note": "fwd 4*D, dkdv 8*D, dq 2*D flops per visited causal pair; rowdot bytes = read O, dO "
                             "+ write D; achieved = work / mean event-timed duration"}
    bwd_ms = kms["rowdot"] + kms["dkdv"] + kms["dq"]
    step_stats = stats(per["step"])
    out = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "S": w.S, "D": w.D,
                   "causal": w.causal, "scale": w.scale, "flops_per_step": flops_step},
        "pct_of_bf16_peak": round(100.0 * tflops / peak, 2),
        "step_kernels": dict(step_stats, tflops_at_median=round(flops_step / (step_stats["median_ms"] * 1e-3) / 1e12,
                                                                  2),
                             note="fwd start to dQ end per step, from the library's kernel events"),
        "forward": {"ms": round(kms["fwd"], 4), "median_ms": kernels["fwd"]["median_ms"],
                    "min_ms": kernels["fwd"]["min_ms"], "tflops": kernels["fwd"]["achieved"],
                    "pct_of_bf16_peak": round(100.0 * kernels["fwd"]["frac"], 2)},
        "backward": {"ms": round(bwd_ms, 4), "tflops": round(w.bwd_flops() / (bwd_ms * 1e-3) / 1e12, 1)},
        "kernels": kernels,
        "roofline": roofline,
        "gfx_clock": clock,
    }
    cf, cb = clock["forward"].get("median_mhz"), clock["fwd_bwd"].get("median_mhz")
    if cf and cb and w.dtype != "f32":
        def cpeak(mhz):
            return CUS * mhz * 1e6 * BF16_FLOP_PER_CLK_CU / 1e12
        out["pct_of_clock_peak"] = {
            "fwd_bwd": round(100 * tflops / cpeak(cb), 2), "fwd_bwd_clock_mhz": cb,
            "forward": round(100 * kernels["fwd"]["achieved"] / cpeak(cf), 2), "forward_clock_mhz": cf,
            "note": "256 CUs x the sampled graphics clock under that work x 4096 bf16 flop/clk/CU; the 2516.6 "
                    f"TFLOP/s peak assumes {clock['forward'].get('max_clk_mhz')} MHz"}
    if not args.no_configs:
        out["configs"] = config_table({w.name})
    if not args.no_sweep:
        out["forward_sweep"] = forward_sweep(10, 3, args.sweep_ms)
    if not args.no_decode:
        out["decode"] = decode_bench(20, 5)
    if not args.no_memory:
        out["memory"] = [peak_memory(w), peak_memory(WORKLOADS["causal_f16_b1_h8_s4096_d64"])]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
