#!/usr/bin/env python3
"""Benchmark of the exact attention forward on one MI355X.

A step is one attn_fwd call (the whole fused path: Q tile load, K/V tile
stream, score MFMA, mask, online softmax, PV MFMA, epilogue) over one batch of
seeded synthetic input of the headline workload, by default
B=2, H=16, S=4096, D=128, fp16, non-causal, Q,K ~ 2 N(0,1), V ~ N(0,1).

Defaults: 100 untimed warm-up launches, then 100 timed ones (about 25 ms
each for the headline workload): the clock settles only after a few dozen back-to-back launches
of a fresh process, and a shorter warm-up would average over that ramp.
Every forward warm-up (the headline's and each other workload's) also lasts
at least 30 ms of wall time, however short the launches; the JSON line
reports the warm-up launches actually run.

Prints ONE JSON line.  `value` is TFLOP/s with FLOPs = 4*B*H*S^2*D (halved when
causal) and the inputs already resident in HBM.  The timed region is the
launches back to back between two HIP events on the stream the kernel runs
on, so the roofline object's average launch duration is the region's time
per launch (gaps between launches included).  `launch_stats` gives the mean,
median, min and max of a second pass with HIP events around every launch
(events that add a few microseconds between launches, hence not in the
timed region).  `shader_clock` is the GFX clock sampled while the
headline kernel runs back to back right after the timed region, with the
socket power, the power cap and the share of that window the firmware
throttled the clock for package power; the reference GEMM carries the same
readings.

The CPU leg runs after all GPU timing: the fp64 oracle, as it stands, over
every row of every timed workload (`cpu_baseline` is its rate on the headline
workload, with the thread count), and every O and LSE element of each GPU run
compared against it (`parity`, and `parity` of each other workload).

The `backward` object times attn_bwd (dQ, dK, dV and D_i for a seeded dO)
on the same inputs, with the forward's O and LSE: TFLOP/s at the usual
10*B*H*S^2*D (five S x S x D GEMMs, halved when causal) and at the 14*B*H*S^2*D
the kernels execute (the dQ kernel recomputes S and dP), plus a parity spot
check of one head against the oracle.

The `unfused` object times the comparator attn_fwd_unfused (S = scale Q K^T
written to HBM in fp32, a row softmax writing P, then O = P V) on the same
inputs, with the HBM bytes it must move at least and its speed against the
fused kernel.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS + % of MI355X fp16/bf16 MFMA peak, hd128 causal/non-causal"
PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA
HEADLINE = "c4_b2h16s4096d128_fp16_peaky"
HEADLINE_SHAPE = (2, 16, 4096, 128, "fp16", False)  # the profiled HBM-traffic figure's workload
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_c4_hbm_traffic.txt")


def flops(B, H, S, D, causal):
    f = 4.0 * B * H * S * S * D
    return f / 2 if causal else f


def min_bytes(B, H, S, D):
    return 8 * B * H * S * D + 4 * B * H * S


# the sources that define the forward kernel and its launch configuration
FWD_SOURCES = ("attn_api.hip", "attn_fwd_kernel.hpp", "attn_grid.hpp")


def strip_comments(src):
    """C/C++ source without its comments and blank lines (string and
    character literals kept as they are), each line right-stripped."""
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
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def kernel_source_hash():
    """Hash of the forward kernel's sources, comments and blank lines left
    out: the committed HBM traffic figure is used only while it matches (the
    backward and the comparator live in other files and do not invalidate
    it, and neither does a comment)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "exact_attention_52_amd", "csrc")
    for name in FWD_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when missing or taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for ln in open(TRAFFIC_FILE):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_inputs(name, seed=0):
    import torch
    from exact_attention_52_amd import inputs
    B, H, S, D, dtype, causal, mult = inputs.WORKLOADS[name]
    q, k, v = inputs.gen_qkv(B, H, S, D, dtype, seed=seed, qk_mult=mult)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    dev = [torch.from_numpy(x.view(np.int16)).view(tdt).to("cuda:0") for x in (q, k, v)]
    return (B, H, S, D, dtype, causal), (q, k, v), dev


# The card's clock settles only after some tens of milliseconds of
# back-to-back work, whatever the number of launches that takes, so every
# forward warm-up runs at least `warmup` launches and at least this long.
MIN_WARM_MS = 30.0


def warm_up(launch, warmup, min_ms=MIN_WARM_MS):
    """Runs launch() at least `warmup` times and for at least min_ms of wall
    time (in batches of up to 10, synchronised); returns the launch count."""
    import torch
    done = 0
    t_start = time.perf_counter()
    while True:
        n = min(10, warmup - done) if done < warmup else 10
        for _ in range(n):
            launch()
        done += n
        torch.cuda.synchronize()
        if done >= warmup and (time.perf_counter() - t_start) * 1e3 >= min_ms:
            return done


def fwd_launcher(ea, q, k, v, scale, causal, o, lse, stream, variant=0):
    """One forward launch: attn_fwd, or attn_fwd_variant's copy schedule `variant`."""
    if variant:
        return lambda: ea.fwd_variant(q, k, v, variant, scale=scale, causal=causal, out=o, lse=lse, stream=stream)
    return lambda: ea.fwd(q, k, v, scale=scale, causal=causal, out=o, lse=lse, stream=stream)


def time_workload(ea, shape, dev, steps, warmup, variant=0):
    """Returns (ms_per_step over the timed region, per-launch ms list, o, lse,
    warm-up launches run).

    The timed region is `steps` launches back to back between two HIP events
    on the kernel's stream: its mean is the average launch duration, gaps
    between launches included.  The per-launch durations come from a second
    pass of as many launches right after it, each between two events of its
    own: those events put a few microseconds of gap between launches (for the
    headline workload the region with them took ~3 % longer per step), so they stay out of the
    timed region and serve only the per-call statistics."""
    import torch
    B, H, S, D, dtype, causal = shape
    scale = float(np.float32(1.0 / math.sqrt(D)))
    q, k, v = dev
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    launch = fwd_launcher(ea, q, k, v, scale, causal, o, lse, stream, variant)
    warmed = warm_up(launch, warmup)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        launch()
    t1.record(stream)
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        launch()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return total / steps, per, o, lse, warmed


PEAK_HBM_GBS = 8000.0  # MI355X HBM3E


def roofline(shape, ms_kernel):
    """The bound of the workload's kernel: MFMA when its FLOPs at the dense
    fp16/bf16 peak take longer than its algorithmic bytes at the HBM peak,
    else HBM; achieved = the algorithmic work per launch / the mean launch."""
    B, H, S, D, dtype, causal = shape
    f, nb = flops(B, H, S, D, causal), min_bytes(B, H, S, D)
    t = ms_kernel * 1e-3
    common = {"traffic": read_traffic() if shape == HEADLINE_SHAPE else None, "algorithmic_flop": f,
              "algorithmic_min_hbm_bytes": nb}
    if f / (PEAK_TFLOPS * 1e12) >= nb / (PEAK_HBM_GBS * 1e9):
        a = f / t / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / PEAK_TFLOPS, 4), **common}
    a = nb / t / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(a / PEAK_HBM_GBS, 4), **common}


def launch_stats(per_ms):
    """Per-launch durations (HIP events around each launch) in microseconds."""
    a = np.asarray(per_ms, dtype=np.float64) * 1e3
    return {"launches": int(a.size), "mean_us": round(float(a.mean()), 2),
            "median_us": round(float(np.median(a)), 2), "min_us": round(float(a.min()), 2),
            "max_us": round(float(a.max()), 2)}


class ClockSampler:
    """The shader (GFX) clock and socket power of cuda:0 read through amdsmi
    (the library behind amd-smi) from a sampling thread while kernels run back
    to back, with the card's power cap and the share of the window the
    firmware spent throttling the clock for package power (its PPT violation
    counter).  Reporting only: any failure leaves a reading None with the
    reason."""

    def __init__(self):
        self.handle, self.error, self.api = None, None, None
        try:
            import amdsmi
            import torch
            amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
            prop = torch.cuda.get_device_properties(0)
            want = (prop.pci_domain_id, prop.pci_bus_id, prop.pci_device_id)
            for h in amdsmi.amdsmi_get_processor_handles():
                dom, bus, rest = amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self.handle = h
            if self.handle is None:
                self.error = "no amdsmi device has cuda:0's PCI address"
            self.api = amdsmi
        except Exception as e:  # noqa: BLE001 -- reporting only
            self.error = f"amdsmi unavailable: {e}"

    def read(self):
        """(mean of the per-XCD current GFX clocks, or the GFX clock, in MHz;
        current socket power in W or None)."""
        m = self.api.amdsmi_get_gpu_metrics_info(self.handle)
        w = m.get("current_socket_power")
        w = float(w) if isinstance(w, (int, float)) and 0 < w < 100000 else None
        clks = m.get("current_gfxclks")
        if isinstance(clks, (list, tuple)):
            vals = [float(c) for c in clks if isinstance(c, (int, float)) and 0 < c < 10000]
            if vals:
                return sum(vals) / len(vals), w
        c = m.get("current_gfxclk")
        if isinstance(c, (int, float)) and 0 < c < 10000:
            return float(c), w
        return float(self.api.amdsmi_get_clock_info(self.handle, self.api.AmdSmiClkType.GFX)["clk"]), w

    def power_cap_w(self):
        try:
            cap = self.api.amdsmi_get_power_cap_info(self.handle).get("power_cap")
            return round(float(cap) / 1e6, 1) if isinstance(cap, (int, float)) and cap > 0 else None
        except Exception:  # noqa: BLE001 -- reporting only
            return None

    def ppt_counters(self):
        """(PPT power-throttle accumulator, sample accumulator) or None."""
        try:
            v = self.api.amdsmi_get_violation_status(self.handle)
            a, n = v.get("acc_ppt_pwr"), v.get("acc_counter")
            return (a, n) if isinstance(a, int) and isinstance(n, int) else None
        except Exception:  # noqa: BLE001 -- reporting only
            return None

    def during(self, launch, ms=1500.0, skip_ms=500.0, period_s=0.005):
        """Runs launch() back to back for about `ms` of wall time (synchronised
        every 20 launches) while a thread samples the clock; the samples of the
        first `skip_ms` are dropped (the metrics table amdsmi reads lags the
        clock by a few hundred milliseconds).  Returns a dict."""
        import threading

        import torch
        if self.handle is None:
            return {"mhz_median": None, "error": self.error}
        samples, watts, errs, stop = [], [], [], threading.Event()
        ppt = []

        def loop():
            while not stop.is_set():
                try:
                    mhz, w = self.read()
                    if (time.perf_counter() - t0) * 1e3 >= skip_ms:
                        if not ppt:
                            ppt.append(self.ppt_counters())
                        samples.append(mhz)
                        if w is not None:
                            watts.append(w)
                except Exception as e:  # noqa: BLE001
                    errs.append(str(e))
                    return
                time.sleep(period_s)

        th = threading.Thread(target=loop, daemon=True)
        n, t0 = 0, time.perf_counter()
        th.start()
        while (time.perf_counter() - t0) * 1e3 < ms:
            for _ in range(20):
                launch()
            n += 20
            torch.cuda.synchronize()
        ppt_end = self.ppt_counters()
        stop.set()
        th.join()
        if not samples:
            return {"mhz_median": None, "error": errs[0] if errs else "no samples"}
        a = np.asarray(samples)
        throttled = None
        if ppt and ppt[0] is not None and ppt_end is not None and ppt_end[1] > ppt[0][1]:
            throttled = round((ppt_end[0] - ppt[0][0]) / (ppt_end[1] - ppt[0][1]), 3)
        return {"mhz_median": round(float(np.median(a)), 1), "mhz_min": round(float(a.min()), 1),
                "mhz_max": round(float(a.max()), 1), "samples": int(a.size), "launches": n,
                "window_ms": round((time.perf_counter() - t0) * 1e3, 1),
                "socket_power_w_median": round(float(np.median(watts)), 1) if watts else None,
                "power_cap_w": self.power_cap_w(),
                "ppt_throttle_share": throttled,
                "source": f"amdsmi gpu_metrics current_gfxclks (mean over the XCDs) and current_socket_power, "
                          f"sampled every {period_s * 1e3:.0f} ms from {skip_ms:.0f} ms on while the kernel ran "
                          f"back to back after the timed region; power_cap_w from the power-cap info; "
                          f"ppt_throttle_share = growth of the PPT power-violation accumulator over the growth "
                          f"of its sample counter in the same window"}


def bwd_flops(B, H, S, D, causal, gemms=5):
    f = 2.0 * gemms * B * H * S * S * D
    return f / 2 if causal else f


def make_do(shape, seed=1):
    import torch
    from exact_attention_52_amd import inputs
    B, H, S, D, dtype, causal = shape
    do, _, _ = inputs.gen_qkv(B, H, S, D, dtype, seed=seed)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    return do, torch.from_numpy(do.view(np.int16)).view(tdt).to("cuda:0")


def time_backward(ea, shape, dev, ddo, steps, warmup):
    """Mean ms per attn_bwd call (HIP events on the launch stream) and the outputs."""
    import torch
    B, H, S, D, dtype, causal = shape
    scale = float(np.float32(1.0 / math.sqrt(D)))
    q, k, v = dev
    stream = torch.cuda.current_stream()
    o, lse = ea.fwd(q, k, v, scale=scale, causal=causal, stream=stream)
    outs = ea.bwd(q, k, v, o, lse, ddo, scale=scale, causal=causal, stream=stream)
    kw = dict(scale=scale, causal=causal, dq=outs[0], dk=outs[1], dv=outs[2], delta=outs[3], stream=stream)
    for _ in range(warmup):
        ea.bwd(q, k, v, o, lse, ddo, **kw)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        ea.bwd(q, k, v, o, lse, ddo, **kw)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps, outs


def bwd_spot_check(shape, words, do_words, outs, head=0):
    """dQ, dK, dV, D_i of one head against the oracle (relative to each tensor's max)."""
    import oracle
    B, H, S, D, dtype, causal = shape
    scale = float(np.float32(1.0 / math.sqrt(D)))
    b, h = divmod(head, H)
    sl = lambda a: np.ascontiguousarray(a[b:b + 1, h:h + 1])  # noqa: E731
    ref = oracle.attn_bwd(*(sl(x) for x in words), sl(do_words), dtype, scale, causal)
    got = [sl(t.float().cpu().numpy().astype(np.float64)) for t in outs]
    u = 2.0 ** -11 if dtype == "fp16" else 2.0 ** -8
    errs = {n: float(np.abs(g - r).max() / max(1.0, np.abs(r).max()))
            for n, g, r in zip(("dq", "dk", "dv", "delta"), got, ref)}
    return {"head": head, "rel_err": errs, "tol": 4 * u, "ok": all(e <= 4 * u for e in errs.values())}


def unfused_bytes(B, H, S, D):
    """HBM bytes the unfused path moves at least: Q, K, V read, S written and
    read (fp32), P written and read (16-bit), the fp32 O before normalisation
    and the per-row factors written and read, O and LSE written."""
    return min_bytes(B, H, S, D) + B * H * S * S * (4 + 4 + 2 + 2) + B * H * S * (D + 1) * 4 * 2


def time_unfused(ea, shape, dev, steps, warmup):
    import torch
    B, H, S, D, dtype, causal = shape
    scale = float(np.float32(1.0 / math.sqrt(D)))
    q, k, v = dev
    stream = torch.cuda.current_stream()
    ws = torch.empty(ea.attn_fwd_unfused_workspace_bytes(B, H, S, D), dtype=torch.uint8, device=q.device)
    o, lse = ea.fwd_unfused(q, k, v, scale=scale, causal=causal, workspace=ws, stream=stream)
    for _ in range(warmup):
        ea.fwd_unfused(q, k, v, scale=scale, causal=causal, out=o, lse=lse, workspace=ws, stream=stream)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        ea.fwd_unfused(q, k, v, scale=scale, causal=causal, out=o, lse=lse, workspace=ws, stream=stream)
    t1.record(stream)
    torch.cuda.synchronize()
    del ws
    torch.cuda.empty_cache()
    return t0.elapsed_time(t1) / steps, o, lse


def reference_gemm(n, steps=50, clock_ms=0.0):
    """Context for the MFMA roofline: a plain fp16 n x n x n torch.matmul (the vendor
    GEMM library) on random N(0,1) data, timed back to back like the attention launches.
    Random-data MFMA work runs the card at its power limit, so this is the dense-MFMA
    rate the box actually sustains; it is not used for any figure of merit.  With
    clock_ms > 0 the GEMM then runs back to back that long under the clock and power
    sampler."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(0)
    a = torch.randn(n, n, device="cuda:0", dtype=torch.float16, generator=g)
    b = torch.randn(n, n, device="cuda:0", dtype=torch.float16, generator=g)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        c = a @ b
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    out = {"what": f"torch.matmul fp16 {n}x{n}x{n}, random N(0,1), {steps} back to back",
           "us_per_call": round(ms * 1e3, 1), "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)}
    if clock_ms > 0:
        out["shader_clock"] = ClockSampler().during(lambda: torch.matmul(a, b, out=c), ms=clock_ms)
    del a, b, c
    torch.cuda.empty_cache()
    return out


def full_oracle(shape, words):
    """The fp64 oracle, as it stands, over every row of the workload; returns
    (O, LSE, wall seconds)."""
    import oracle
    B, H, S, D, dtype, causal = shape
    scale = float(np.float32(1.0 / math.sqrt(D)))
    t = time.perf_counter()
    o_ref, l_ref = oracle.attn_fwd(*words, dtype, scale, causal)
    return o_ref, l_ref, time.perf_counter() - t


def parity_all(shape, o_host, lse_host, o_ref, l_ref):
    """Every O and LSE element of the GPU output against the oracle's."""
    B, H, S, D, dtype, causal = shape
    eo = float(np.abs(o_host.astype(np.float64) - o_ref).max())
    el = float((np.abs(lse_host.astype(np.float64) - l_ref) / np.maximum(1.0, np.abs(l_ref))).max())
    tol = 2e-3 if dtype == "fp16" else 1.6e-2
    return {"rows": int(B * H * S), "elements_o": int(o_ref.size), "max_abs_err_o": eo, "max_err_lse": el,
            "tol_o": tol, "tol_lse": 1e-4, "ok": bool(eo <= tol and el <= 1e-4)}


def oracle_rate(shape, seconds):
    """The oracle's rate in the GPU figure's FLOP convention (4*D per query-key
    pair, exactly halved for causal)."""
    import oracle
    B, H, S, D, dtype, causal = shape
    fl = flops(B, H, S, D, causal)
    return {"value": fl / seconds / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(seconds, 2),
            "sample": f"all {B * H * S} query rows of the workload (100%), fp64 two-pass oracle, "
                      f"{seconds:.1f} s wall on {oracle.num_threads()} threads"}


def host(o, lse):
    return o.float().cpu().numpy(), lse.cpu().numpy()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the card's clock ramps over a process's first few dozen launches
    # (headline workload: ~340 us per launch for the first 20, ~265 for the next 20, a
    # steady ~241 from about the 60th on), so the default warm-up covers it
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--variant", type=int, default=0,
                    help="time attn_fwd_variant's copy schedule VARIANT instead of attn_fwd (A/B runs; "
                         "0 is attn_fwd itself)")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg: the timed fp64 oracle over every workload and the "
                         "comparison of every output element against it")
    ap.add_argument("--clock-ms", type=float, default=1500.0,
                    help="after the timed region, run the headline kernel back to back this long "
                         "while sampling the shader clock (0: skip)")
    ap.add_argument("--no-others", action="store_true", help="skip timing the other workloads")
    ap.add_argument("--ref-gemm", type=int, default=8192,
                    help="also time an fp16 N^3 torch.matmul as context for the MFMA roofline (0: skip)")
    ap.add_argument("--no-backward", action="store_true", help="skip timing attn_bwd")
    ap.add_argument("--no-unfused", action="store_true", help="skip timing the unfused comparator")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one element-wise add reading and writing this many MiB "
                         "(calibrates the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the attention forward "
              "shards by batch*head with no communication, so N GPUs run N independent copies.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_52_amd as ea
    from exact_attention_52_amd import inputs
    ea._lib.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    shape, words, dev = make_inputs(args.workload)
    B, H, S, D, dtype, causal = shape
    ms_step, per, o, lse, warmed = time_workload(ea, shape, dev, args.steps, args.warmup, args.variant)
    stats = launch_stats(per)
    # one launch per step: the timed region's mean launch duration
    ms_kernel = ms_step
    f = flops(B, H, S, D, causal)
    value = f / (ms_step * 1e-3) / 1e12
    achieved = f / (ms_kernel * 1e-3) / 1e12
    print(f"# {args.workload}: {ms_step * 1e3:.1f} us/step, kernel {stats}, "
          f"{achieved:.1f} TFLOP/s ({achieved / PEAK_TFLOPS:.1%} of peak)", file=sys.stderr, flush=True)
    outputs = {args.workload: (shape, words, *host(o, lse))}

    clock = None
    if args.clock_ms > 0:
        scale = float(np.float32(1.0 / math.sqrt(D)))
        stream = torch.cuda.current_stream()
        clock = ClockSampler().during(fwd_launcher(ea, *dev, scale, causal, o, lse, stream, args.variant),
                                      ms=args.clock_ms)
        print(f"# shader clock: {clock}", file=sys.stderr, flush=True)
    del o, lse

    if args.calib_copy_mib:
        # a plain streaming kernel of known traffic for HBM-counter calibration:
        # reads and writes exactly calib_copy_mib MiB
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    backward = None
    if not args.no_backward:
        do_words, ddo = make_do(shape)
        ms_b, outs = time_backward(ea, shape, dev, ddo, max(5, args.steps // 2), max(2, args.warmup // 2))
        conv = bwd_flops(B, H, S, D, causal) / (ms_b * 1e-3) / 1e12
        executed = bwd_flops(B, H, S, D, causal, gemms=7) / (ms_b * 1e-3) / 1e12
        backward = {"workload": args.workload, "us_per_call": round(ms_b * 1e3, 2),
                    "tflops": round(conv, 1), "frac_of_peak": round(conv / PEAK_TFLOPS, 4),
                    "executed_tflops": round(executed, 1),
                    "parity_spot_check": bwd_spot_check(shape, words, do_words, outs)}
        print(f"# backward: {backward}", file=sys.stderr, flush=True)
        del outs, ddo

    unfused, unfused_out = None, None
    if not args.no_unfused:
        ms_u, o_u, lse_u = time_unfused(ea, shape, dev, max(5, args.steps // 5), 2)
        nb = unfused_bytes(B, H, S, D)
        unfused = {"workload": args.workload, "us_per_call": round(ms_u * 1e3, 2),
                   "tflops": round(f / (ms_u * 1e-3) / 1e12, 1),
                   "hbm_bytes_min": nb, "hbm_bound_us": round(nb / 8e12 * 1e6, 1),
                   "achieved_gbps_of_min": round(nb / (ms_u * 1e-3) / 1e9, 1),
                   "fused_speedup": round(ms_u / ms_kernel, 2)}
        unfused_out = host(o_u, lse_u)
        print(f"# unfused comparator: {unfused}", file=sys.stderr, flush=True)
        del o_u, lse_u
    del dev
    torch.cuda.empty_cache()

    others = {}
    if not args.no_others:
        for name in inputs.WORKLOADS:
            if name == args.workload:
                continue
            shp, wds, dv = make_inputs(name)
            ms_o, per_o, o_o, l_o, _ = time_workload(ea, shp, dv, max(5, args.steps // 2), max(2, args.warmup // 2))
            st = launch_stats(per_o)
            fl = flops(shp[0], shp[1], shp[2], shp[3], shp[5])
            t_us = round(ms_o * 1e3, 2)
            others[name] = {"us_per_call": t_us, "launch_stats": st,
                            "tflops": round(fl / (t_us * 1e-6) / 1e12, 1),
                            "frac_of_peak": round(fl / (t_us * 1e-6) / 1e12 / PEAK_TFLOPS, 4)}
            outputs[name] = (shp, wds, *host(o_o, l_o))
            if args.clock_ms > 0 and t_us >= 50.0:
                # the steady clock of this workload's kernel, back to back
                sc = float(np.float32(1.0 / math.sqrt(shp[3])))
                others[name]["shader_clock"] = ClockSampler().during(
                    fwd_launcher(ea, *dv, sc, shp[5], o_o, l_o, torch.cuda.current_stream(), 0), ms=args.clock_ms)
            del o_o, l_o
            if not args.no_backward:
                _, ddo = make_do(shp)
                ms_b, _ = time_backward(ea, shp, dv, ddo, max(5, args.steps // 5), 2)
                flb = bwd_flops(shp[0], shp[1], shp[2], shp[3], shp[5])
                others[name]["bwd_us_per_call"] = round(ms_b * 1e3, 2)
                others[name]["bwd_tflops"] = round(flb / (ms_b * 1e-3) / 1e12, 1)
                del ddo
            print(f"# {name}: {others[name]}", file=sys.stderr, flush=True)
            del dv
            torch.cuda.empty_cache()

    gemm = reference_gemm(args.ref_gemm, clock_ms=args.clock_ms) if args.ref_gemm > 0 and not args.no_others else None
    if gemm:
        print(f"# reference gemm: {gemm}", file=sys.stderr, flush=True)

    # The CPU leg, after all GPU timing: the fp64 oracle over every row of
    # each timed workload, timed, and every output element of the GPU run
    # compared against it.
    cpu, parity = None, None
    if not args.no_cpu_baseline:
        for name, (shp, wds, o_h, l_h) in outputs.items():
            o_ref, l_ref, secs = full_oracle(shp, wds)
            par = parity_all(shp, o_h, l_h, o_ref, l_ref)
            rate = oracle_rate(shp, secs)
            print(f"# {name}: oracle {secs:.2f} s on {rate['cores']} threads; parity {par}",
                  file=sys.stderr, flush=True)
            if name == args.workload:
                cpu, parity = rate, par
                if unfused_out is not None:
                    unfused["parity"] = parity_all(shp, *unfused_out, o_ref, l_ref)
            else:
                others[name]["parity"] = par
                others[name]["cpu_oracle"] = {k: rate[k] for k in ("value", "unit", "cores", "seconds")}
            del o_ref, l_ref
    del outputs

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_launches_run": warmed,
        "warmup_min_ms": MIN_WARM_MS,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded Philox4x32-10 + Box-Muller)",
        "config": {"workload": args.workload, "variant": args.variant, "B": B, "H": H, "S": S, "D": D, "dtype": dtype,
                   "causal": causal, "scale": "1/sqrt(D)", "global_batch": B, "seq_len": S,
                   "parallelism": "single GPU"},
        "roofline": roofline(shape, ms_kernel),
        "launch_stats": stats,
        "shader_clock": clock,
        "cpu_baseline": cpu,
        "parity": parity,
        "backward": backward,
        "unfused": unfused,
        "other_workloads": others,
        "reference_gemm": gemm,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
