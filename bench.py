"""Benchmark of the online-softmax hot path on one MI355X.

One step is one pass of the whole path over resident synthetic inputs:
  1. row softmax, float32, 32768 x 8192      (HBM-bound, 1 read + 1 write)
  2. row softmax, bfloat16, 32768 x 8192     (same, half the bytes)
  3. fused causal attention forward, bfloat16, B=8 H=40 N=2048 D=128
     (LLaMA-2-13B-shaped layer; bound by the bf16 matrix cores)

Also timed, outside the step (its own loop over the same number of launches):
  4. attention backward (dQ, dK, dV from the forward's O and LSE) on the same
     layer, reported under ``attention_backward`` and in ``rooflines`` with
     ``"in_step": false``.

Printed: one JSON line.  ``value`` is the softmax throughput of the
bandwidth-scale workload (algorithmic bytes of both softmax runs / their
kernel time); the attention throughput is in ``attention``.  ``rooflines``
holds each kernel against its roofline; ``roofline`` repeats the kernel that
takes the largest share of a step.  Kernel times come from HIP events recorded
on the launch stream around every launch of the timed steps.

Context fields: ``copy_ceiling`` is the fastest of 20 device-to-device
``hipMemcpyAsync`` calls on the float32 softmax bytes, with their median (the
practical streaming ceiling the softmax runs are compared with) and ``sclk_mhz`` the engine clock read from the driver's
``pp_dpm_sclk`` while the timed steps run (null where the file is absent).

``--only`` runs a single unit (for profiler runs; ``attn_long``, the B1 H32
N16384 D128 causal workload, runs only this way); ``--copy`` times a plain
device copy of the float32 softmax bytes (the counter calibration kernel).
"""

import argparse
import hashlib
import json
import math
import os
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16: 256 CU x 4096 FLOP/clk x 2.4 GHz

METRIC = "softmax GB/s (% HBM peak); attention fwd TFLOPS (% bf16 MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
SRC_DIR = os.path.join(ROOT, "online_softmax_06_amd", "csrc")


def kernel_source_hash(fname):
    h = hashlib.sha256()
    for f in (fname, "osm_device.h"):
        with open(os.path.join(SRC_DIR, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic():
    """Per-kernel HBM bytes per launch from the committed counter summary.

    Lines look like ``unit=<name> src=<hash> fetch_bytes=<n> write_bytes=<n>``.
    A unit whose kernel source hash no longer matches gets no figure.
    """
    out = {}
    if not os.path.exists(TRAFFIC_FILE):
        return out
    with open(TRAFFIC_FILE) as f:
        for line in f:
            kv = dict(re.findall(r"(\w+)=(\S+)", line))
            if "unit" in kv and "src" in kv:
                out[kv["unit"]] = kv
    return out


class Unit:
    def __init__(self, name, kernel, src, launch, work, bound, peak, unit, workload, in_step=True):
        self.name, self.kernel, self.src = name, kernel, src
        self.launch, self.work, self.bound, self.peak = launch, work, bound, peak
        self.unit, self.workload, self.in_step = unit, workload, in_step
        self.times_ms = []


def make_units(torch, osm, osm_inputs, only):
    units = []
    c = osm_inputs.SOFTMAX_LARGE
    for dt, tag in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        name = f"softmax_{tag}"
        if only not in (None, name):
            continue
        x = osm_inputs.softmax_large(dtype=dt, device="cuda")
        y = torch.empty_like(x)
        nbytes = 2 * x.numel() * x.element_size()  # one read + one write per element
        units.append(Unit(
            name, f"softmax_resident_kernel ({tag})", "softmax_rows.hip",
            (lambda x=x, y=y: osm.softmax_rows(x, out=y)), nbytes, "hbm", HBM_PEAK_GBS, "GB/s",
            f"softmax_large {c['rows']}x{c['cols']} {tag}"))
    if only in (None, "attn"):
        cfg = osm_inputs.attention_config("attn_llama13b", device="cuda")
        a = cfg["cfg"]
        o = torch.empty_like(cfg["q"])
        lse = torch.empty((a["B"], a["H"], a["N"]), dtype=torch.float32, device="cuda")
        # Algorithmic FLOPs: QK^T and PV over the unmasked (query, key) pairs,
        # 2 * 2 * D per pair; causal pairs = N (N + 1) / 2 per head.
        pairs = a["N"] * (a["N"] + 1) // 2 if a["causal"] else a["N"] * a["N"]
        flops = 4 * a["D"] * pairs * a["B"] * a["H"]
        units.append(Unit(
            "attn", "attn_fwd_kernel<128, causal>", "attn_fwd.hip",
            (lambda cfg=cfg, o=o, lse=lse: osm.attn_fwd(cfg["q"], cfg["k"], cfg["v"], cfg["scale"],
                                                        cfg["causal"], out=o, lse=lse)),
            flops, "mfma", BF16_MFMA_PEAK_TFLOPS, "TFLOP/s",
            f"attn_llama13b B{a['B']} H{a['H']} N{a['N']} D{a['D']} causal"))
    if only == "attn_long":
        # Profiling only (never part of the default step): the long-context
        # causal workload, B1 H32 N16384 D128, for its counters.
        cfg = osm_inputs.attention_config("attn_long", device="cuda")
        a = cfg["cfg"]
        o = torch.empty_like(cfg["q"])
        lse = torch.empty((a["B"], a["H"], a["N"]), dtype=torch.float32, device="cuda")
        pairs = a["N"] * (a["N"] + 1) // 2 if a["causal"] else a["N"] * a["N"]
        flops = 4 * a["D"] * pairs * a["B"] * a["H"]
        units.append(Unit(
            "attn_long", "attn_fwd_kernel<128, causal> (8 wavefronts)", "attn_fwd.hip",
            (lambda cfg=cfg, o=o, lse=lse: osm.attn_fwd(cfg["q"], cfg["k"], cfg["v"], cfg["scale"],
                                                        cfg["causal"], out=o, lse=lse)),
            flops, "mfma", BF16_MFMA_PEAK_TFLOPS, "TFLOP/s",
            f"attn_long B{a['B']} H{a['H']} N{a['N']} D{a['D']} causal", in_step=False))
    if only in (None, "attn_bwd"):
        cfg = osm_inputs.attention_config("attn_llama13b", device="cuda")
        a = cfg["cfg"]
        do = osm_inputs.attention_grad_output(a["B"], a["H"], a["N"], a["D"], seed=a["seed"],
                                              device="cuda")
        o, lse = osm.attn_fwd(cfg["q"], cfg["k"], cfg["v"], cfg["scale"], cfg["causal"])
        grads = [torch.empty_like(cfg["q"]) for _ in range(3)]
        # Algorithmic FLOPs: the five products of the backward (S recomputed,
        # dP, dV, dK, dQ), 2 * D each per unmasked (query, key) pair.
        pairs = a["N"] * (a["N"] + 1) // 2 if a["causal"] else a["N"] * a["N"]
        flops = 10 * a["D"] * pairs * a["B"] * a["H"]
        units.append(Unit(
            "attn_bwd", "attn_bwd dq + dkdv kernels <128, causal>", "attn_bwd.hip",
            (lambda cfg=cfg, o=o, lse=lse, do=do, g=grads: osm.attn_bwd(
                cfg["q"], cfg["k"], cfg["v"], o, lse, do, scale=cfg["scale"],
                causal=cfg["causal"], dq=g[0], dk=g[1], dv=g[2])),
            flops, "mfma", BF16_MFMA_PEAK_TFLOPS, "TFLOP/s",
            f"attn_llama13b B{a['B']} H{a['H']} N{a['N']} D{a['D']} causal, backward",
            in_step=False))
    return units


def cpu_baseline(torch, osm_inputs, budget_s):
    """Time the float64 oracle on bounded samples of the same workloads."""
    import numpy as np
    from oracle import attention_ref, softmax_rows_ref
    try:
        import threadpoolctl
        blas_threads = max(i["num_threads"] for i in threadpoolctl.threadpool_info())
    except Exception:
        blas_threads = None
    c = osm_inputs.SOFTMAX_LARGE
    x = osm_inputs.softmax_large(device="cuda")
    rows_done, t_sm = 0, 0.0
    chunk = 1024
    while rows_done < c["rows"] and t_sm < budget_s * 0.5:
        xs = x[rows_done:rows_done + chunk].double().cpu().numpy()
        t0 = time.perf_counter()
        softmax_rows_ref(xs)
        t_sm += time.perf_counter() - t0
        rows_done += xs.shape[0]
    del x
    sm_bytes = 2 * rows_done * c["cols"] * 4
    cfg = osm_inputs.attention_config("attn_llama13b", device="cuda")
    a = cfg["cfg"]
    heads = osm_inputs.sample_heads(a["B"], a["H"], a["B"] * a["H"], a["seed"], [(0, 0)])
    done, t_at = [], 0.0
    for (b, h) in heads:
        if t_at >= budget_s * 0.25:
            break
        q, k, v = (cfg[n][b, h][None, None].double().cpu().numpy() for n in ("q", "k", "v"))
        t0 = time.perf_counter()
        attention_ref(q, k, v, cfg["scale"], True)
        t_at += time.perf_counter() - t0
        done.append((b, h))
    at_flops = 4 * a["D"] * (a["N"] * (a["N"] + 1) // 2) * len(done)
    from oracle import attention_bwd_head_ref
    do = osm_inputs.attention_grad_output(a["B"], a["H"], a["N"], a["D"], seed=a["seed"],
                                          device="cuda")
    done_b, t_bw = [], 0.0
    for (b, h) in heads:
        if t_bw >= budget_s * 0.25:
            break
        q, k, v, g = (t[b, h].double().cpu().numpy() for t in (cfg["q"], cfg["k"], cfg["v"], do))
        t0 = time.perf_counter()
        attention_bwd_head_ref(q, k, v, g, cfg["scale"], True)
        t_bw += time.perf_counter() - t0
        done_b.append((b, h))
    bw_flops = 10 * a["D"] * (a["N"] * (a["N"] + 1) // 2) * len(done_b)
    return {
        "value": round(sm_bytes / t_sm / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"float64 three-pass softmax oracle (numpy, single-threaded) on the first "
                   f"{rows_done} of {c['rows']} rows of softmax_large fp32 ({t_sm:.1f} s)"),
        "attention": {
            "value": round(at_flops / t_at / 1e12, 6), "unit": "TFLOP/s",
            "cores": blas_threads, "kind": "oracle",
            "sample": (f"float64 materialised-score oracle (numpy + BLAS) on {len(done)} of "
                       f"{a['B'] * a['H']} (b, h) slices of attn_llama13b ({t_at:.1f} s)")},
        "attention_backward": {
            "value": round(bw_flops / t_bw / 1e12, 6), "unit": "TFLOP/s",
            "cores": blas_threads, "kind": "oracle",
            "sample": (f"float64 softmax-Jacobian gradient oracle (numpy + BLAS) on "
                       f"{len(done_b)} of {a['B'] * a['H']} (b, h) slices of attn_llama13b "
                       f"({t_bw:.1f} s); FLOPs counted as the library's five products")},
    }


class SclkSampler:
    """Reads the current engine clock (the level marked '*' in the driver's
    pp_dpm_sclk) every few milliseconds on a side thread."""

    def __init__(self):
        import glob
        self.paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    def _read(self):
        for p in self.paths:
            try:
                for line in open(p):
                    if line.rstrip().endswith("*"):
                        m = re.search(r"(\d+)\s*Mhz", line, re.IGNORECASE)
                        if m:
                            return int(m.group(1))
            except OSError:
                pass
        return None

    def _run(self):
        while not self._stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(0.005)

    def start(self):
        if self.paths:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self):
        # Samples taken while the GPU was busy (the idle level is far below).
        busy = [v for v in self.samples if v >= 1000]
        if not busy:
            return None
        busy.sort()
        return {"median": busy[len(busy) // 2], "min": busy[0], "max": busy[-1],
                "samples": len(busy), "source": "pp_dpm_sclk during the timed steps"}


def copy_ceiling(torch, osm_inputs, steps=20):
    """Device-to-device hipMemcpyAsync of the float32 softmax bytes."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int, ctypes.c_void_p]
    x = osm_inputs.softmax_large(device="cuda")
    y = torch.empty_like(x)
    nbytes = x.numel() * 4
    st = torch.cuda.current_stream()
    def one():
        # 3 = hipMemcpyDeviceToDevice
        if hip.hipMemcpyAsync(y.data_ptr(), x.data_ptr(), nbytes, 3, st.cuda_stream) != 0:
            raise RuntimeError("hipMemcpyAsync failed")
    for _ in range(3):
        one()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(st)
    for i in range(steps):
        one()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    del x, y
    # A ceiling: the fastest copy, with the median beside it.
    ms, med = per[0], per[len(per) // 2]
    return {"GB/s": round(2 * nbytes / ms / 1e6, 1), "ms": round(ms, 5),
            "median_GB/s": round(2 * nbytes / med / 1e6, 1),
            "frac_of_hbm_peak": round(2 * nbytes / ms / 1e6 / HBM_PEAK_GBS, 4),
            "method": "hipMemcpyAsync device-to-device, 1 GiB read + 1 GiB written; "
                      "fastest of the timed copies"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["softmax_f32", "softmax_bf16", "attn", "attn_bwd",
                                       "attn_long"], default=None,
                    help="time one unit (for profiler runs); attn_long runs only here")
    ap.add_argument("--copy", action="store_true", help="time a plain device copy instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              "supported: the kernels shard by (batch, head) or by row with no exchange, and "
              "this benchmark measures one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch
    import online_softmax_06_amd as osm
    import osm_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    osm.load_library()

    if args.copy:
        x = osm_inputs.softmax_large(device="cuda")
        y = torch.empty_like(x)
        for _ in range(args.warmup):
            y.copy_(x)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        for _ in range(args.steps):
            y.copy_(x)
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        print(json.dumps({"copy_bytes": 2 * x.numel() * 4, "ms": ms,
                          "GB/s": 2 * x.numel() * 4 / ms / 1e6}))
        return

    all_units = make_units(torch, osm, osm_inputs, args.only)
    units = [u for u in all_units if u.in_step]
    extra = [u for u in all_units if not u.in_step]
    for _ in range(args.warmup):
        for u in all_units:
            u.launch()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    marks = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in units] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    sclk = SclkSampler()
    t_start.record(stream)
    for s in range(args.steps):
        for i, u in enumerate(units):
            marks[s][i][0].record(stream)
            u.launch()
            marks[s][i][1].record(stream)
    t_end.record(stream)
    sclk.start()  # samples while the queued steps run
    torch.cuda.synchronize()
    sclk.stop()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps if units else 0.0
    for s in range(args.steps):
        for i, u in enumerate(units):
            u.times_ms.append(marks[s][i][0].elapsed_time(marks[s][i][1]))
    # Units outside the step: their own loop, the same number of launches.
    for u in extra:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            u.launch()
            e1.record(stream)
        torch.cuda.synchronize()
        u.times_ms = [e0.elapsed_time(e1) for e0, e1 in ev]

    traffic = read_traffic()
    rooflines = []
    for u in all_units:
        avg_ms = sum(u.times_ms) / len(u.times_ms)
        med_ms = sorted(u.times_ms)[len(u.times_ms) // 2]
        achieved = u.work / (avg_ms * 1e-3) / (1e9 if u.unit == "GB/s" else 1e12)
        tr = traffic.get(u.name)
        tr_bytes = None
        if tr and tr.get("src") == kernel_source_hash(u.src):
            tr_bytes = int(float(tr["fetch_bytes"])) + int(float(tr["write_bytes"]))
        rooflines.append({
            "unit_name": u.name, "kernel": u.kernel, "workload": u.workload,
            "bound": u.bound, "achieved": round(achieved, 2), "peak": u.peak, "unit": u.unit,
            "frac": round(achieved / u.peak, 4), "traffic": tr_bytes,
            "algorithmic": u.work, "avg_ms": round(avg_ms, 5), "median_ms": round(med_ms, 5),
            "min_ms": round(min(u.times_ms), 5), "max_ms": round(max(u.times_ms), 5),
            "in_step": u.in_step})
    in_step = [r for r in rooflines if r["in_step"]] or rooflines
    dominant = max(in_step, key=lambda r: r["avg_ms"])

    sm = [r for r in rooflines if r["unit_name"].startswith("softmax")]
    at = [r for r in rooflines if r["unit_name"] == "attn"]
    bw = [r for r in rooflines if r["unit_name"] == "attn_bwd"]
    if sm:
        sm_bytes = sum(r["algorithmic"] for r in sm)
        sm_ms = sum(r["avg_ms"] for r in sm)
        value, unit = sm_bytes / (sm_ms * 1e-3) / 1e9, "GB/s"
    else:
        first = (at or bw or rooflines)[0]
        value, unit = first["achieved"], first["unit"]

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 softmax math; bf16 MFMA with f32 accumulation (attention)",
        "data": "synthetic (seeded), resident in HBM",
        "config": {
            "workload": ("softmax_large 32768x8192 (fp32 run + bf16 run) + attn_llama13b "
                         "B8 H40 N2048 D128 causal bf16"),
            "softmax_rows": 32768, "softmax_cols": 8192,
            "attn": {"B": 8, "H": 40, "N": 2048, "D": 128, "causal": True},
            "parallelism": "single GPU",
        },
        "value_frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4) if unit == "GB/s" else None,
        "roofline": {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac",
                                              "traffic")} | {"kernel": dominant["kernel"]},
        "rooflines": rooflines,
    }
    if at:
        result["attention"] = {"value": at[0]["achieved"], "unit": "TFLOP/s",
                               "frac_of_bf16_peak": at[0]["frac"],
                               "flop_convention": "4*D per unmasked (query, key) pair"}
    if bw:
        result["attention_backward"] = {
            "value": bw[0]["achieved"], "unit": "TFLOP/s", "frac_of_bf16_peak": bw[0]["frac"],
            "avg_ms": bw[0]["avg_ms"], "in_step": False,
            "flop_convention": "10*D per unmasked (query, key) pair (five products)"}
    result["sclk_mhz"] = sclk.summary()
    if args.only is None:
        cc = copy_ceiling(torch, osm_inputs)
        if sm:
            cc["softmax_frac_of_copy"] = round(value / cc["GB/s"], 4)
        result["copy_ceiling"] = cc
    if not args.no_cpu_baseline and args.only is None:
        result["cpu_baseline"] = cpu_baseline(torch, osm_inputs, args.cpu_budget)
        result["cpu_baseline"]["host_cpus"] = len(os.sched_getaffinity(0))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
